"""Short text summaries of rocprofv3 output for the files kept under profiles/.

    python -m weight_sequence_layers_amd.profiling stats  OUT.md  TRACE_DIR   "<command>"
    python -m weight_sequence_layers_amd.profiling traffic OUT.md FETCH_DIR WRITE_DIR \
        WORKLOAD "<fetch command>" "<write command>"
    python -m weight_sequence_layers_amd.profiling mfma   OUT.md  PMC_DIR     "<command>"

`stats` turns a `rocprofv3 --kernel-trace --stats` directory into a table of kernel
durations. `traffic` turns one `--pmc FETCH_SIZE` and one `--pmc WRITE_SIZE` run of
`bench.py --calib-copy-mib 1024` into HBM bytes per launch of each stage kernel: each
counter is summed over its instances per dispatch, averaged over the dispatches of a
kernel, and scaled by what the same counter reads for the reference copy kernel (which
reads and writes exactly --calib-copy-mib MiB). The traffic table records the digest of
the kernel sources it was taken at; bench.py reports traffic only while it matches.
"""
from __future__ import annotations

import csv
import glob
import hashlib
import os
import re
import sys
from collections import defaultdict

PKG = os.path.dirname(os.path.abspath(__file__))

# stage name -> pattern of the kernels that implement it
STAGE_KERNELS = [
    # k_front<BM, BN, WGM, WGN, FW, MODE, BK>: MODE 0 applies, 1 and 2 take gradients
    ("front_q", r"k_front<(\d+, ){5}0, \d+>$"),
    ("front_k", r"k_front<(\d+, ){5}[12], \d+>$"),
    ("out", r"k_out<.*, 0>$"),
    ("mse", r"k_out<.*, [12]>$"),
    ("contract", r"k_contract(_sum)?<"),
    ("ns_gram", r"k_ns_gram<"),
    ("ns_poly", r"k_ns_poly<"),
    ("ns_update", r"k_ns_update<"),
    ("renorm", r"k_renorm"),
    ("split", r"k_split"),
    ("resident", r"k_small_gelu<"),
]


def source_digest() -> str:
    """Hash of the kernel sources (every file under csrc/)."""
    h = hashlib.sha256()
    csrc = os.path.join(PKG, "csrc")
    for f in sorted(os.listdir(csrc)):
        with open(os.path.join(csrc, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def _short(name: str) -> str:
    return re.sub(r"\(.*", "", name).strip()


def _one(pattern: str, d: str) -> str:
    found = glob.glob(os.path.join(d, "**", pattern), recursive=True)
    if not found:
        raise FileNotFoundError(f"no {pattern} under {d}")
    return found[0]


def stats_md(trace_dir: str, command: str) -> str:
    rows = list(csv.DictReader(open(_one("*kernel_stats.csv", trace_dir))))
    out = ["# Kernel durations", "", "Command (repository root, one MI355X):", "",
           f"    {command}", "", f"source digest: {source_digest()}", "",
           "| kernel | calls | average us | total ms | % |", "|---|---|---|---|---|"]
    for r in rows:
        out.append(f"| `{_short(r['Name'])}` | {r['Calls']} | "
                   f"{float(r['AverageNs']) / 1e3:.1f} | {float(r['TotalDurationNs']) / 1e6:.2f} | "
                   f"{float(r['Percentage']):.1f} |")
    return "\n".join(out) + "\n"


def _per_kernel(pmc_dir: str, counter: str):
    """kernel -> (dispatches, mean over dispatches of the counter summed over instances)."""
    per = defaultdict(lambda: defaultdict(float))
    for r in csv.DictReader(open(_one("*counter_collection.csv", pmc_dir))):
        if r["Counter_Name"] != counter:
            continue
        per[_short(r["Kernel_Name"])][r["Dispatch_Id"]] += float(r["Counter_Value"])
    return {k: (len(v), sum(v.values()) / len(v)) for k, v in per.items()}


def traffic_md(fetch_dir: str, write_dir: str, workload: str, fetch_cmd: str,
               write_cmd: str, calib_mib: int = 1024) -> str:
    fetch = _per_kernel(fetch_dir, "FETCH_SIZE")
    write = _per_kernel(write_dir, "WRITE_SIZE")
    # the reference is the elementwise kernel that reads the most (the add, not the fill
    # that initialises its source)
    calib = sorted((k for k in fetch if "elementwise" in k), key=lambda k: -fetch[k][1])
    if not calib:
        raise RuntimeError("reference copy kernel not found (run bench.py with --calib-copy-mib)")
    kib = calib_mib * 1024
    f_scale = kib / fetch[calib[0]][1]
    w_scale = kib / write[calib[0]][1]
    out = [f"# HBM traffic per launch, {workload} workload", "",
           "Commands (repository root, one MI355X), one counter per run:", "",
           f"    {fetch_cmd}", f"    {write_cmd}", "",
           f"Calibration: the reference kernel reads and writes {calib_mib} MiB; it read "
           f"{fetch[calib[0]][1]:.0f} KiB on FETCH_SIZE and {write[calib[0]][1]:.0f} KiB on "
           f"WRITE_SIZE, so fetch values are scaled by {f_scale:.4f} and write values by "
           f"{w_scale:.4f}.", "", f"source digest: {source_digest()}", "",
           "Each counter is summed over its instances per dispatch and averaged over "
           "dispatches; a stage served by several kernels sums them. The last column is "
           "scaled fetch + write in bytes.", "",
           "| stage | kernels | dispatches | fetch KiB (raw) | write KiB (raw) | HBM bytes per launch |",
           "|---|---|---|---|---|---|"]
    for stage, pat in STAGE_KERNELS:
        ks = [k for k in fetch if re.search(pat, k)]
        if not ks:
            continue
        f = sum(fetch[k][1] for k in ks)
        w = sum(write.get(k, (0, 0.0))[1] for k in ks)
        n = sum(fetch[k][0] for k in ks)
        total = 1024 * (f * f_scale + w * w_scale)
        out.append(f"| {stage} | {', '.join('`' + k + '`' for k in ks)} | {n} | {f:.0f} | "
                   f"{w:.0f} | {total:.0f} |")
    return "\n".join(out) + "\n"


def mfma_md(pmc_dir: str, command: str, cus: int = 256, simds_per_cu: int = 4,
            xcds: int = 8) -> str:
    """Executed MFMA utilisation per kernel: SQ_VALU_MFMA_BUSY_CYCLES summed over SIMDs
    over (GRBM_GUI_ACTIVE per XCD x SIMD count), plus instruction mix per MFMA."""
    per = defaultdict(lambda: defaultdict(float))
    disp = defaultdict(set)
    for r in csv.DictReader(open(_one("*counter_collection.csv", pmc_dir))):
        k = _short(r["Kernel_Name"])
        per[k][r["Counter_Name"]] += float(r["Counter_Value"])
        disp[k].add(r["Dispatch_Id"])
    out = ["# Executed MFMA utilisation per kernel", "", "Command (repository root, one MI355X):",
           "", f"    {command}", "", f"source digest: {source_digest()}", "",
           "utilisation = SQ_VALU_MFMA_BUSY_CYCLES / (GRBM_GUI_ACTIVE / XCDs x SIMDs), summed "
           "over the kernel's dispatches; it counts the MFMA work the kernel executes, plane "
           "products included.", "",
           "| kernel | dispatches | MFMA busy % | VALU / MFMA | LDS / MFMA |", "|---|---|---|---|---|"]
    for k, v in sorted(per.items(), key=lambda kv: -kv[1].get("SQ_VALU_MFMA_BUSY_CYCLES", 0)):
        m = v.get("SQ_INSTS_MFMA", 0)
        if not m or "GRBM_GUI_ACTIVE" not in v:
            continue
        util = v["SQ_VALU_MFMA_BUSY_CYCLES"] / (v["GRBM_GUI_ACTIVE"] / xcds * cus * simds_per_cu)
        out.append(f"| `{k}` | {len(disp[k])} | {100 * util:.1f} | "
                   f"{v.get('SQ_INSTS_VALU', 0) / m:.2f} | {v.get('SQ_INSTS_LDS', 0) / m:.2f} |")
    return "\n".join(out) + "\n"


def main(argv):
    if len(argv) >= 4 and argv[1] == "stats":
        text = stats_md(argv[3], argv[4] if len(argv) > 4 else "")
    elif len(argv) >= 4 and argv[1] == "mfma":
        text = mfma_md(argv[3], argv[4] if len(argv) > 4 else "")
    elif len(argv) >= 8 and argv[1] == "traffic":
        text = traffic_md(argv[3], argv[4], argv[5], argv[6], argv[7])
    else:
        print(__doc__, file=sys.stderr)
        return 2
    with open(argv[2], "w") as fh:
        fh.write(text)
    print(text)
    return 0


if __name__ == "__main__":
    sys.exit(main(sys.argv))
