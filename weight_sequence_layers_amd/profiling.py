"""Short text summaries of rocprofv3 output for the files kept under profiles/.

    python -m weight_sequence_layers_amd.profiling stats  OUT.md  TRACE_DIR   "<command>"
    python -m weight_sequence_layers_amd.profiling traffic OUT.md FETCH_DIR WRITE_DIR \
        WORKLOAD "<fetch command>" "<write command>"
    python -m weight_sequence_layers_amd.profiling mfma   OUT.md  PMC_DIR     "<command>"
    python -m weight_sequence_layers_amd.profiling counters OUT.md TITLE DIR... -- "<cmd>"...

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
# (stage, kernels, companions): each launch the library brackets for a stage runs one of the
# `kernels` (several patterns are alternative instantiations, e.g. by plane count) and any
# of the `companions` (kernels launched inside the same bracket, e.g. a split-K sum)
STAGE_KERNELS = [
    # k_front<BM, BN, WGM, WGN, FW, MODE, BK, PR>: MODE 0 applies, 1 and 2 take gradients
    ("front_q", r"k_front<(\d+, ){5}0, \d+, \d+>$", None),
    ("front_k", r"k_front<(\d+, ){5}[12], \d+, \d+>$", None),
    # k_out<BM, BN, WGM, WGN, MODE, PR>: MODE 0 is the query output, 1 and 2 the MSE error
    ("out", r"k_out<(\d+, ){4}0, \d+>$", None),
    ("mse", r"k_out<(\d+, ){4}[12], \d+>$", None),
    ("contract", r"k_contract<", r"k_contract_sum<"),
    ("ns_gram", r"k_ns_gram<", None),
    ("ns_poly", r"k_ns_poly<", None),
    ("ns_update", r"k_ns_update<", None),
    ("ns_small", r"k_ns_small<", None),
    ("renorm", r"k_renorm", None),
    ("split", r"ttt::k_split", None),
    ("resident", r"k_small_gelu<", None),
    ("dq", r"k_dq<|k_rowgemm<", None),
    ("tfront", r"k_tfront<", r"k_eta_sum"),
    ("ns_bwd", r"k_gemm2<", r"k_ns_fin"),
]


def source_digest(part: str = "layer") -> str:
    """Hash of the kernel sources: part "layer" covers every file under csrc/ that the TTT
    layer is built from, "block" the files of the block around it (ttt_block*)."""
    h = hashlib.sha256()
    csrc = os.path.join(PKG, "csrc")
    for f in sorted(os.listdir(csrc)):
        if f.startswith("ttt_block") != (part == "block"):
            continue
        with open(os.path.join(csrc, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def _short(name: str) -> str:
    """The kernel's name without its argument list and anonymous-namespace qualifier."""
    name = name.replace("(anonymous namespace)::", "")
    if name.endswith(")") and "(" in name:
        name = name[:name.rindex("(")]
    return name.strip()


def _one(pattern: str, d: str) -> str:
    found = glob.glob(os.path.join(d, "**", pattern), recursive=True)
    if not found:
        raise FileNotFoundError(f"no {pattern} under {d}")
    return found[0]


def stats_md(trace_dir: str, command: str) -> str:
    rows = list(csv.DictReader(open(_one("*kernel_stats.csv", trace_dir))))
    out = ["# Kernel durations", "", "Command (repository root, one MI355X):", "",
           f"    {command}", "", f"source digest: {source_digest()}", f"block source digest: {source_digest('block')}", "",
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
           f"{w_scale:.4f}.", "", f"source digest: {source_digest()}", f"block source digest: {source_digest('block')}", "",
           "Each counter is summed over its instances per dispatch. Per launch of a stage: "
           "the bytes of all its dispatches (the alternative instantiations that serve it "
           "and the companion kernels launched with it) over the number of its launches "
           "(the dispatches of the alternatives). The last column is scaled fetch + write "
           "in bytes.", "",
           "| stage | kernels | dispatches | fetch KiB (raw) | write KiB (raw) | HBM bytes per launch |",
           "|---|---|---|---|---|---|"]
    for stage, pat, comp in STAGE_KERNELS:
        ks = [k for k in fetch if re.search(pat, k)]
        if not ks:
            continue
        cs = [k for k in fetch if comp and re.search(comp, k)]
        n = sum(fetch[k][0] for k in ks)   # launches of the stage
        # KiB over every dispatch of the stage's kernels, per launch
        f = sum(fetch[k][0] * fetch[k][1] for k in ks + cs) / n
        w = sum(write.get(k, (0, 0.0))[0] * write.get(k, (0, 0.0))[1] for k in ks + cs) / n
        total = 1024 * (f * f_scale + w * w_scale)
        out.append(f"| {stage} | {', '.join('`' + k + '`' for k in ks + cs)} | {n} | "
                   f"{f:.0f} | {w:.0f} | {total:.0f} |")
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
           "", f"    {command}", "", f"source digest: {source_digest()}", f"block source digest: {source_digest('block')}", "",
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


def counters_md(pmc_dirs, command_lines, title: str) -> str:
    """Per-kernel averages (per dispatch, each counter summed over its instances) of every
    counter in one or more `rocprofv3 --pmc` directories, plus derived ratios when their
    counters are present: L2 hit rate, average latency of the L2's memory reads in cycles
    (outstanding-request level over requests), share of requests that went to DRAM, and the
    share of wave cycles spent waiting."""
    vals = defaultdict(dict)
    disp = defaultdict(int)
    for d in pmc_dirs:
        per = defaultdict(lambda: defaultdict(float))
        ids = defaultdict(set)
        for r in csv.DictReader(open(_one("*counter_collection.csv", d))):
            k = _short(r["Kernel_Name"])
            per[k][r["Counter_Name"]] += float(r["Counter_Value"])
            ids[k].add(r["Dispatch_Id"])
        for k, cs in per.items():
            n = len(ids[k])
            disp[k] = max(disp[k], n)
            for c, v in cs.items():
                vals[k][c] = v / n
    names = sorted({c for v in vals.values() for c in v})
    out = [f"# {title}", "", "Commands (repository root, one MI355X), one counter set per run:",
           ""] + [f"    {c}" for c in command_lines] + [
           "", f"source digest: {source_digest()}", f"block source digest: {source_digest('block')}", "",
           "Per dispatch, each counter summed over its instances and averaged over the "
           "kernel's dispatches. Derived: L2 hit % = TCC_HIT / (TCC_HIT + TCC_MISS); "
           "read latency (cycles) = TCC_EA0_RDREQ_LEVEL / TCC_EA0_RDREQ; DRAM % = "
           "TCC_EA0_RDREQ_DRAM / TCC_EA0_RDREQ; wait % = SQ_WAIT_ANY / SQ_WAVE_CYCLES.", ""]
    derived = ["L2 hit %", "read latency", "DRAM %", "wait %"]
    out.append("| kernel | dispatches | " + " | ".join(derived + names) + " |")
    out.append("|---|---|" + "---|" * (len(derived) + len(names)))
    for k in sorted(vals, key=lambda k: -vals[k].get("SQ_WAVE_CYCLES", vals[k].get(
            "TCC_EA0_RDREQ_sum", 0))):
        v = vals[k]
        g = lambda *cs: [v.get(c, v.get(c + "_sum")) for c in cs]
        hit, miss = g("TCC_HIT", "TCC_MISS")
        lvl, req, dram = g("TCC_EA0_RDREQ_LEVEL", "TCC_EA0_RDREQ", "TCC_EA0_RDREQ_DRAM")
        wa, wc = g("SQ_WAIT_ANY", "SQ_WAVE_CYCLES")
        d = [f"{100 * hit / (hit + miss):.1f}" if hit is not None and miss is not None and hit + miss else "",
             f"{lvl / req:.0f}" if lvl is not None and req else "",
             f"{100 * dram / req:.1f}" if dram is not None and req else "",
             f"{100 * wa / wc:.1f}" if wa is not None and wc else ""]
        out.append(f"| `{k}` | {disp[k]} | " + " | ".join(d) + " | " +
                   " | ".join(f"{v[c]:.4g}" if c in v else "" for c in names) + " |")
    return "\n".join(out) + "\n"


def main(argv):
    if len(argv) >= 4 and argv[1] == "stats":
        text = stats_md(argv[3], argv[4] if len(argv) > 4 else "")
    elif len(argv) >= 4 and argv[1] == "mfma":
        text = mfma_md(argv[3], argv[4] if len(argv) > 4 else "")
    elif len(argv) >= 5 and argv[1] == "counters":
        # counters OUT.md TITLE DIR1 [DIR2 ...] -- CMD1 [CMD2 ...]
        sep = argv.index("--") if "--" in argv else len(argv)
        text = counters_md(argv[4:sep], argv[sep + 1:], argv[3])
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
