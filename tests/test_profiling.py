"""The profile summaries' arithmetic, on synthetic rocprofv3 counter files: HBM bytes per
launch of a stage average its alternative kernels by dispatch and add the companion kernels
launched with it, after scaling by the reference copy."""
import csv
import os

import weight_sequence_layers_amd.profiling as P

FIELDS = ["Kernel_Name", "Dispatch_Id", "Counter_Name", "Counter_Value"]


def _write(d, rows):
    os.makedirs(d, exist_ok=True)
    with open(os.path.join(d, "x_counter_collection.csv"), "w", newline="") as fh:
        w = csv.DictWriter(fh, fieldnames=FIELDS)
        w.writeheader()
        for r in rows:
            w.writerow(dict(zip(FIELDS, r)))


def _stage_bytes(text, stage):
    for line in text.splitlines():
        if line.startswith(f"| {stage} |"):
            return float(line.split("|")[-2])
    raise KeyError(stage)


def test_traffic_per_launch(tmp_path):
    ref = "void at::native::vectorized_elementwise_kernel<4>(x)"
    f = [(ref, "0", "FETCH_SIZE", 512.0)]      # reads half of what it moves: scale 2
    w = [(ref, "0", "WRITE_SIZE", 1024.0)]     # exact: scale 1
    for i in range(3):   # two-plane instantiation, 3 launches
        f.append(("void ttt::k_ns_update<2>(a)", f"1{i}", "FETCH_SIZE", 100.0))
        w.append(("void ttt::k_ns_update<2>(a)", f"1{i}", "WRITE_SIZE", 10.0))
    for i in range(2):   # one-plane instantiation, 2 launches
        f.append(("void ttt::k_ns_update<1>(a)", f"2{i}", "FETCH_SIZE", 50.0))
        w.append(("void ttt::k_ns_update<1>(a)", f"2{i}", "WRITE_SIZE", 10.0))
    for i in range(2):   # a contraction and its partial sum per launch
        f.append(("void ttt::k_contract<1>(a)", f"3{i}", "FETCH_SIZE", 40.0))
        w.append(("void ttt::k_contract<1>(a)", f"3{i}", "WRITE_SIZE", 4.0))
        f.append(("void ttt::k_contract_sum<1>(a)", f"4{i}", "FETCH_SIZE", 8.0))
        w.append(("void ttt::k_contract_sum<1>(a)", f"4{i}", "WRITE_SIZE", 2.0))
    _write(str(tmp_path / "f"), f)
    _write(str(tmp_path / "w"), w)
    t = P.traffic_md(str(tmp_path / "f"), str(tmp_path / "w"), "x", "f", "w", calib_mib=1)
    assert _stage_bytes(t, "ns_update") == 1024 * ((3 * 100 + 2 * 50) / 5 * 2 + 10)
    assert _stage_bytes(t, "contract") == 1024 * ((40 + 8) * 2 + (4 + 2))


def test_kernel_names_shortened():
    assert P._short("void ttt::(anonymous namespace)::k_blk_linear<1>(ttt::LinearArgs)") == \
        "void ttt::k_blk_linear<1>"
    assert P._short("void ttt::k_ns_gram<128, 4, 4, 2, 1, 1>(ttt::NsArgs)") == \
        "void ttt::k_ns_gram<128, 4, 4, 2, 1, 1>"
    assert P._short("__amd_rocclr_copyBuffer") == "__amd_rocclr_copyBuffer"


def test_stage_of_each_kernel_name():
    # every stage kernel's name (as rocprofv3 reports it, shortened) maps to one stage
    import re
    cases = {
        "void ttt::k_front<128, 128, 2, 4, 0, 0, 32, 0>": "front_q",
        "void ttt::k_front<64, 64, 2, 2, 0, 0, 64, 3>": "front_q",
        "void ttt::k_front<128, 128, 2, 4, 0, 1, 64, 0>": "front_k",
        "void ttt::k_front<64, 64, 2, 2, 0, 1, 32, 2>": "front_k",
        "void ttt::k_front<128, 128, 2, 4, 1, 2, 32, 0>": "front_k",
        "void ttt::k_out<128, 128, 2, 4, 0, 0>": "out",
        "void ttt::k_out<64, 64, 2, 2, 0, 3>": "out",
        "void ttt::k_out<128, 128, 2, 4, 1, 0>": "mse",
        "void ttt::k_out<128, 128, 2, 4, 2, 0>": "mse",
        "void ttt::k_contract<64, 128, 2, 4, 3, 3>": "contract",
        "void ttt::k_ns_update<128, 128, 2, 4, 2, 32, 1, 1>": "ns_update",
        "void ttt::k_renorm<4>": "renorm",
        "ttt::k_split3": "split",
    }
    for name, stage in cases.items():
        hits = [s for s, pat, _ in P.STAGE_KERNELS if re.search(pat, name)]
        assert hits == [stage], (name, hits)
