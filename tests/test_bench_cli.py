"""Host-side checks of bench.py's command line (no GPU is touched)."""
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.mark.parametrize("n", ["2", "8", "0"])
def test_more_than_one_gpu_is_refused(n):
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", n],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode != 0
    assert "one GPU" in (r.stdout + r.stderr)


def test_cpu_baseline_leg_reports_its_sample():
    sys.path.insert(0, ROOT)
    import bench
    import ttt_inputs as ti
    res = bench.cpu_baseline(ti.CONFIGS["tiny"], min_seconds=0.0)
    assert res["kind"] == "oracle" and res["unit"] == "tokens/s" and res["value"] > 0
    assert res["cores"] >= 1 and "1 of 1" in res["sample"]
    json.dumps(res)


@pytest.mark.parametrize("name", ["tiny", "lm", "long", "imageset"])
def test_stage_flops_add_up_to_the_layer_total(name):
    # the per-stage algorithmic FLOP the roofline uses sum to the layer's total
    sys.path.insert(0, ROOT)
    import bench
    import ttt_inputs as ti
    cfg = ti.CONFIGS[name]
    f = bench.stage_flops(cfg)
    total = sum(v for k, v in f.items() if k != "resident")
    assert abs(total - bench.total_flops(cfg)) <= 1e-9 * total


def test_chunk_backward_flop_accounting():
    """The chunk backward's per-stage FLOP sum to 58 b d dh per problem for the GEMMs on
    tokens and 15 (14 m^2 n + 8 m^3) for Newton-Schulz (five iterations forward and back,
    three matrices)."""
    import bench
    import ttt_inputs as ti
    cfg = ti.CONFIGS["lm"].replace(seq_len=2048)
    P, b, d, dh = 8, 2048, 512, 1024
    total = sum(bench.chunk_backward_flops(cfg).values())
    expect = P * (58.0 * b * d * dh + 15 * (14.0 * d * d * dh + 8.0 * d ** 3))
    assert abs(total - expect) <= 1e-9 * expect


def test_recorded_traffic_only_for_the_workload_as_profiled():
    # profiles/lm_traffic.md holds the bytes of the default LM run; a command line that
    # changes the kernels' work gets none
    import argparse
    sys.path.insert(0, ROOT)
    import bench
    plain = argparse.Namespace(batch=None, momentum=0.0, lr=None, weight_decay=0.0, planes=None)
    assert bench.traffic_for(plain, "lm", "ns_update") == bench.recorded_traffic("lm", "ns_update")
    for kw in (dict(batch=8), dict(momentum=0.9), dict(lr="0.5"), dict(weight_decay=0.1),
               dict(planes="1,1,1,0")):
        assert bench.traffic_for(argparse.Namespace(**{**vars(plain), **kw}), "lm",
                                 "ns_update") is None
