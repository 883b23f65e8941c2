"""Host-side checks of bench.py (no GPU): the one-GPU refusal, the algorithmic
FLOP count and the rule that an HBM traffic figure is reported only when it was
taken on the current kernel source."""

import json
import os
import subprocess
import sys

import bench

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2", "--steps", "1",
                        "--warmup", "0"], capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr


def test_prefill_flops_count_visible_pairs():
    # causal: row i sees i + 1 keys, 4 D FLOPs per visible (query, key) pair
    for B, H, L, D in ((1, 1, 1, 64), (1, 1, 128, 64), (8, 16, 1024, 128), (1, 40, 4096, 128)):
        pairs = sum(i + 1 for i in range(L))
        assert bench.prefill_flops(B, H, L, D, True) == 4.0 * D * pairs * B * H
        assert bench.prefill_flops(B, H, L, D, False) == 4.0 * D * L * L * B * H
    # the workloads' headline figures
    assert bench.prefill_flops(8, 16, 1024, 128, True) == 34393292800.0
    assert bench.prefill_flops(1, 40, 4096, 128, True) == 171840634880.0


def test_traffic_only_for_the_current_kernel_source():
    with open(os.path.join(ROOT, "profiles", "traffic.json")) as f:
        tj = json.load(f)
    ent = tj["prefill_c2"]
    assert bench.load_traffic("prefill_c2", ent["source_digest"]) == ent["hbm_bytes_per_launch"]
    assert bench.load_traffic("prefill_c2", "0" * 16) is None
    assert bench.load_traffic("no_such_workload", ent["source_digest"]) is None
