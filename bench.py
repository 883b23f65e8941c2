#!/usr/bin/env python3
"""Benchmark of the tiled-attention hot path on one MI355X.

One step = one causal bf16 prefill of the 1.3B-model attention shape
(B=8, H=16, L=1024, D=128) through ``attn_prefill``; ``value`` is its
algorithmic TFLOP/s (4*D per visible query/key pair, causal pairs only),
inputs resident in HBM before the timed region. The same run also times the
paged-decode workloads (64 sequences x 40 heads, lengths U[128, 4096], q_len 1;
and 4 x 40 heads, 32768 keys, q_len 5, 16 splits, shared 2048-token prefix)
and reports their KV GB/s against the HBM peak under ``paged_decode``.

Kernel durations come from HIP events recorded on the stream the kernels run
on (torch's current stream, which the binding passes to the library). The
``cpu_baseline`` leg times the float64 CPU oracle on a bounded sample of the
same workload on this host's cores.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W]
"""

import argparse
import hashlib
import json
import math
import os
import sys
import time

PEAK_BF16_TFLOPS = 2500.0  # MI355X dense bf16 matrix peak, TFLOP/s
PEAK_HBM_GBS = 8000.0      # MI355X HBM3E peak, GB/s
ROOT = os.path.dirname(os.path.abspath(__file__))


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def prefill_flops(B, H, L, D, causal):
    pairs = L * (L + 1) // 2 if causal else L * L
    return 4.0 * D * pairs * B * H


def prefill_bytes(B, H, L, D, elem=2):
    return 4.0 * B * H * L * D * elem  # read Q, K, V once, write O once


def paged_bytes(lens, H, D, q_len, elem=2):
    kv = 2.0 * H * D * elem * sum(lens)
    qo = 2.0 * len(lens) * H * q_len * D * elem
    return kv, kv + qo


def source_digest(*names):
    h = hashlib.sha256()
    for n in names:
        with open(os.path.join(ROOT, "attention_tiled_qk_amd", "csrc", n), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def load_traffic(kernel_key, digest, algo_bytes):
    """HBM traffic per launch from committed rocprofv3 counter runs, if they were
    taken on the current kernel source; else None."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        data = json.load(f)
    ent = data.get(kernel_key)
    if not ent or ent.get("source_digest") != digest:
        return None
    return ent.get("hbm_bytes_per_launch")


def time_launches(torch, fn, warmup, steps):
    """Average duration (ms) of fn() over `steps` launches, HIP events per launch."""
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    starts = [torch.cuda.Event(enable_timing=True) for _ in range(steps)]
    ends = [torch.cuda.Event(enable_timing=True) for _ in range(steps)]
    t0 = time.perf_counter()
    for i in range(steps):
        starts[i].record()
        fn()
        ends[i].record()
    torch.cuda.synchronize()
    wall = (time.perf_counter() - t0) * 1e3
    per = [s.elapsed_time(e) for s, e in zip(starts, ends)]
    return sum(per) / len(per), wall, per


def cpu_baseline(spec, budget_s):
    """Time the oracle on as many heads of `spec` as fit in about budget_s."""
    import numpy as np
    import oracle
    from workloads import prefill_inputs
    try:
        from threadpoolctl import threadpool_info
        blas_threads = max((i.get("num_threads", 1) for i in threadpool_info()), default=1)
    except Exception:  # pragma: no cover
        blas_threads = None
    q, k, v = prefill_inputs(spec)
    pairs = [(b, h) for b in range(spec.B) for h in range(spec.H)]
    done = 0
    t0 = time.perf_counter()
    for b, h in pairs:
        oracle.dense_attention(q[b, h], k[b, h], v[b, h], spec.scale, spec.causal)
        done += 1
        if time.perf_counter() - t0 >= budget_s:
            break
    dt = time.perf_counter() - t0
    flops = prefill_flops(1, done, spec.L, spec.D, spec.causal)
    cores = len(os.sched_getaffinity(0))
    del np
    return {
        "value": flops / dt / 1e12,
        "unit": "TFLOP/s",
        "cores": blas_threads if blas_threads else cores,
        "host_cores": cores,
        "kind": "oracle",
        "sample": f"{done} of {len(pairs)} (batch, head) pairs of the same workload, float64, "
                  f"{dt:.1f} s wall; rate counts the same algorithmic (causal) FLOPs as the GPU",
    }


def bench_decode(torch, api, spec, warmup, steps):
    from workloads import paged_inputs
    log(f"[bench] building {spec.name} inputs")
    inp = paged_inputs(spec)
    dq, dk, dv, dt, dl = (t.cuda() for t in (inp.q, inp.k_pool, inp.v_pool, inp.block_tables,
                                              inp.seq_lens))
    lens = inp.seq_lens.tolist()
    B, H, q_len, D = inp.q.shape
    width = inp.block_tables.shape[1]
    ws_bytes = api.attn_paged_workspace_bytes(B, H, q_len, D, width, spec.num_splits)
    ws = torch.empty(max(ws_bytes // 4, 1), device="cuda", dtype=torch.float32)
    o = torch.empty_like(dq)
    splits = spec.num_splits

    def call():
        api.attn_paged_decode(dq, dk, dv, dt, dl, causal=spec.causal, scale=spec.scale,
                              num_splits=splits, o=o, workspace=ws)

    ms, wall, _ = time_launches(torch, call, warmup, steps)
    kv, total = paged_bytes(lens, H, D, q_len)
    unique_kv = kv
    if spec.shared_prefix_blocks:
        shared_tokens = spec.shared_prefix_blocks * 16
        unique_kv = kv - (B - 1) * 2.0 * H * D * 2 * shared_tokens
    res = {
        "workload": spec.name,
        "num_splits": splits if splits else "auto",
        "ms_per_call": ms,
        "kv_bytes": kv,
        "kv_GBps": kv / (ms * 1e-3) / 1e9,
        "frac_hbm_peak": kv / (ms * 1e-3) / 1e9 / PEAK_HBM_GBS,
    }
    if spec.shared_prefix_blocks:
        res["unique_kv_bytes"] = unique_kv
        res["unique_kv_GBps"] = unique_kv / (ms * 1e-3) / 1e9
    log(f"[bench] {spec.name}: {ms * 1e3:.1f} us/call, {res['kv_GBps']:.0f} GB/s")
    del dq, dk, dv, dt, dl, ws, o
    torch.cuda.empty_cache()
    return res


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--cpu-seconds", type=float, default=15.0,
                    help="budget of the CPU oracle baseline (0 disables it)")
    ap.add_argument("--no-decode", action="store_true", help="skip the paged-decode workloads")
    args = ap.parse_args()

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU only: this library has no multi-GPU path "
              "(attention shards by head with no exchange; see the design notes). "
              "Run with --gpus 1.", file=sys.stderr)
        sys.exit(2)

    import torch
    import attention_tiled_qk_amd as api
    from workloads import C2, C4, C5, prefill_inputs

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(2)

    spec = C2
    log(f"[bench] building {spec.name} inputs")
    q, k, v = (t.cuda() for t in prefill_inputs(spec))
    o = torch.empty_like(q)

    def step():
        api.attn_prefill(q, k, v, causal=spec.causal, scale=spec.scale, o=o)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    starts = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps)]
    ends = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        starts[i].record()
        step()
        ends[i].record()
    torch.cuda.synchronize()
    wall_ms = (time.perf_counter() - t0) * 1e3
    kernel_ms = sum(s.elapsed_time(e) for s, e in zip(starts, ends)) / args.steps
    ms_per_step = wall_ms / args.steps

    flops = prefill_flops(spec.B, spec.H, spec.L, spec.D, spec.causal)
    value = flops / (ms_per_step * 1e-3) / 1e12
    achieved = flops / (kernel_ms * 1e-3) / 1e12
    digest = source_digest("prefill_bf16.hip", "common.h")
    traffic = load_traffic("prefill_bf16_c2", digest, prefill_bytes(spec.B, spec.H, spec.L, spec.D))
    log(f"[bench] {spec.name}: {kernel_ms * 1e3:.1f} us/launch (events), "
        f"{ms_per_step * 1e3:.1f} us/step (wall), {achieved:.0f} TFLOP/s")

    out = {
        "metric": "prefill attn TFLOP/s (%MFMA peak); paged-decode KV GB/s (%HBM peak)",
        "value": value,
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "causal prefill bf16 B=8 H=16 L=1024 D=128 (1.3B-model attention shape)",
                   "B": spec.B, "H": spec.H, "L": spec.L, "D": spec.D, "causal": spec.causal,
                   "seed": spec.seed},
        "roofline": {
            "kernel": "prefill_bf16_kernel<128,4,causal>",
            "bound": "mfma",
            "achieved": achieved,
            "peak": PEAK_BF16_TFLOPS,
            "unit": "TFLOP/s",
            "frac": achieved / PEAK_BF16_TFLOPS,
            "traffic": traffic,
            "algorithmic_flops_per_launch": flops,
            "launch_ms_events": kernel_ms,
        },
    }
    del q, k, v, o
    torch.cuda.empty_cache()

    if not args.no_decode:
        decode = {}
        for s in (C4, C5):
            decode[s.name[:2]] = bench_decode(torch, api, s, args.warmup, max(args.steps // 2, 5))
        decode["bound"] = "hbm"
        decode["peak_GBps"] = PEAK_HBM_GBS
        out["paged_decode"] = decode

    if args.cpu_seconds > 0:
        log(f"[bench] cpu baseline (oracle, ~{args.cpu_seconds:.0f} s)")
        out["cpu_baseline"] = cpu_baseline(spec, args.cpu_seconds)
    else:
        out["cpu_baseline"] = None

    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
