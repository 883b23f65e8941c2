#!/usr/bin/env python3
"""Benchmark of the tiled-attention hot path on one MI355X.

One step = one causal bf16 prefill of the 1.3B-model attention shape
(B=8, H=16, L=1024, D=128) through ``attn_prefill``; ``value`` is its
algorithmic TFLOP/s (4*D FLOPs per visible query/key pair, causal pairs only)
over the wall clock of the timed steps, inputs resident in HBM before the timed
region. ``roofline`` prices the prefill kernel alone, its average duration
taken from HIP events recorded around the timed back-to-back launches on the
stream the library launches on (torch's current stream, which the binding
passes down).

The same run also measures, under ``secondary``:
  * c1: causal fp32 prefill B=1, H=1, L=128, D=64 (the correctness case; time only);
  * c3: causal bf16 prefill B=1, H=40, L=4096, D=128 (13B-style long prompt);
  * c4: paged decode, 64 sequences x 40 heads, q_len 1, lengths U[128, 4096];
  * c5: paged verify, 4 sequences x 40 heads, q_len 5, 32768 keys, shared
    2048-token prefix, 16 splits merged by log-sum-exp;
  * c4g: grouped-query paged decode, 64 sequences, 64 query heads over 8 KV
    heads, q_len 1, lengths U[128, 4096];
  * cpf: chunked prefill over the paged cache, 8 sequences x 40 heads, a
    512-token chunk after a 3584-token cached prefix;
  * append: writing that 512-token chunk's K and V into the paged pools
    (attn_paged_append), priced against HBM bandwidth;
  * c4f8: the c4 decode over an FP8 (E4M3) cache with per-(block, head)
    scales (attn_paged_decode_fp8): one byte per cached value;
each with its own roofline entry (MFMA TFLOP/s or HBM GB/s); and
  * probe: the read bandwidth HBM sustains for the paged kernels' access
    patterns -- 4 KiB and 2 KiB blocks of a 2.5 GiB buffer in random order,
    and 4 KiB blocks in address order (probe/, a library of its own: loads only,
    nontemporal like the paged kernels; random 4 KiB also with the default
    cache policy).
Each prefill and paged decode entry also carries ``cache_control``: the median
single-launch time with warm caches and after a 512 MiB pass that evicts the
MALL, so that the timed rate can be read against a cold-cache one. It runs
before the warm-up and the timed launches, and not under ``--only``.
The
``cpu_baseline`` leg times the float64 CPU oracle on a bounded sample of the
c2 workload on this host's cores.

``--only NAME`` runs a single workload (c1, c2, c3, c4, c5, c4g, cpf, append, c4f8, probe, or
``copy``: a plain device-to-device copy of 2 GiB used to calibrate HBM byte
counters) and prints its entry; that is the form the profiler runs use.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--only NAME]
"""

import argparse
import hashlib
import json
import os
import sys
import time

PEAK_BF16_TFLOPS = 2500.0  # MI355X dense bf16 matrix peak, TFLOP/s
PEAK_HBM_GBS = 8000.0      # MI355X HBM3E peak, GB/s
ROOT = os.path.dirname(os.path.abspath(__file__))
METRIC = "prefill attn TFLOP/s (%MFMA peak); paged-decode KV GB/s (%HBM peak)"


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def prefill_flops(B, H, L, D, causal):
    pairs = L * (L + 1) // 2 if causal else L * L
    return 4.0 * D * pairs * B * H


def source_digest(*names):
    h = hashlib.sha256()
    for n in names:
        with open(os.path.join(ROOT, "attention_tiled_qk_amd", "csrc", n), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


KERNEL_SOURCES = {
    "prefill": ("prefill_bf16.hip", "common.h"),
    "paged": ("paged.hip", "common.h"),
    "append": ("kv_append.hip", "common.h"),
}


def load_traffic(key, digest):
    """HBM bytes per launch from the committed rocprofv3 counter runs, if they
    were taken on the current kernel source; else None."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        data = json.load(f)
    ent = data.get(key)
    if not ent or ent.get("source_digest") != digest:
        return None
    return ent.get("hbm_bytes_per_launch")


def time_launches(torch, fn, warmup, steps):
    """Average launch duration (ms) from HIP events recorded on the launch stream
    around `steps` back-to-back calls, and the wall time (ms) of those calls.

    Events bracket the whole run rather than each call: the host enqueues faster
    than the kernels run, so the stream never idles between launches and the
    event interval is the kernels' own time."""
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    start.record()
    for _ in range(steps):
        fn()
    end.record()
    torch.cuda.synchronize()
    wall = (time.perf_counter() - t0) * 1e3
    return start.elapsed_time(end) / steps, wall


FLUSH_BYTES = 512 << 20  # twice the MI355X's 256 MB last-level (MALL) cache
WITH_CACHE_CONTROL = True  # off for --only, the single-workload runs the profiler traces


def cache_control(torch, fn, calls=20):
    """Single launches timed one by one with HIP events, with the caches warm
    and cold. Each sample runs the same work -- one pass over a 512 MiB scratch
    buffer and two launches -- and times the second launch: warm, the pass
    comes first and the untimed launch re-reads the inputs into the caches;
    cold, the pass sits between the two launches and evicts the L2s and the
    MALL. The pass is a write (which also leaves dirty lines for the timed
    launch to share HBM with while they drain) or a read (which leaves none).
    The medians (us) bound the help the last-level cache gives the timed rate,
    whose back-to-back launches may find part of their inputs still cached."""
    scratch = torch.empty(FLUSH_BYTES, dtype=torch.uint8, device="cuda")
    words = scratch.view(torch.int32)
    sink = torch.empty((), dtype=torch.int64, device="cuda")
    passes = {"write": lambda i: scratch.fill_(i & 255),
              "read": lambda i: torch.sum(words, dim=0, dtype=torch.int64, out=sink)}
    res = {"flush_bytes": FLUSH_BYTES, "calls": calls}
    fn()
    torch.cuda.synchronize()
    for kind, flush in passes.items():
        res[kind] = {}
        for name, between in (("warm_us", False), ("flushed_us", True)):
            evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
                   for _ in range(calls)]
            for i, (a, b) in enumerate(evs):
                if not between:
                    flush(i)
                fn()
                if between:
                    flush(i)
                a.record()
                fn()
                b.record()
            torch.cuda.synchronize()
            times = sorted(a.elapsed_time(b) * 1e3 for a, b in evs)
            res[kind][name] = times[calls // 2]
    del scratch, words, sink
    torch.cuda.empty_cache()
    log("[bench]   cache control (single launches, medians): " + ", ".join(
        f"{kind} pass {r['warm_us']:.1f} us warm / {r['flushed_us']:.1f} us flushed"
        for kind, r in ((k, res[k]) for k in passes)))
    return res


def device_info(torch):
    """Compute units and peak engine clock of the current device, the peaks the
    rooflines are priced against, and the dense bf16 matrix peak implied by
    the units and clock (4096 FLOP per clock per CU)."""
    import ctypes
    dev = torch.cuda.current_device()
    p = torch.cuda.get_device_properties(dev)
    info = {"name": p.name, "arch": p.gcnArchName, "compute_units": p.multi_processor_count,
            "peak_bf16_tflops_used": PEAK_BF16_TFLOPS, "peak_hbm_gbs_used": PEAK_HBM_GBS}
    try:
        hip = ctypes.CDLL("libamdhip64.so.7")
        khz = ctypes.c_int(0)
        HIP_ATTR_CLOCK_RATE_KHZ = 5  # hipDeviceAttributeClockRate
        if hip.hipDeviceGetAttribute(ctypes.byref(khz), HIP_ATTR_CLOCK_RATE_KHZ, dev) == 0 and khz.value > 0:
            info["max_engine_clock_mhz"] = khz.value / 1e3
            info["peak_bf16_tflops_from_clock"] = p.multi_processor_count * 4096 * khz.value * 1e3 / 1e12
    except OSError:
        pass
    return info


def cpu_baseline(spec, budget_s):
    """Time the oracle on the host: one warm-up head, then up to three passes
    over the workload's (batch, head) pairs (each pass cut short at a third of
    the budget), reporting the median pass rate."""
    import statistics
    import oracle
    from workloads import prefill_inputs
    try:
        from threadpoolctl import threadpool_info
        blas_threads = max((i.get("num_threads", 1) for i in threadpool_info()), default=1)
    except Exception:  # pragma: no cover
        blas_threads = None
    q, k, v = prefill_inputs(spec)
    pairs = [(b, h) for b in range(spec.B) for h in range(spec.H)]
    oracle.dense_attention(q[0, 0], k[0, 0], v[0, 0], spec.scale, spec.causal)  # warm-up
    rates, done_per_pass, walls = [], [], []
    for _ in range(3):
        done = 0
        t0 = time.perf_counter()
        for b, h in pairs:
            oracle.dense_attention(q[b, h], k[b, h], v[b, h], spec.scale, spec.causal)
            done += 1
            if time.perf_counter() - t0 >= budget_s / 3:
                break
        dt = time.perf_counter() - t0
        rates.append(prefill_flops(1, done, spec.L, spec.D, spec.causal) / dt / 1e12)
        done_per_pass.append(done)
        walls.append(dt)
    cores = len(os.sched_getaffinity(0))
    lo, hi = min(done_per_pass), max(done_per_pass)
    span = f"{lo}" if lo == hi else f"{lo}-{hi}"
    return {
        "value": statistics.median(rates),
        "unit": "TFLOP/s",
        "cores": blas_threads if blas_threads else cores,
        "host_cores": cores,
        "kind": "oracle",
        "sample": f"median of 3 passes over {span} of the "
                  f"{len(pairs)} (batch, head) pairs of the c2 workload, float64, "
                  f"{sum(walls):.1f} s wall in all; the rate counts the same algorithmic (causal) "
                  f"FLOPs as the GPU although the oracle computes every pair of the square",
    }


def bench_prefill(torch, api, spec, warmup, steps, key):
    import ctypes
    from workloads import prefill_inputs
    log(f"[bench] building {spec.name} inputs")
    q, k, v = (t.cuda() for t in prefill_inputs(spec))
    o = torch.empty_like(q)
    api.attn_prefill(q, k, v, causal=spec.causal, scale=spec.scale, o=o)  # validates once
    # the same C-ABI call with its arguments marshalled once, so that the host
    # enqueues faster than the kernel runs and back-to-back launches keep the
    # stream busy
    P = ctypes.c_void_p
    args = (P(q.data_ptr()), P(k.data_ptr()), P(v.data_ptr()), P(o.data_ptr()), None,
            spec.B, spec.H, spec.L, spec.D, int(spec.causal), ctypes.c_float(spec.scale),
            api.ATTN_BF16, P(torch.cuda.current_stream().cuda_stream))
    fn = api.lib.attn_prefill

    def call():
        if fn(*args) != 0:
            raise RuntimeError("attn_prefill failed")

    control = cache_control(torch, call) if WITH_CACHE_CONTROL else None
    kernel_ms, wall = time_launches(torch, call, warmup, steps)
    flops = prefill_flops(spec.B, spec.H, spec.L, spec.D, spec.causal)
    achieved = flops / (kernel_ms * 1e-3) / 1e12
    traffic = load_traffic(key, source_digest(*KERNEL_SOURCES["prefill"]))
    log(f"[bench] {spec.name}: {kernel_ms * 1e3:.1f} us/launch (events), "
        f"{wall / steps * 1e3:.1f} us/step (wall), {achieved:.0f} TFLOP/s "
        f"({achieved / PEAK_BF16_TFLOPS:.1%} of peak)")
    del q, k, v, o
    torch.cuda.empty_cache()
    return {
        "workload": spec.name,
        "ms_per_step": wall / steps,
        "value": flops / (wall / steps * 1e-3) / 1e12,
        "roofline": {
            "kernel": f"prefill_bf16_pipe_kernel<{spec.D}, 4, 64, causal={int(spec.causal)}>",
            "bound": "mfma",
            "achieved": achieved,
            "peak": PEAK_BF16_TFLOPS,
            "unit": "TFLOP/s",
            "frac": achieved / PEAK_BF16_TFLOPS,
            "traffic": traffic,
            "algorithmic_flops_per_launch": flops,
            "launch_us_events": kernel_ms * 1e3,
        },
        "cache_control": control,
    }


def bench_prefill_f32(torch, api, spec, warmup, steps):
    """The fp32 correctness case: launch-latency bound, reported as time only."""
    import ctypes
    from workloads import prefill_inputs
    q, k, v = (t.cuda() for t in prefill_inputs(spec))
    o = torch.empty_like(q)
    api.attn_prefill(q, k, v, causal=spec.causal, scale=spec.scale, o=o)  # validates once
    P = ctypes.c_void_p
    args = (P(q.data_ptr()), P(k.data_ptr()), P(v.data_ptr()), P(o.data_ptr()), None,
            spec.B, spec.H, spec.L, spec.D, int(spec.causal), ctypes.c_float(spec.scale),
            api.ATTN_F32, P(torch.cuda.current_stream().cuda_stream))
    fn = api.lib.attn_prefill

    def call():
        if fn(*args) != 0:
            raise RuntimeError("attn_prefill failed")

    ms, wall = time_launches(torch, call, warmup, steps)
    flops = prefill_flops(spec.B, spec.H, spec.L, spec.D, spec.causal)
    log(f"[bench] {spec.name}: {ms * 1e3:.1f} us/launch (events), {wall / steps * 1e3:.1f} us/step (wall)")
    return {"workload": spec.name, "ms_per_step": wall / steps, "launch_us_events": ms * 1e3,
            "algorithmic_flops_per_launch": flops,
            "note": "correctness configuration; launch-latency bound, time only"}


def bench_paged(torch, api, spec, warmup, steps, key):
    from workloads import paged_inputs
    log(f"[bench] building {spec.name} inputs")
    inp = paged_inputs(spec)
    dq, dk, dv, dt, dl = (t.cuda() for t in (inp.q, inp.k_pool, inp.v_pool, inp.block_tables,
                                              inp.seq_lens))
    lens = inp.seq_lens.tolist()
    B, Hq, q_len, D = inp.q.shape
    H = inp.k_pool.shape[1]  # KV heads (fewer than Hq for grouped-query attention)
    width = inp.block_tables.shape[1]
    ws_bytes = api.attn_paged_gqa_workspace_bytes(B, Hq, H, q_len, D, width, spec.num_splits)
    ws = torch.empty(max(ws_bytes // 4, 1), device="cuda", dtype=torch.float32)
    o = torch.empty_like(dq)
    api.attn_paged_decode(dq, dk, dv, dt, dl, causal=spec.causal, scale=spec.scale,
                          num_splits=spec.num_splits, o=o, workspace=ws)  # validates once
    import ctypes
    P = ctypes.c_void_p
    heads = (Hq,) if Hq == H else (Hq, H)
    args = (P(dq.data_ptr()), P(dk.data_ptr()), P(dv.data_ptr()), P(dt.data_ptr()),
            P(dl.data_ptr()), P(o.data_ptr()), None, B, *heads, q_len, D, dk.shape[0], width, 16,
            int(spec.causal), ctypes.c_float(spec.scale), spec.num_splits, P(ws.data_ptr()),
            ctypes.c_size_t(ws.numel() * 4), api.ATTN_BF16,
            P(torch.cuda.current_stream().cuda_stream))
    fn = api.lib.attn_paged_decode if Hq == H else api.lib.attn_paged_decode_gqa

    def call():
        if fn(*args) != 0:
            raise RuntimeError("paged decode failed")

    control = cache_control(torch, call) if WITH_CACHE_CONTROL else None
    ms, wall = time_launches(torch, call, warmup, steps)
    # K and V bytes of every visible token, as the sequences address them
    kv = 2.0 * H * D * 2 * sum(lens)
    # bytes that must come from HBM: the shared prefix blocks are read once
    unique_kv = kv - (B - 1) * 2.0 * H * D * 2 * spec.shared_prefix_blocks * 16
    gbs = unique_kv / (ms * 1e-3) / 1e9
    traffic = load_traffic(key, source_digest(*KERNEL_SOURCES["paged"]))
    log(f"[bench] {spec.name}: {ms * 1e3:.1f} us/call, {gbs:.0f} GB/s ({gbs / PEAK_HBM_GBS:.1%})")
    res = {
        "workload": spec.name,
        "num_splits": spec.num_splits if spec.num_splits else "auto",
        "ms_per_step": wall / steps,
        "value": unique_kv / (wall / steps * 1e-3) / 1e9,
        "roofline": {
            "kernel": "paged_attn_kernel<128> (+ lse_merge_kernel when split)",
            "bound": "hbm",
            "achieved": gbs,
            "peak": PEAK_HBM_GBS,
            "unit": "GB/s",
            "frac": gbs / PEAK_HBM_GBS,
            "traffic": traffic,
            "algorithmic_bytes_per_launch": unique_kv,
            "logical_kv_bytes": kv,
            "launch_us_events": ms * 1e3,
        },
        "cache_control": control,
    }
    del dq, dk, dv, dt, dl, ws, o
    torch.cuda.empty_cache()
    return res


def bench_paged_prefill(torch, api, spec, warmup, steps, key):
    import ctypes
    from workloads import paged_inputs
    log(f"[bench] building {spec.name} inputs")
    inp = paged_inputs(spec)
    dq, dk, dv, dt, dl = (t.cuda() for t in (inp.q, inp.k_pool, inp.v_pool, inp.block_tables,
                                              inp.seq_lens))
    B, H, q_len, D = inp.q.shape
    o = torch.empty_like(dq)
    api.attn_paged_prefill(dq, dk, dv, dt, dl, causal=spec.causal, scale=spec.scale, o=o)
    P = ctypes.c_void_p
    args = (P(dq.data_ptr()), P(dk.data_ptr()), P(dv.data_ptr()), P(dt.data_ptr()),
            P(dl.data_ptr()), P(o.data_ptr()), None, B, H, q_len, D, dk.shape[0],
            inp.block_tables.shape[1], 16, int(spec.causal), ctypes.c_float(spec.scale),
            api.ATTN_BF16, P(torch.cuda.current_stream().cuda_stream))
    fn = api.lib.attn_paged_prefill

    def call():
        if fn(*args) != 0:
            raise RuntimeError("attn_paged_prefill failed")

    control = cache_control(torch, call) if WITH_CACHE_CONTROL else None
    ms, wall = time_launches(torch, call, warmup, steps)
    # visible (query, key) pairs: query t of a sequence of n keys sees n - q_len + t + 1
    pairs = 0
    for n in inp.seq_lens.tolist():
        pairs += sum(n - q_len + t + 1 for t in range(q_len)) if spec.causal else n * q_len
    flops = 4.0 * D * H * pairs
    achieved = flops / (ms * 1e-3) / 1e12
    traffic = load_traffic(key, source_digest(*KERNEL_SOURCES["prefill"]))
    log(f"[bench] {spec.name}: {ms * 1e3:.1f} us/launch, {achieved:.0f} TFLOP/s "
        f"({achieved / PEAK_BF16_TFLOPS:.1%} of peak)")
    del dq, dk, dv, dt, dl, o
    torch.cuda.empty_cache()
    return {
        "workload": spec.name,
        "ms_per_step": wall / steps,
        "value": flops / (wall / steps * 1e-3) / 1e12,
        "roofline": {
            "kernel": f"prefill_bf16_pipe_kernel<{D}, paged>",
            "bound": "mfma",
            "achieved": achieved,
            "peak": PEAK_BF16_TFLOPS,
            "unit": "TFLOP/s",
            "frac": achieved / PEAK_BF16_TFLOPS,
            "traffic": traffic,
            "algorithmic_flops_per_launch": flops,
            "launch_us_events": ms * 1e3,
        },
        "cache_control": control,
    }


def bench_paged_fp8(torch, api, spec, warmup, steps, key):
    import ctypes
    from workloads import paged_inputs_fp8
    log(f"[bench] building {spec.name} inputs")
    inp = paged_inputs_fp8(spec)
    dq, dk, dv, dks, dvs, dt, dl = (t.cuda() for t in (inp.q, inp.k_codes, inp.v_codes,
                                                        inp.k_scale, inp.v_scale,
                                                        inp.block_tables, inp.seq_lens))
    lens = inp.seq_lens.tolist()
    B, Hq, q_len, D = inp.q.shape
    H = inp.k_codes.shape[1]
    width = inp.block_tables.shape[1]
    ws_bytes = api.attn_paged_gqa_workspace_bytes(B, Hq, H, q_len, D, width, spec.num_splits)
    ws = torch.empty(max(ws_bytes // 4, 1), device="cuda", dtype=torch.float32)
    o = torch.empty_like(dq)
    api.attn_paged_decode_fp8(dq, dk, dv, dks, dvs, dt, dl, causal=spec.causal, scale=spec.scale,
                              num_splits=spec.num_splits, o=o, workspace=ws)  # validates once
    P = ctypes.c_void_p
    args = (P(dq.data_ptr()), P(dk.data_ptr()), P(dv.data_ptr()), P(dks.data_ptr()),
            P(dvs.data_ptr()), P(dt.data_ptr()), P(dl.data_ptr()), P(o.data_ptr()), None, B, Hq,
            H, q_len, D, dk.shape[0], width, 16, int(spec.causal), ctypes.c_float(spec.scale),
            spec.num_splits, P(ws.data_ptr()), ctypes.c_size_t(ws.numel() * 4),
            P(torch.cuda.current_stream().cuda_stream))
    fn = api.lib.attn_paged_decode_fp8

    def call():
        if fn(*args) != 0:
            raise RuntimeError("attn_paged_decode_fp8 failed")

    control = cache_control(torch, call) if WITH_CACHE_CONTROL else None
    ms, wall = time_launches(torch, call, warmup, steps)
    # one byte per cached K and V value, plus the two scales of each (block, head)
    blocks = sum(-(-n // 16) for n in lens)
    kv = 2.0 * H * D * sum(lens) + 2.0 * 4 * H * blocks
    gbs = kv / (ms * 1e-3) / 1e9
    log(f"[bench] {spec.name}: {ms * 1e3:.1f} us/call, {gbs:.0f} GB/s ({gbs / PEAK_HBM_GBS:.1%})")
    del dq, dk, dv, dks, dvs, dt, dl, ws, o
    torch.cuda.empty_cache()
    return {
        "workload": spec.name,
        "num_splits": spec.num_splits if spec.num_splits else "auto",
        "ms_per_step": wall / steps,
        "value": kv / (wall / steps * 1e-3) / 1e9,
        "roofline": {
            "kernel": "paged_attn_kernel<128, fp8> (+ lse_merge_kernel when split)",
            "bound": "hbm",
            "achieved": gbs,
            "peak": PEAK_HBM_GBS,
            "unit": "GB/s",
            "frac": gbs / PEAK_HBM_GBS,
            "traffic": load_traffic(key, source_digest(*KERNEL_SOURCES["paged"])),
            "algorithmic_bytes_per_launch": kv,
            "launch_us_events": ms * 1e3,
        },
        "cache_control": control,
    }


def bench_append(torch, api, spec, warmup, steps, key):
    """K/V of one q_len-token chunk per sequence written into the pools."""
    import ctypes
    from workloads import paged_layout
    log(f"[bench] building append inputs for {spec.name}")
    lens, tables, total, _ = paged_layout(spec)
    B, H, n_new, D = spec.B, spec.H, spec.q_len, spec.D
    g = torch.Generator(device="cuda").manual_seed(spec.seed)
    k_new = torch.randn((B, H, n_new, D), device="cuda", generator=g).to(torch.bfloat16)
    v_new = torch.randn((B, H, n_new, D), device="cuda", generator=g).to(torch.bfloat16)
    k_pool = torch.zeros((total, H, 16, D), device="cuda", dtype=torch.bfloat16)
    v_pool = torch.zeros_like(k_pool)
    dt, dl = tables.cuda(), lens.cuda()
    api.attn_paged_append(k_new, v_new, k_pool, v_pool, dt, dl)  # validates once
    P = ctypes.c_void_p
    args = (P(k_new.data_ptr()), P(v_new.data_ptr()), P(k_pool.data_ptr()), P(v_pool.data_ptr()),
            P(dt.data_ptr()), P(dl.data_ptr()), B, H, n_new, D, total, tables.shape[1], 16,
            api.ATTN_BF16, P(torch.cuda.current_stream().cuda_stream))
    fn = api.lib.attn_paged_append

    def call():
        if fn(*args) != 0:
            raise RuntimeError("attn_paged_append failed")

    ms, wall = time_launches(torch, call, warmup, steps)
    moved = 2.0 * 2 * B * H * n_new * D * 2  # K and V: read once, written once
    gbs = moved / (ms * 1e-3) / 1e9
    log(f"[bench] append {spec.name}: {ms * 1e3:.1f} us/launch, {gbs:.0f} GB/s "
        f"({gbs / PEAK_HBM_GBS:.1%})")
    del k_new, v_new, k_pool, v_pool, dt, dl
    torch.cuda.empty_cache()
    return {
        "workload": f"kv_append_bf16_{B}seq_{H}h_{n_new}tok_d{D}",
        "ms_per_step": wall / steps,
        "value": moved / (wall / steps * 1e-3) / 1e9,
        "roofline": {
            "kernel": f"paged_append_kernel<{D}>",
            "bound": "hbm",
            "achieved": gbs,
            "peak": PEAK_HBM_GBS,
            "unit": "GB/s",
            "frac": gbs / PEAK_HBM_GBS,
            "traffic": load_traffic(key, source_digest(*KERNEL_SOURCES["append"])),
            "algorithmic_bytes_per_launch": moved,
            "launch_us_events": ms * 1e3,
        },
    }


def bench_copy(torch, warmup, steps):
    """Plain 2 GiB device copy: the calibration kernel for HBM byte counters."""
    n = 1 << 31
    src = torch.empty(n, dtype=torch.uint8, device="cuda").fill_(1)
    dst = torch.empty_like(src)
    ms, wall = time_launches(torch, lambda: dst.copy_(src), warmup, steps)
    log(f"[bench] copy 2 GiB: {ms * 1e3:.1f} us, {2 * n / (ms * 1e-3) / 1e9:.0f} GB/s (read+write)")
    return {"workload": "copy_2GiB", "bytes_read": n, "bytes_written": n,
            "ms_per_step": wall / steps, "GBps_read_plus_write": 2 * n / (ms * 1e-3) / 1e9}


def bench_probe(torch, api, warmup, steps):
    import probe
    """Read-bandwidth ceilings of the paged kernels' access patterns: whole
    blocks of a 2.5 GiB buffer read in a random order -- 4 KiB, one bf16 cache
    slab of a (block, head) at D = 128, and 2 KiB, one FP8 slab -- and in
    address order, through the probe library's probe_block_read (loads only,
    8192 waves),
    with nontemporal loads (the policy of the paged kernels) and, for the
    random 4 KiB case, the default policy too."""
    total = 5 << 29
    buf = torch.zeros(total, dtype=torch.uint8, device="cuda")
    g = torch.Generator().manual_seed(12)
    n_waves = 8192
    sink = torch.empty(n_waves * 64, dtype=torch.int32, device="cuda")
    res = {"workload": "read_probe_2.5GiB",
           "note": "bytes read / time; the ceiling the paged kernels' block reads can reach"}
    for name, bb, shuffled, nt in (("random_4KiB_nt", 4096, True, True),
                                   ("random_2KiB_nt", 2048, True, True),
                                   ("linear_4KiB_nt", 4096, False, True),
                                   ("random_4KiB_default", 4096, True, False)):
        n = total // bb
        ids = torch.randperm(n, generator=g) if shuffled else torch.arange(n)
        order = ids.to(torch.int32).cuda()
        ms, _ = time_launches(
            torch, lambda: probe.probe_block_read(buf, bb, order, n_waves, nontemporal=nt, sink=sink),
            warmup, steps)
        gbs = total / (ms * 1e-3) / 1e9
        log(f"[bench] read probe {name}: {ms * 1e3:.1f} us, {gbs:.0f} GB/s ({gbs / PEAK_HBM_GBS:.1%})")
        res[name] = {"GBps": gbs, "frac_of_peak": gbs / PEAK_HBM_GBS, "launch_us_events": ms * 1e3}
        del order
    del buf, sink
    torch.cuda.empty_cache()
    return res


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--cpu-seconds", type=float, default=15.0,
                    help="budget of the CPU oracle baseline (0 disables it)")
    ap.add_argument("--only", choices=["c1", "c2", "c3", "c4", "c5", "c4g", "cpf", "append", "c4f8", "copy",
                                       "probe"],
                    help="run one workload and print its entry only")
    args = ap.parse_args()

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU only: this library has no multi-GPU path "
              "(attention shards by head with no exchange; see the design notes). "
              "Run with --gpus 1.", file=sys.stderr)
        sys.exit(2)

    import torch
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(2)
    import attention_tiled_qk_amd as api
    from workloads import C1, C2, C3, C4, C4F8, C4G, C5, CPF

    steps, warmup = args.steps, args.warmup
    runners = {
        "c1": lambda: bench_prefill_f32(torch, api, C1, warmup, steps),
        "c2": lambda: bench_prefill(torch, api, C2, warmup, steps, "prefill_c2"),
        "c3": lambda: bench_prefill(torch, api, C3, warmup, max(steps // 2, 3), "prefill_c3"),
        "c4": lambda: bench_paged(torch, api, C4, warmup, max(steps // 2, 3), "paged_c4"),
        "c5": lambda: bench_paged(torch, api, C5, warmup, max(steps // 2, 3), "paged_c5"),
        "c4g": lambda: bench_paged(torch, api, C4G, warmup, max(steps // 2, 3), "paged_c4g"),
        "cpf": lambda: bench_paged_prefill(torch, api, CPF, warmup, max(steps // 2, 3), "prefill_cpf"),
        "append": lambda: bench_append(torch, api, CPF, warmup, max(steps // 2, 3), "append_cpf"),
        "c4f8": lambda: bench_paged_fp8(torch, api, C4F8, warmup, max(steps // 2, 3), "paged_c4f8"),
        "copy": lambda: bench_copy(torch, warmup, steps),
        "probe": lambda: bench_probe(torch, api, 3, 20),
    }
    if args.only:
        global WITH_CACHE_CONTROL
        WITH_CACHE_CONTROL = False
        print(json.dumps({"only": args.only, **runners[args.only]()}), flush=True)
        return

    main_res = runners["c2"]()
    out = {
        "metric": METRIC,
        "value": main_res["value"],
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": steps,
        "warmup": warmup,
        "ms_per_step": main_res["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "causal prefill bf16 B=8 H=16 L=1024 D=128 (1.3B-model attention shape)",
                   "B": C2.B, "H": C2.H, "L": C2.L, "D": C2.D, "causal": C2.causal,
                   "seed": C2.seed},
        "roofline": main_res["roofline"],
        "device": device_info(torch),
        "secondary": {name: runners[name]() for name in ("c1", "c3", "c4", "c5", "c4g", "cpf", "append", "c4f8",
                                                         "probe")},
    }
    if args.cpu_seconds > 0:
        log(f"[bench] cpu baseline (oracle, ~{args.cpu_seconds:.0f} s)")
        out["cpu_baseline"] = cpu_baseline(C2, args.cpu_seconds)
    else:
        out["cpu_baseline"] = None
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
