"""Benchmark of the KDA prefill hot path on one MI355X.

One step = one pass of the whole path over one synthetic batch:
    kda_state_gather -> kda_chunk_prefill -> kda_state_scatter
on the end-to-end workload: 200 sequences with lengths log-uniform in
[64, 8192] (about 335k tokens), H=32, K=V=128, bf16 q/k/v, fp32 g and beta,
and a bf16 state cache [4096,32,128,128] whose rows carry a 4096-element gap
(address span > 4 GiB); int32 gather indices with duplicates and 10% false
flags, unique scatter targets.  Inputs are resident in HBM before timing.

Prints ONE JSON line: whole-step tokens/s, per-stage kernel times from HIP
events on the launch stream, the chunk kernel's HBM roofline fraction, copy
bandwidths, the other configurations of the metric under "configs" (state
copy with int32 and int64 indices, varlen and long prefill, each with its own
roofline), and the oracle timed on the host's cores on bounded samples (all
threads and one thread; scalar gather/scatter at one and all threads).
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "KDA prefill tokens/s (H=32,K=V=128) + state gather/scatter GB/s, 1 GPU"
HBM_PEAK_GBPS = 8000.0
MFMA_BF16_PEAK_TFLOPS = 2500.0  # dense bf16 matrix peak of MI355X
H, K, V = 32, 128, 128
NUM_ROWS = 4096
MAX_SELECTED = 256
CHUNK_SRC = os.path.join(ROOT, "kda_recurrent_state_amd", "csrc", "chunk_prefill.hip")
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "chunk_prefill_e2e_traffic.json")
SOURCES = [os.path.join(ROOT, "kda_recurrent_state_amd", "csrc", f)
           for f in ("chunk_prefill.hip", "state_copy.hip", "decode.hip", "int8_ckpt.hip", "kda_api.cpp")]


def chunk_bytes_per_launch(T: int, N: int) -> int:
    """Algorithmic HBM bytes of one kda_chunk_prefill launch on this workload.

    Per token-head: q, k, v, o at 2 B x 128 (bf16) = 1024 B, g at 4 B x 128 =
    512 B, beta 4 B -> 1540 B.  Per (sequence, head): the bf16 initial and
    final states, 2 x 128 x 128 x 2 B = 64 KiB.  Plus cu_seqlens.
    """
    per_tok = 2 * K + 2 * K + 2 * V + 4 * K + 4 + 2 * V
    return T * H * per_tok + N * H * 2 * (K * V * 2) + 4 * (N + 1)


def chunk_flops_per_token_head(C: int = 64, Kd: int = K, Vd: int = V) -> float:
    """Algorithmic flops per token-head of the chunk form (multiply-add = 2),
    counting only the triangles the method needs, for full chunks of C tokens
    (stage order of page "PR #33465 完整报告", section "关键源码片段"):
    A_kk (strict lower) and A_qk (lower) over K, the unit lower-triangular
    inverse (C^3/3), W and U (lower-triangular times C x K and C x V),
    V_new = U - W S, the state update Kbar^T V_new plus the decay, and
    O = Qg S + A_qk V_new.  About 1.41e5 at C = 64, K = V = 128."""
    lo, slo = C * (C + 1) / 2, C * (C - 1) / 2
    per_chunk = (2 * slo * Kd + 2 * lo * Kd + C ** 3 / 3 + 2 * lo * Kd + 2 * lo * Vd + 2 * C * Kd * Vd
                 + 2 * Kd * C * Vd + Kd * Vd + 2 * C * Kd * Vd + 2 * lo * Vd)
    return per_chunk / C


def pct(xs):
    """p10 / p50 / p90 of a list of times."""
    a = np.asarray(xs, dtype=np.float64)
    return {"p10": float(np.percentile(a, 10)), "p50": float(np.percentile(a, 50)), "p90": float(np.percentile(a, 90))}


def sha256_file(path: str) -> str:
    with open(path, "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()


def stored_traffic(T: int, N: int):
    """HBM traffic per launch from committed rocprofv3 counter runs, if they
    were taken on the current chunk kernel source and this workload."""
    if not os.path.exists(TRAFFIC_FILE):
        return None
    with open(TRAFFIC_FILE) as f:
        rec = json.load(f)
    if rec.get("chunk_prefill_hip_sha256") != sha256_file(CHUNK_SRC):
        return None
    if rec.get("T") != T or rec.get("N") != N:
        return None
    return int(rec["hbm_bytes_per_launch"])


def stored_kernel_traffic(json_name: str, kernel_prefix: str):
    """HBM bytes per launch (read + write) of one kernel from a committed
    rocprofv3 counter summary, if it was taken on the current source."""
    path = os.path.join(ROOT, "profiles", json_name)
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f)
    if rec.get("source_sha256") != sha256_file(os.path.join(ROOT, rec["source"])):
        return None
    hits = [v for k, v in rec["kernels"].items() if k.startswith(kernel_prefix)]
    if len(hits) != 1:
        return None
    return int(hits[0]["hbm_read_bytes_per_launch"] + hits[0]["hbm_write_bytes_per_launch"])


def build_workload(seed: int, device):
    import torch
    import kda_workloads as wl

    lengths = wl.lengths_e2e(seed)
    inp = wl.device_prefill_inputs(lengths, H, K, V, dtype="bf16", seed=seed, device=device, initial=False)
    back, off, shape, strides = wl.device_cache(NUM_ROWS, H, V, K, dtype="bf16", gap=wl.GAP, offset=0,
                                                seed=seed + 1, device=device)
    cache = torch.as_strided(back.view(torch.bfloat16), shape, strides, off)
    N = len(lengths)
    gidx, flags, sidx = wl.e2e_copy_indices(seed, N, NUM_ROWS)
    packed_in = torch.empty((MAX_SELECTED, H, V, K), dtype=torch.bfloat16, device=device)
    packed_out = torch.empty((MAX_SELECTED, H, V, K), dtype=torch.bfloat16, device=device)
    out = torch.empty_like(inp["v"])
    import kda_recurrent_state_amd as kda
    ws_bytes = max(1, kda.kda_chunk_prefill_workspace_size(inp["T"], N, H, K, V))
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device=device)
    return dict(inp=inp, cache=cache, backing=back, N=N, lengths=lengths,
                gidx=torch.from_numpy(gidx).to(device), flags=torch.from_numpy(flags).to(device),
                sidx=torch.from_numpy(sidx).to(device), gidx_np=gidx, flags_np=flags, sidx_np=sidx,
                packed_in=packed_in, packed_out=packed_out, out=out, ws=ws)


def cpu_baseline(seed: int, budget_s: float, single_budget_s: float = 8.0, copy_budget_s: float = 6.0):
    """The oracle, as it stands, on bounded samples of the same workloads.

    * recurrence, all threads (``value``): the fp64 token recurrence with
      OpenMP over (sequence, head) chains on the first sequences of the e2e
      batch, sized to ``budget_s`` after a calibration run;
    * recurrence, one thread: the same on fewer sequences;
    * scalar gather / scatter GB/s at one thread and at all threads: the
      oracle's element-by-element copy on the copy workload's row format
      (fp32 rows [32,128,128] = 2 MiB, 4096-element gaps), the selection
      split into contiguous parts, one per thread.
    """
    import concurrent.futures as cf

    import kda_workloads as wl
    import oracle

    oracle.build(force=False)
    threads = oracle.default_threads()
    lengths = wl.lengths_e2e(seed)

    def run(lens, nthreads):
        inp = wl.host_prefill_inputs(lens, H, K, V, dtype="bf16", seed=seed + 11, initial=True, init_dtype="bf16")
        t0 = time.perf_counter()
        oracle.kda_recurrence(inp["q"], inp["k"], inp["v"], inp["g"], inp["beta"], inp["cu_seqlens"],
                              inp["initial"], threads=nthreads)
        return time.perf_counter() - t0

    def sample_for(rate, budget):
        target_tokens = max(64, int(rate * budget))
        sample, tot = [], 0
        for L in lengths:
            if tot + L > target_tokens and sample:
                break
            sample.append(L)
            tot += L
        return sample

    # calibrate on one short sequence, then size the samples to the budgets
    probe = [min(lengths)]
    rate1 = sum(probe) / max(run(probe, 1), 1e-6)   # one thread: all heads of one sequence
    sample = sample_for(rate1 * min(threads, H), budget_s)
    dt = run(sample, threads)
    sample1 = sample_for(rate1, single_budget_s)
    dt1 = run(sample1, 1)

    # scalar copies: 64 rows of the copy workload's format, 32 selected
    rows, S = 64, 32
    backing, off, shape, strides = wl.host_cache(rows, H, V, K, dtype="f32", gap=wl.GAP, offset=1024, seed=seed)
    gidx = wl.copy_indices(seed, S, rows, 2, "int32")
    flags = wl.copy_flags(seed, S, 3)
    sidx = wl.copy_indices(seed + 1, S, rows, 2, "int32", unique=True)
    payload = H * V * K * 4
    g_bytes = (int(((gidx >= 0) & (gidx < rows) & (flags != 0)).sum()) + S) * payload
    s_bytes = 2 * int(((sidx >= 0) & (sidx < rows)).sum()) * payload
    packed = oracle.state_gather(backing, off, shape, strides, gidx, flags)

    def copy_rate(nthreads, what):
        parts = [p for p in np.array_split(np.arange(S), nthreads) if len(p)]
        def one(p):
            if what == "gather":
                oracle.state_gather(backing, off, shape, strides, gidx[p], flags[p])
            else:
                oracle.state_scatter(backing, off, shape, strides, sidx[p], packed[p], in_place=True)
        reps, t_used = 0, 0.0
        with cf.ThreadPoolExecutor(max_workers=len(parts)) as ex:
            while reps == 0 or t_used < copy_budget_s / 4:
                t0 = time.perf_counter()
                list(ex.map(one, parts))
                t_used += time.perf_counter() - t0
                reps += 1
        return reps * (g_bytes if what == "gather" else s_bytes) / t_used / 1e9

    copy = {"gather_GBps_1_thread": copy_rate(1, "gather"), "gather_GBps_all_threads": copy_rate(threads, "gather"),
            "scatter_GBps_1_thread": copy_rate(1, "scatter"),
            "scatter_GBps_all_threads": copy_rate(threads, "scatter"),
            "sample": "fp32 cache [%d,32,128,128] with row stride payload+4096, %d rows selected (2 invalid "
                      "indices, 3 false flags in gather; unique targets in scatter), element-by-element raw-bit "
                      "copy; algorithmic bytes as for the GPU copies" % (rows, S)}
    return {"value": sum(sample) / dt, "unit": "tokens/s", "cores": threads, "kind": "oracle",
            "sample": "first %d of the %d e2e sequences (%d tokens, all %d heads, K=V=128), fp64 token "
                      "recurrence, %d threads, %.1f s" % (len(sample), len(lengths), sum(sample), H, threads, dt),
            "single_thread": {"value": sum(sample1) / dt1, "unit": "tokens/s", "cores": 1,
                              "sample": "first %d e2e sequences (%d tokens, all %d heads), %.1f s"
                                        % (len(sample1), sum(sample1), H, dt1)},
            "copy": copy}


def calibrate_copy(device, gib: float = 1.0):
    """A plain device copy of known size, for scaling rocprofv3 byte counters."""
    import torch
    n = int(gib * (1 << 30)) // 2
    src = torch.empty(n, dtype=torch.bfloat16, device=device).fill_(1.0)
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"calibration_copy_bytes_read": n * 2, "calibration_copy_bytes_written": n * 2}))


WARMUP_MIN_S = 0.25  # every warm-up also runs until this much wall time has passed (clocks settle)


def warm_up(fn, warmup: int, min_s: float = WARMUP_MIN_S) -> int:
    """Run fn() at least ``warmup`` times and for at least ``min_s`` seconds
    (synchronising every few calls); returns the number of calls made."""
    import torch
    n, t0 = 0, time.perf_counter()
    while n < warmup or time.perf_counter() - t0 < min_s:
        fn()
        n += 1
        if n % 4 == 0:
            torch.cuda.synchronize()
    torch.cuda.synchronize()
    return n


def _timed(fn, steps, warmup):
    """Run fn() warmup + steps times; HIP events on the current stream around each call."""
    import torch
    stream = torch.cuda.current_stream()
    warm_up(fn, warmup)
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
    t0 = time.perf_counter()
    for a, b in evs:
        a.record(stream)
        fn()
        b.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    return wall * 1e3 / steps, float(np.mean([a.elapsed_time(b) for a, b in evs]))


def measure_copy(dev, seed: int, steps: int, warmup: int):
    """State copy workload: fp32 cache [1024,32,128,128] with row stride
    payload+4096 at a storage offset, S=256 gathered (with replacement) and
    scattered (unique targets), 13 invalid indices, 26 false flags; int32 and
    int64 indices.  GB/s = algorithmic bytes / average event time of a call."""
    import torch
    import kda_recurrent_state_amd as kda
    import kda_workloads as wl
    nrows, S = 1024, 256
    back, off, shape, strides = wl.device_cache(nrows, H, V, K, dtype="f32", gap=wl.GAP, offset=1024,
                                                seed=seed, device=dev)
    cache = torch.as_strided(back.view(torch.float32), shape, strides, off)
    packed = torch.empty((S, H, V, K), dtype=torch.float32, device=dev)
    payload = H * V * K * 4
    res = {}
    for it in ("int32", "int64"):
        gidx = wl.copy_indices(seed, S, nrows, 13, it, unique=False, huge=True)
        flags = wl.copy_flags(seed, S, 26)
        sidx = wl.copy_indices(seed + 1, S, nrows, 13, it, unique=True, huge=True)
        gi, fl, si = (torch.from_numpy(x).to(dev) for x in (gidx, flags, sidx))
        n_read = int(((gidx >= 0) & (gidx < nrows) & (flags != 0)).sum())
        n_valid = int(((sidx >= 0) & (sidx < nrows)).sum())
        g_bytes, s_bytes = (n_read + S) * payload, 2 * n_valid * payload
        _, g_ms = _timed(lambda: kda.kda_state_gather(cache, gi, fl, packed), steps, warmup)
        _, s_ms = _timed(lambda: kda.kda_state_scatter(cache, si, packed), steps, warmup)
        g_gbps, s_gbps = g_bytes / (g_ms * 1e-3) / 1e9, s_bytes / (s_ms * 1e-3) / 1e9
        res[it] = {"gather_GBps": g_gbps, "scatter_GBps": s_gbps, "gather_ms": g_ms, "scatter_ms": s_ms,
                   "gather_bytes": g_bytes, "scatter_bytes": s_bytes,
                   "gather_frac_hbm": g_gbps / HBM_PEAK_GBPS, "scatter_frac_hbm": s_gbps / HBM_PEAK_GBPS}
    del back, cache, packed
    torch.cuda.synchronize()
    worst = min(min(r["gather_GBps"], r["scatter_GBps"]) for r in res.values())
    avg = float(np.mean([x for r in res.values() for x in (r["gather_GBps"], r["scatter_GBps"])]))
    return {"value": avg, "unit": "GB/s", "dtype": "f32",
            "workload": "state copy: fp32 cache [1024,32,128,128], row stride payload+4096, S=256, 13 invalid "
                        "indices, 26 false flags, int32 and int64 indices",
            "roofline": {"bound": "hbm", "achieved": avg, "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                         "frac": avg / HBM_PEAK_GBPS, "traffic": None, "kernel": "state_copy_kernel",
                         "worst_call_frac": worst / HBM_PEAK_GBPS},
            "per_index_type": res, "steps": steps, "warmup": warmup}


def measure_chunk(dev, seed: int, steps: int, warmup: int, which: str):
    """Chunk prefill on the varlen workload (16 sequences of U[512,4096]
    tokens, fp32 initial and final states) or the long one (one 65536-token
    sequence; initial state gathered from a bf16 cache row, final state
    scattered back as bf16).  The roofline is that of the kda_chunk_prefill
    call: its algorithmic bytes / its average event time (for the long
    sequence the call is the segment-parallel chain of kernels)."""
    import torch
    import kda_recurrent_state_amd as kda
    import kda_workloads as wl
    stream = torch.cuda.current_stream()
    if which == "varlen":
        lengths = wl.lengths_varlen(seed)
        inp = wl.device_prefill_inputs(lengths, H, K, V, dtype="bf16", seed=seed, device=dev, init_dtype="f32")
        state_bytes = 4
        desc = "varlen chunk prefill: 16 sequences, lengths U[512,4096], H=32, K=V=128, fp32 initial/final states"
    else:
        lengths = wl.lengths_long()
        inp = wl.device_prefill_inputs(lengths, H, K, V, dtype="bf16", seed=seed, device=dev, initial=False)
        state_bytes = 2
        desc = ("long prefill: one 65536-token sequence, H=32, K=V=128, state gathered from / scattered to "
                "bf16 cache rows [4,32,128,128] (row gap 4096)")
    T, N = inp["T"], inp["N"]
    out = torch.empty_like(inp["v"])
    fin = torch.empty((N, H, V, K), dtype=torch.float32 if which == "varlen" else torch.bfloat16, device=dev)
    ws = torch.empty(max(1, kda.kda_chunk_prefill_workspace_size(T, N, H, K, V)), dtype=torch.uint8, device=dev)
    if which == "long":
        back, off, shape, strides = wl.device_cache(4, H, V, K, dtype="bf16", gap=wl.GAP, offset=0,
                                                    seed=seed + 1, device=dev)
        cache = torch.as_strided(back.view(torch.bfloat16), shape, strides, off)
        gi = torch.tensor([1], dtype=torch.int32, device=dev)
        si = torch.tensor([3], dtype=torch.int32, device=dev)
        fl = torch.ones(1, dtype=torch.uint8, device=dev)
        init = torch.empty((1, H, V, K), dtype=torch.bfloat16, device=dev)
    else:
        init = inp["initial"]

    def step(ev=None):
        if which == "long":
            kda.kda_state_gather(cache, gi, fl, init)
        if ev is not None:
            ev[0].record(stream)
        kda.kda_chunk_prefill(inp["q"], inp["k"], inp["v"], inp["g"], inp["beta"], inp["cu_seqlens"],
                              initial_state=init, out=out, final_state=fin, workspace=ws)
        if ev is not None:
            ev[1].record(stream)
        if which == "long":
            kda.kda_state_scatter(cache, si, fin)

    warm_up(step, warmup)
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(steps)]
    t0 = time.perf_counter()
    for i in range(steps):
        step(evs[i])
    torch.cuda.synchronize()
    ms_wall = (time.perf_counter() - t0) * 1e3 / steps
    c_ms = [e[0].elapsed_time(e[1]) for e in evs]
    c_avg = float(np.mean(c_ms))
    nbytes = T * H * (2 * K + 2 * K + 2 * V + 4 * K + 4 + 2 * V) + N * H * 2 * K * V * state_bytes + 4 * (N + 1)
    achieved = nbytes / (c_avg * 1e-3) / 1e9
    return {"value": T / (c_avg * 1e-3), "unit": "tokens/s", "dtype": "bf16", "workload": desc,
            "tokens": T, "sequences": N, "seed": seed, "ms_per_step": ms_wall, "chunk_prefill_ms": c_avg,
            "chunk_prefill_percentiles_ms": pct(c_ms),
            "roofline": {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                         "frac": achieved / HBM_PEAK_GBPS, "traffic": None, "kernel": "kda_chunk_prefill",
                         "algorithmic_bytes_per_launch": nbytes, "avg_launch_ms": c_avg},
            "steps": steps, "warmup": warmup}


def bench_other(args, dev):
    """Secondary workloads (their own line, not the headline): copy, varlen,
    long, int8, decode."""
    import torch
    import kda_recurrent_state_amd as kda
    import kda_workloads as wl
    base = {"metric": METRIC, "unit": "tokens/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
            "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16", "data": "synthetic"}
    if args.workload == "copy":
        m = measure_copy(dev, args.seed, args.steps, args.warmup)
        base.update({"metric": "state gather/scatter GB/s, 1 GPU", "unit": "GB/s", "value": m["value"],
                     "dtype": "f32", "ms_per_step": None,
                     "config": {"workload": m["workload"], "seq_len": None, "seed": args.seed},
                     "roofline": m["roofline"], "per_index_type": m["per_index_type"]})
        return base
    if args.workload in ("varlen", "long"):
        m = measure_chunk(dev, args.seed, args.steps, args.warmup, args.workload)
        base.update({"value": m["value"], "ms_per_step": m["ms_per_step"],
                     "config": {"workload": m["workload"], "tokens": m["tokens"], "global_batch": m["sequences"],
                                "seq_len": m["tokens"], "seed": args.seed},
                     "roofline": m["roofline"], "chunk_prefill_percentiles_ms": m["chunk_prefill_percentiles_ms"]})
        return base
    if args.workload == "int8":
        slots, S = 1024, 256
        qd = torch.zeros((slots, H, V, K), dtype=torch.int8, device=dev)
        sc = torch.zeros((slots, H, 1, K), dtype=torch.float32, device=dev)
        gen = torch.Generator(device=dev)
        gen.manual_seed(args.seed)
        xs = torch.randn((S, H, V, K), generator=gen, device=dev) * 0.1
        back = torch.empty_like(xs)
        idx = torch.from_numpy(wl.rng(args.seed + 2).permutation(slots)[:S].astype(np.int32)).to(dev)
        _, q_ms = _timed(lambda: kda.kda_ckpt_quantize_scatter(qd, sc, idx, xs), args.steps, args.warmup)
        _, d_ms = _timed(lambda: kda.kda_ckpt_dequantize_gather(qd, sc, idx, packed=back), args.steps, args.warmup)
        n = S * H * V * K
        q_bytes = n * 4 + n + S * H * K * 4 + 4 * S
        d_bytes = n + S * H * K * 4 + n * 4 + 4 * S
        q_gbps, d_gbps = q_bytes / (q_ms * 1e-3) / 1e9, d_bytes / (d_ms * 1e-3) / 1e9
        avg = (q_gbps + d_gbps) / 2
        base.update({"metric": "INT8 checkpoint store/load GB/s, 1 GPU", "unit": "GB/s", "value": avg, "dtype": "f32",
                     "ms_per_step": q_ms + d_ms,
                     "config": {"workload": "INT8 checkpoint codec: 256 fp32 states [32,128,128] quantised into "
                                            "a 1024-slot int8 store and dequantised back to fp32", "seq_len": None,
                                "seed": args.seed},
                     "roofline": {"bound": "hbm", "achieved": avg, "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                                  "frac": avg / HBM_PEAK_GBPS, "traffic": None,
                                  "kernel": "quantize_scatter_kernel + dequantize_gather_kernel"},
                     "per_kernel": {"quantize_GBps": q_gbps, "quantize_ms": q_ms, "quantize_bytes": q_bytes,
                                    "quantize_traffic": stored_kernel_traffic("int8_codec_traffic.json",
                                                                              "quantize_scatter_kernel"),
                                    "dequantize_GBps": d_gbps, "dequantize_ms": d_ms, "dequantize_bytes": d_bytes,
                                    "dequantize_traffic": stored_kernel_traffic("int8_codec_traffic.json",
                                                                                "dequantize_gather_kernel")}})
        return base
    if args.workload == "decode":
        nseq, nrows = 512, NUM_ROWS
        back, off, shape, strides = wl.device_cache(nrows, H, V, K, dtype="bf16", gap=wl.GAP, offset=0,
                                                    seed=args.seed + 1, device=dev)
        cache = torch.as_strided(back.view(torch.bfloat16), shape, strides, off)
        inp = wl.device_prefill_inputs([1] * nseq, H, K, V, dtype="bf16", seed=args.seed, device=dev, initial=False)
        idx = torch.from_numpy(wl.rng(args.seed + 2).permutation(nrows)[:nseq].astype(np.int32)).to(dev)
        out = torch.empty_like(inp["v"])
        fn = lambda: kda.kda_recurrent_decode(cache, idx, inp["q"], inp["k"], inp["v"], inp["g"],  # noqa: E731
                                              inp["beta"], out=out)
        nbytes = nseq * H * (2 * K * V * 2 + 2 * K + 2 * K + 2 * V + 4 * K + 4 + 2 * V) + 4 * nseq
        ms_wall, ms_ev = _timed(fn, args.steps, args.warmup)
        base.update({"metric": "KDA recurrent decode tokens/s (H=32,K=V=128), 1 GPU", "value": nseq / (ms_wall * 1e-3),
                     "ms_per_step": ms_wall,
                     "config": {"workload": "recurrent decode: 512 sequences x 1 token, H=32, K=V=128, bf16 q/k/v, "
                                            "fp32 g/beta, states updated in place in a bf16 cache [4096,32,128,128] "
                                            "with a 4096-element row gap", "global_batch": nseq, "seq_len": 1,
                                "seed": args.seed},
                     "roofline": {"bound": "hbm", "achieved": nbytes / (ms_ev * 1e-3) / 1e9, "peak": HBM_PEAK_GBPS,
                                  "unit": "GB/s", "frac": nbytes / (ms_ev * 1e-3) / 1e9 / HBM_PEAK_GBPS,
                                  "traffic": stored_kernel_traffic("decode_traffic.json", "recurrent_decode_kernel"),
                                  "kernel": "recurrent_decode_kernel",
                                  "algorithmic_bytes_per_launch": nbytes, "avg_launch_ms": ms_ev}})
        return base
    raise ValueError(args.workload)


def bench_ckpt(args, dev, interval: int = 1024):
    """The e2e step with prefill checkpoints: every 1024 tokens of each
    sequence the state is written (bf16) and then scattered into free cache
    rows, next to the final states."""
    import torch
    import kda_recurrent_state_amd as kda
    w = build_workload(args.seed, dev)
    inp, N = w["inp"], w["N"]
    T = int(inp["T"])
    offs = kda.checkpoint_offsets(w["lengths"], interval)
    n_ck = offs[-1]
    used = set(int(x) for x in w["sidx_np"].tolist())
    free = [r for r in range(NUM_ROWS) if r not in used][:n_ck]
    assert len(free) == n_ck
    ck_idx = torch.tensor(free, dtype=torch.int32, device=dev)
    ck_cu = torch.tensor(offs, dtype=torch.int32, device=dev)
    ck = torch.empty((max(n_ck, 1), H, V, K), dtype=torch.bfloat16, device=dev)
    pin, pout = w["packed_in"][:N], w["packed_out"][:N]
    stream = torch.cuda.current_stream()

    def step(ev=None):
        if ev is not None:
            ev[0].record(stream)
        kda.kda_state_gather(w["cache"], w["gidx"], w["flags"], pin)
        if ev is not None:
            ev[1].record(stream)
        kda.kda_chunk_prefill(inp["q"], inp["k"], inp["v"], inp["g"], inp["beta"], inp["cu_seqlens"],
                              initial_state=pin, out=w["out"], final_state=pout, workspace=w["ws"],
                              ckpt_interval=interval, ckpt_cu=ck_cu, ckpt_states=ck[:n_ck])
        if ev is not None:
            ev[2].record(stream)
        kda.kda_state_scatter(w["cache"], w["sidx"], pout)
        kda.kda_state_scatter(w["cache"], ck_idx, ck[:n_ck])
        if ev is not None:
            ev[3].record(stream)

    warm_up(step, args.warmup)
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(args.steps)]
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(evs[i])
    torch.cuda.synchronize()
    ms = (time.perf_counter() - t0) * 1e3 / args.steps
    c_avg = float(np.mean([e[1].elapsed_time(e[2]) for e in evs]))
    s_avg = float(np.mean([e[2].elapsed_time(e[3]) for e in evs]))
    ck_bytes = n_ck * H * V * K * 2
    nbytes = chunk_bytes_per_launch(T, N) + ck_bytes
    return {"metric": METRIC, "value": T / (ms * 1e-3), "unit": "tokens/s", "n_gpus": 1, "steps": args.steps,
            "warmup": args.warmup, "ms_per_step": ms, "higher_is_better": True, "scaling": "weak",
            "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
            "config": {"workload": "e2e prefill step with checkpoints: the e2e step plus the state after every "
                                   "%d tokens of each sequence (%d checkpoints, bf16) scattered into free cache rows"
                                   % (interval, n_ck),
                       "global_batch": N, "seq_len": T, "tokens": T, "checkpoints": n_ck, "seed": args.seed},
            "roofline": {"bound": "hbm", "achieved": nbytes / (c_avg * 1e-3) / 1e9, "peak": HBM_PEAK_GBPS,
                         "unit": "GB/s", "frac": nbytes / (c_avg * 1e-3) / 1e9 / HBM_PEAK_GBPS, "traffic": None,
                         "kernel": "kda_chunk_prefill (with checkpoints)", "algorithmic_bytes_per_launch": nbytes,
                         "avg_launch_ms": c_avg},
            "stages_ms": {"chunk_prefill": c_avg, "scatter_final_and_checkpoints": s_avg},
            "checkpoint_bytes": ck_bytes}


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--seed", type=int, default=41)
    ap.add_argument("--cpu-budget", type=float, default=12.0,
                    help="seconds of multi-threaded oracle work for the CPU baseline")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--sub-steps", type=int, default=20,
                    help="timed steps of each other configuration carried in the headline line (copy, varlen, long)")
    ap.add_argument("--no-sub-configs", action="store_true",
                    help="leave the copy / varlen / long configurations out of the headline line")
    ap.add_argument("--calibrate-copy", action="store_true", help="run only a plain 1 GiB device copy")
    ap.add_argument("--workload", default="e2e", choices=["e2e", "varlen", "long", "copy", "ckpt", "decode", "int8"],
                    help="e2e (default, the headline step); varlen / long: the chunk prefill on 16 sequences of "
                         "512-4096 tokens / one 65536-token sequence (state gathered from and scattered to a bf16 "
                         "cache for long); copy: state gather/scatter on an fp32 [1024,32,128,128] cache; ckpt: "
                         "the e2e step plus checkpoints every 1024 tokens scattered into cache rows; decode: one recurrent "
                         "decode step of 512 sequences against a bf16 [4096,32,128,128] cache; int8: the INT8 checkpoint "
                         "codec on 256 fp32 states")
    args = ap.parse_args()

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py: this path runs on one GPU; --gpus %d is not supported (sequences and heads shard "
              "across GPUs with no exchange)" % args.gpus, file=sys.stderr)
        sys.exit(2)

    import torch
    import kda_recurrent_state_amd as kda
    from kda_recurrent_state_amd import _lib
    if not os.path.exists(_lib.LIB_PATH):
        import __graft_entry__
        __graft_entry__.build()
    kda.load_library()
    dev = torch.device("cuda:0")
    if args.calibrate_copy:
        calibrate_copy(dev)
        return

    if args.workload == "ckpt":
        print(json.dumps(bench_ckpt(args, dev)))
        return
    if args.workload != "e2e":
        print(json.dumps(bench_other(args, dev)))
        return

    w = build_workload(args.seed, dev)
    inp, N = w["inp"], w["N"]
    T = int(inp["T"])
    S = N
    pin, pout = w["packed_in"][:S], w["packed_out"][:S]
    stream = torch.cuda.current_stream()

    def step(ev=None):
        if ev is not None:
            ev[0].record(stream)
        kda.kda_state_gather(w["cache"], w["gidx"], w["flags"], pin)
        if ev is not None:
            ev[1].record(stream)
        kda.kda_chunk_prefill(inp["q"], inp["k"], inp["v"], inp["g"], inp["beta"], inp["cu_seqlens"],
                              initial_state=pin, out=w["out"], final_state=pout, workspace=w["ws"])
        if ev is not None:
            ev[2].record(stream)
        kda.kda_state_scatter(w["cache"], w["sidx"], pout)
        if ev is not None:
            ev[3].record(stream)

    warm_up(step, args.warmup)
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(evs[i])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    g_ms = [e[0].elapsed_time(e[1]) for e in evs]
    c_ms = [e[1].elapsed_time(e[2]) for e in evs]
    s_ms = [e[2].elapsed_time(e[3]) for e in evs]
    ms_per_step = wall * 1e3 / args.steps
    tokens_per_s = T / (ms_per_step * 1e-3)

    payload = H * V * K * 2
    flags_np, gidx_np, sidx_np = w["flags_np"], w["gidx_np"], w["sidx_np"]
    n_read = int(((gidx_np >= 0) & (gidx_np < NUM_ROWS) & (flags_np != 0)).sum())
    n_valid_s = int(((sidx_np >= 0) & (sidx_np < NUM_ROWS)).sum())
    gather_bytes = (n_read + S) * payload
    scatter_bytes = 2 * n_valid_s * payload
    chunk_bytes = chunk_bytes_per_launch(T, N)
    c_avg = float(np.mean(c_ms))
    achieved = chunk_bytes / (c_avg * 1e-3) / 1e9
    traffic = stored_traffic(T, N)
    g_avg, s_avg = float(np.mean(g_ms)), float(np.mean(s_ms))
    fl_tok = chunk_flops_per_token_head()
    flops = fl_tok * T * H
    t_hbm, t_mfma = chunk_bytes / (HBM_PEAK_GBPS * 1e9), flops / (MFMA_BF16_PEAK_TFLOPS * 1e12)
    t_roof = max(t_hbm, t_mfma)

    # the other configurations of the metric, each with its own roofline:
    # copy (fp32 rows, int32 and int64 indices), varlen and long prefill
    subs = None
    if not args.no_sub_configs:
        sw = min(3, args.warmup)
        subs = {"copy": measure_copy(dev, args.seed, args.sub_steps, sw),
                "varlen": measure_chunk(dev, args.seed, args.sub_steps, sw, "varlen"),
                "long": measure_chunk(dev, args.seed, args.sub_steps, sw, "long")}

    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(args.seed, args.cpu_budget)

    line = {
        "metric": METRIC,
        "value": tokens_per_s,
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "e2e prefill step: gather -> chunk KDA -> scatter; %d sequences, lengths "
                               "log-uniform [64,8192], H=32, K=V=128, bf16 q/k/v, fp32 g/beta, bf16 cache "
                               "[4096,32,128,128] with 4096-element row gap" % N,
                   "global_batch": N, "seq_len": T, "tokens": T, "parallelism": "none (1 GPU)",
                   "seed": args.seed},
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                     "frac": achieved / HBM_PEAK_GBPS, "traffic": traffic,
                     "kernel": "kda_chunk_prefill", "algorithmic_bytes_per_launch": chunk_bytes,
                     "avg_launch_ms": c_avg},
        "cpu_baseline": cpu,
        "configs": subs,
        "stages_ms": {"gather": g_avg, "chunk_prefill": c_avg, "scatter": s_avg},
        "copy_GBps": {"gather": gather_bytes / (g_avg * 1e-3) / 1e9,
                      "scatter": scatter_bytes / (s_avg * 1e-3) / 1e9,
                      "gather_frac_hbm": gather_bytes / (g_avg * 1e-3) / 1e9 / HBM_PEAK_GBPS,
                      "scatter_frac_hbm": scatter_bytes / (s_avg * 1e-3) / 1e9 / HBM_PEAK_GBPS,
                      "gather_bytes": gather_bytes, "scatter_bytes": scatter_bytes},
        "chunk_tokens_per_s": T / (c_avg * 1e-3),
        "mfma": {"flop_convention": "chunk form, triangles only, C=64 (%.0f flop per token-head)" % fl_tok,
                 "algorithmic_tflops": flops / (c_avg * 1e-3) / 1e12,
                 "frac_bf16_dense_peak": flops / (c_avg * 1e-3) / 1e12 / MFMA_BF16_PEAK_TFLOPS},
        "attainable": {"t_roof_ms": t_roof * 1e3, "t_meas_ms": c_avg,
                       "frac": t_roof / (c_avg * 1e-3), "bound": "hbm" if t_hbm >= t_mfma else "mfma"},
        "samples_ms": {k: [round(x, 4) for x in v] for k, v in (("gather", g_ms), ("chunk_prefill", c_ms),
                                                                ("scatter", s_ms))},
        "percentiles_ms": {"gather": pct(g_ms), "chunk_prefill": pct(c_ms), "scatter": pct(s_ms)},
        "sources_sha256": {os.path.basename(f): sha256_file(f)[:16] for f in SOURCES},
        "gpu": torch.cuda.get_device_name(0),
    }
    print(json.dumps(line))


if __name__ == "__main__":
    main()
