#!/usr/bin/env python3
"""Benchmark of the GQA hot path on one MI355X.

Default workload (one JSON line on stdout):
  decode, Llama-3-8B-shaped layer: B=32, Hq=32, Hkv=8, d=128, 8192 cached
  tokens per sequence, bf16 cache, fp32 accumulation.  A step is one full
  decode call (split kernel + log-sum-exp merge) over the whole batch.
  value = KV-cache bytes read per step / step time (GB/s).
  The same run also times causal prefill (B=2, Hq=32, Hkv=8, N=4096, d=128)
  and its backward (dq, dk, dv) and reports their TFLOP/s in the "prefill"
  and "prefill_backward" objects, with the vendor's bf16 GEMM timed beside
  the prefill as the board's attainable dense-product rate
  ("prefill.matmul_reference") and torch's own flash attention, forward and
  backward, on the same prefill inputs ("vendor_attention_reference" in
  both objects).

Inputs are seeded synthetic N(0,1) values; K/V are resident in HBM before the
timed region and rotated over several copies so the 256 MB MALL cannot serve
repeated steps.  Kernel durations come from HIP events on the stream the
kernels run on (torch's current stream, which the binding launches on).

  python bench.py [--steps K] [--warmup W] [--workload llama3-8b|wide-group|mqa-128k|group-32|group-71|
                  paged-llama3-8b|paged-wide-group|fp8-llama3-8b|fp8-wide-group|fp8-mqa-128k|
                  mla-decode]
                  [--page-size P] [--no-cpu-baseline] [--expanded]
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import numpy as np  # noqa: E402

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, GB/s
BF16_MFMA_PEAK_TFLOPS = 2500.0  # MI355X dense bf16 matrix cores, TFLOP/s
MALL_BYTES = 256 * 2 ** 20
METRIC = "GQA decode KV-read GB/s (% of HBM peak) + causal prefill TFLOP/s (% MFMA)"
COUNTERS = os.path.join(ROOT, "profiles", "counters.json")
CSRC = os.path.join(ROOT, "grouped_query_attention_gqa_amd", "csrc")
# the sources each measured kernel is built from (a counter entry is used only
# while their digest is unchanged)
KERNEL_SOURCES = {
    "decode_split": ("decode.hip", "api.hip", "gqa_device.hpp", "gqa_launch.hpp"),
    "decode_wide": ("decode_wide.hip", "api.hip", "gqa_device.hpp", "gqa_launch.hpp"),
    "prefill_causal": ("prefill.hip", "prefill_tiles.hpp", "gqa_device.hpp", "gqa_launch.hpp"),
    "prefill_bwd_dq": ("prefill_bwd.hip", "prefill_tiles.hpp", "gqa_device.hpp", "gqa_launch.hpp"),
    "prefill_bwd_dkdv": ("prefill_bwd.hip", "prefill_tiles.hpp", "gqa_device.hpp", "gqa_launch.hpp"),
}


def kernel_source_digest(kernel: str) -> str:
    h = hashlib.sha256()
    for name in KERNEL_SOURCES[kernel]:
        with open(os.path.join(CSRC, name), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


# ---------------------------------------------------------------------------
# algorithmic work (the bytes and FLOPs the method itself must move / do)
# ---------------------------------------------------------------------------

def decode_kv_bytes(seq_lens, hkv, d, elem):
    """K and V of every attended token: 2 * sum(T_b) * Hkv * d * elem."""
    return 2 * int(np.sum(seq_lens, dtype=np.int64)) * hkv * d * elem


def decode_split_bytes(seq_lens, hq, hkv, d, elem):
    """Algorithmic bytes of the split kernel: the attended K/V plus q."""
    return decode_kv_bytes(seq_lens, hkv, d, elem) + len(seq_lens) * hq * d * elem


def decode_flops(seq_lens, hq, d):
    return 4 * hq * d * int(np.sum(seq_lens, dtype=np.int64))


def prefill_flops(b, hq, n, d):
    """Exact causal count: row i attends i+1 keys at 4*d FLOPs per key."""
    return 4 * b * hq * d * n * (n + 1) // 2


def prefill_backward_flops(b, hq, n, d):
    """Algorithmic FLOPs of the causal backward: five products of the
    forward's size (S recomputed, dP, dV, dQ, dK), 2.5x the forward."""
    return 2.5 * prefill_flops(b, hq, n, d)


def prefill_bytes(b, hq, hkv, n, d):
    """q, k, v in bf16 and the fp32 output."""
    return b * n * d * (2 * hq + 2 * 2 * hkv + 4 * hq)


# ---------------------------------------------------------------------------

def event_time_ms(fn, iters, torch, batches: int = 5, min_per_batch: int = 20):
    """Duration of fn() per call over exactly `iters` timed calls.

    The calls are split into at most `batches` runs of at least
    `min_per_batch` back-to-back calls (one run when `iters` is small), each
    bracketed by HIP events on the current stream; the median batch average
    is returned (GPU clocks move under sustained load).  Before every start
    event one untimed call is enqueued, so the GPU is already busy while the
    host records the event and enqueues the timed calls: the host's launch
    latency of the first timed call stays outside the timed region."""
    nb = max(1, min(batches, iters // min_per_batch))
    sizes = [iters // nb + (1 if i < iters % nb else 0) for i in range(nb)]
    times = []
    done = 0
    for per in sizes:
        if per == 0:
            continue
        start, stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        fn(done)   # untimed lead-in call: covers the host's enqueue of what follows
        done += 1
        start.record()
        for _ in range(per):
            fn(done)
            done += 1
        stop.record()
        torch.cuda.synchronize()
        times.append(start.elapsed_time(stop) / per)
    times.sort()
    return times[len(times) // 2]


def load_counters(kernel: str, workload: str):
    """HBM bytes per launch (FETCH_SIZE + WRITE_SIZE, calibrated) from the
    committed rocprofv3 counter runs, or None when there is no entry or the
    kernel's sources changed since the counters were taken."""
    try:
        with open(COUNTERS) as f:
            data = json.load(f)
    except (OSError, ValueError):
        return None
    entry = data.get("kernels", {}).get(f"{kernel}|{workload}")
    if not entry or entry.get("source_digest") != kernel_source_digest(kernel):
        return None
    return entry.get("traffic_bytes")


CALIBRATION_BYTES = 256 * 2 ** 20   # read and written by the --calibration-copy kernel
COUNTED_KERNELS = {   # kernel-name substring -> sources key
    "decode_split_bf16": "decode_split",
    "prefill_causal_bf16": "prefill_causal",
    "prefill_bwd_dq": "prefill_bwd_dq",
    "prefill_bwd_dkdv": "prefill_bwd_dkdv",
    "decode_wide_bf16": "decode_wide",
}


def matmul_reference(torch, iters: int, n: int = 8192) -> dict:
    """The vendor library's bf16 GEMM on the same GPU in the same run: one
    n x n x n torch.matmul (hipBLASLt) on contiguous operands, timed like the
    prefill.  It is the attainable matrix-core rate of a plain dense product
    on this board, where sustained MFMA load lowers the shader clock below
    the 2.4 GHz the 2.5 PFLOP/s figure assumes; context for the prefill's
    fraction, not a peak the roofline uses."""
    a = torch.randn(n, n, device="cuda", dtype=torch.bfloat16)
    b = torch.randn(n, n, device="cuda", dtype=torch.bfloat16)
    c = torch.empty(n, n, device="cuda", dtype=torch.bfloat16)

    def mm(i):
        torch.matmul(a, b, out=c)

    for i in range(5):
        mm(i)
    ms = event_time_ms(mm, iters, torch)
    tf = 2.0 * n ** 3 / (ms * 1e-3) / 1e12
    del a, b, c
    return {"kernel": f"torch.matmul bf16 {n}x{n}x{n} (hipBLASLt), contiguous operands", "value": round(tf, 2),
            "unit": "TFLOP/s", "ms_per_call": round(ms, 5),
            "pct_of_mfma_peak": round(100 * tf / BF16_MFMA_PEAK_TFLOPS, 2)}


def vendor_attention_reference(torch, q, k, v, ours, scale: float, iters: int, flops: int) -> dict:
    """torch's own causal attention on the same prefill inputs, with the
    flash backend forced (on ROCm an AOTriton kernel; enable_gqa lets it
    read the grouped K/V in place), timed like the prefill.  Context for the
    prefill's rate, with the largest difference from this library's output;
    None in every figure if the backend is not available."""
    import torch.nn.functional as F
    from torch.nn.attention import SDPBackend, sdpa_kernel
    name = "torch scaled_dot_product_attention, flash backend, is_causal, enable_gqa"
    try:
        with sdpa_kernel(SDPBackend.FLASH_ATTENTION):
            def call(i):
                return F.scaled_dot_product_attention(q, k, v, is_causal=True, scale=scale, enable_gqa=True)

            o = call(0)
            torch.cuda.synchronize()
            diff = float((o.float() - ours).abs().max())
            ms = event_time_ms(call, iters, torch)
    except Exception as e:   # an optional context figure never stops the bench
        return {"kernel": name, "value": None, "unit": "TFLOP/s", "error": str(e)[:200]}
    tf = flops / (ms * 1e-3) / 1e12
    return {"kernel": name, "value": round(tf, 2), "unit": "TFLOP/s", "ms_per_call": round(ms, 5),
            "max_abs_diff_from_this_library": round(diff, 6)}


def vendor_attention_backward_reference(torch, q, k, v, dout, ours, scale: float, iters: int,
                                        flops: float) -> dict:
    """The backward of torch's flash-backend causal attention (enable_gqa, so
    the K/V gradients are summed over each group) on the same inputs and
    upstream gradient, timed like this library's backward; context, with the
    largest difference of each gradient from this library's, relative to that
    gradient's largest magnitude."""
    import torch.nn.functional as F
    from torch.nn.attention import SDPBackend, sdpa_kernel
    name = "torch scaled_dot_product_attention backward, flash backend, is_causal, enable_gqa"
    try:
        with sdpa_kernel(SDPBackend.FLASH_ATTENTION):
            qr, kr, vr = (t.detach().clone().requires_grad_(True) for t in (q, k, v))
            o = F.scaled_dot_product_attention(qr, kr, vr, is_causal=True, scale=scale, enable_gqa=True)

            def call(i):
                return torch.autograd.grad(o, (qr, kr, vr), dout, retain_graph=True)

            grads = call(0)
            torch.cuda.synchronize()
            rel = max(float((g.float() - r).abs().max() / r.abs().max()) for g, r in zip(grads, ours))
            del grads
            ms = event_time_ms(call, iters, torch, min_per_batch=5)
    except Exception as e:   # an optional context figure never stops the bench
        return {"kernel": name, "value": None, "unit": "TFLOP/s", "error": str(e)[:200]}
    tf = flops / (ms * 1e-3) / 1e12
    return {"kernel": name, "value": round(tf, 2), "unit": "TFLOP/s", "ms_per_call": round(ms, 5),
            "max_rel_diff_from_this_library": round(rel, 6)}


def vendor_decode_reference(torch, q, ks, vs, ours, scale: float, iters: int, kv_bytes: int) -> dict:
    """torch's own attention for the same decode step: the one query token of
    every head against the whole cache (every sequence full, so no mask),
    flash backend forced, K/V read in place through enable_gqa, rotated over
    the same cache copies and timed like the step.  Context for the decode
    rate, with the largest difference from this library's output."""
    import torch.nn.functional as F
    from torch.nn.attention import SDPBackend, sdpa_kernel
    name = "torch scaled_dot_product_attention, flash backend, enable_gqa, one query token"
    q4 = q.unsqueeze(2)
    try:
        with sdpa_kernel(SDPBackend.FLASH_ATTENTION):
            def call(i):
                return F.scaled_dot_product_attention(q4, ks[i % len(ks)], vs[i % len(vs)], scale=scale,
                                                      enable_gqa=True)

            o = call(0)
            torch.cuda.synchronize()
            diff = float((o.squeeze(2).float() - ours).abs().max())
            ms = event_time_ms(call, iters, torch)
    except Exception as e:   # an optional context figure never stops the bench
        return {"kernel": name, "value": None, "unit": "GB/s", "error": str(e)[:200]}
    return {"kernel": name, "value": round(kv_bytes / (ms * 1e-3) / 1e9, 2), "unit": "GB/s",
            "ms_per_step": round(ms, 5), "max_abs_diff_from_this_library": round(diff, 6)}


def record_counters(fetch_csv: str, write_csv: str, workload: str) -> dict:
    """Build profiles/counters.json from two rocprofv3 --pmc runs of
    ``bench.py --calibration-copy`` (one with FETCH_SIZE, one with WRITE_SIZE).

    Each counter (KiB per dispatch) is scaled by the factor that maps its
    reading for the calibration copy kernel (the last elementwise dispatch:
    256 MiB read, 256 MiB written) onto the bytes that kernel moves."""
    import csv

    def per_kernel(path, counter):
        rows = [r for r in csv.DictReader(open(path)) if r["Counter_Name"] == counter]
        calib = [float(r["Counter_Value"]) for r in rows if "elementwise" in r["Kernel_Name"]]
        if not calib:
            raise SystemExit(f"{path}: no calibration copy dispatch (run bench.py --calibration-copy)")
        factor = CALIBRATION_BYTES / (calib[-1] * 1024)
        vals = {}
        for r in rows:
            for sub, name in COUNTED_KERNELS.items():
                if sub in r["Kernel_Name"]:
                    vals.setdefault(name, []).append(float(r["Counter_Value"]))
        return factor, {k: sum(v) / len(v) for k, v in vals.items()}, {k: len(v) for k, v in vals.items()}

    ff, fetch, nf = per_kernel(fetch_csv, "FETCH_SIZE")
    wf, write, nw = per_kernel(write_csv, "WRITE_SIZE")
    # entries of other workloads recorded earlier are kept; this run's replace theirs
    try:
        with open(COUNTERS) as f:
            kept = json.load(f).get("kernels", {})
    except (OSError, ValueError):
        kept = {}
    out = {"calibration": {"kernel": "torch.neg over 64 Mi float32 (256 MiB read + 256 MiB written)",
                           "fetch_factor": round(ff, 4), "write_factor": round(wf, 4)},
           "kernels": kept}
    for name in fetch:
        wl = "prefill-4k" if name.startswith("prefill") else workload
        fb, wb = fetch[name] * 1024 * ff, write.get(name, 0.0) * 1024 * wf
        out["kernels"][f"{name}|{wl}"] = {
            "source_digest": kernel_source_digest(name),
            "fetch_kib_raw": round(fetch[name], 1), "write_kib_raw": round(write.get(name, 0.0), 1),
            "dispatches": [nf[name], nw.get(name, 0)],
            "fetch_factor": round(ff, 4), "write_factor": round(wf, 4),
            "fetch_bytes": int(fb), "write_bytes": int(wb), "traffic_bytes": int(fb + wb)}
    return out


def cpu_baseline_decode(inp, budget_s: float, pg=None, fq=None, max_passes: int = 50):
    """Time the float64 oracle on the host, one whole sequence of the workload
    per call, cycling over the batch until about `budget_s` seconds of oracle
    time have been spent (input conversion to float64 is not timed).  For a
    paged workload the oracle is decode_paged over that sequence's pages."""
    from threadpoolctl import threadpool_info, threadpool_limits
    import gqa_inputs as gi
    import oracle
    cores = min(16, len(os.sched_getaffinity(0)))
    cfg = inp.cfg
    elem = 2 if cfg.dtype == "bf16" else 4
    calls, t_used, bytes_done = 0, 0.0, 0
    with threadpool_limits(limits=cores):
        used = max([p.get("num_threads", 1) for p in threadpool_info()] or [1])
        while t_used < budget_s and calls < max_passes * cfg.batch:
            b = calls % cfg.batch
            q = gi.to_f64(inp.q[b:b + 1], cfg.dtype)
            if fq is not None:
                t0 = time.perf_counter()
                oracle.decode_fp8(q, fq.k_cache[b:b + 1], fq.v_cache[b:b + 1], fq.k_scale, fq.v_scale,
                                  inp.seq_lens[b:b + 1], cfg.scale)
            elif pg is None:
                kf = gi.to_f64(inp.k_cache[b:b + 1], cfg.dtype)
                vf = gi.to_f64(inp.v_cache[b:b + 1], cfg.dtype)
                t0 = time.perf_counter()
                oracle.decode(q, kf, vf, inp.seq_lens[b:b + 1], cfg.scale)
            else:
                n = -(-int(inp.seq_lens[b]) // pg.page_size)
                ids = pg.block_table[b, :n]
                kf = gi.to_f64(pg.k_pages[ids], cfg.dtype)
                vf = gi.to_f64(pg.v_pages[ids], cfg.dtype)
                table = np.arange(n, dtype=np.int32)[None, :]
                t0 = time.perf_counter()
                oracle.decode_paged(q, kf, vf, table, inp.seq_lens[b:b + 1], pg.page_size, cfg.scale)
            t_used += time.perf_counter() - t0
            calls += 1
            bytes_done += decode_kv_bytes(inp.seq_lens[b:b + 1], cfg.num_kv_heads, cfg.head_dim,
                                          1 if fq is not None else elem)
    what = "decode_paged" if pg is not None else "decode_fp8" if fq is not None else "decode"
    return {"value": round(bytes_done / t_used / 1e9, 4), "unit": "GB/s", "cores": int(used),
            "kind": "oracle",
            "sample": f"{calls} single-sequence oracle.{what} calls cycling over the {cfg.batch} sequences of "
                      f"the same workload ({calls / cfg.batch:.2f} passes; float64 numpy, explicit K/V repeat), "
                      f"{t_used:.1f} s of oracle time; value = K/V bytes of the cache / oracle time"}


def cpu_baseline_prefill(p, budget_s: float):
    """Time the float64 oracle's causal prefill on the host, one (sequence,
    KV head) group per call -- the g query heads that share one KV head, with
    that head's K and V -- cycling over the groups of the workload until about
    `budget_s` seconds of oracle time have been spent.  The rate is the exact
    causal FLOP count of the groups done (the same count the GPU figure uses)
    over the oracle time; conversion to float64 is not timed."""
    from threadpoolctl import threadpool_info, threadpool_limits
    import gqa_inputs as gi
    import oracle
    cfg = p.cfg
    g = cfg.num_q_heads // cfg.num_kv_heads
    groups = [(b, j) for b in range(cfg.batch) for j in range(cfg.num_kv_heads)]
    cores = min(16, len(os.sched_getaffinity(0)))
    calls, t_used, flops = 0, 0.0, 0
    with threadpool_limits(limits=cores):
        used = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
        while t_used < budget_s and calls < len(groups):
            b, j = groups[calls]
            q = gi.to_f64(p.q[b:b + 1, j * g:(j + 1) * g], "bf16")
            k = gi.to_f64(p.k[b:b + 1, j:j + 1], "bf16")
            v = gi.to_f64(p.v[b:b + 1, j:j + 1], "bf16")
            t0 = time.perf_counter()
            oracle.prefill_causal(q, k, v, cfg.scale)
            t_used += time.perf_counter() - t0
            calls += 1
            flops += prefill_flops(1, g, cfg.seq_len, cfg.head_dim)
    return {"value": round(flops / t_used / 1e12, 6), "unit": "TFLOP/s", "cores": int(used), "kind": "oracle",
            "sample": f"{calls} of the {len(groups)} (sequence, KV head) groups of {gi.describe(cfg)}: "
                      f"oracle.prefill_causal over the group's {g} query heads (float64 numpy, explicit K/V "
                      f"repeat, full score matrix then the causal mask), {t_used:.1f} s of oracle time; "
                      f"value = exact causal FLOPs of those groups / oracle time"}


# Figures the source pages themselves report, on other hardware and for whole
# systems: context for the measured numbers, never a target or a baseline.
PAGE_FIGURES = [
    {"source": "deepconcepts.dev, 'Grouped-Query Attention', opening interactive example",
     "what": "decode throughput of Qwen3-8B at 8k tokens of context, 8 vs 32 KV heads",
     "value": "1,738 vs 413 tokens/s", "hardware": "NVIDIA H100",
     "kind": "interactive estimate, whole model (49 vs 11 resident sequences)"},
    {"source": "inferencex.semianalysis.com, 'KV head replication', 'How to read it in InferenceX'",
     "what": "gain of the low-concurrency tuning round (TP8 attention plus expert parallelism), "
             "1k input / 1k output",
     "value": "+22.9% at concurrency 4, +18.1% at concurrency 8", "hardware": "Google Ironwood TPU",
     "kind": "measured, whole serving system"},
]


def bench_wide(args, torch, gi, gqa) -> dict:
    """Decode in the absorbed-MLA shape (gqa_decode_wide): 128 query heads
    over one 576-column cached row per token whose first 512 columns are the
    value.  value = cached-row bytes read per step / step time."""
    cfg = gi.WIDE_CONFIGS["mla-decode"]
    inp = gi.make_wide(cfg)
    B, Hq, Hkv, T = cfg.batch, cfg.num_q_heads, cfg.num_kv_heads, cfg.max_seq_len
    lens64 = inp.seq_lens.astype(np.int64)
    kv_bytes = int(lens64.sum()) * Hkv * cfg.d_k * 2
    flops = int(lens64.sum()) * Hq * (cfg.d_k + cfg.d_v) * 2
    q = torch.from_numpy(inp.q.view(np.int16)).view(torch.bfloat16).cuda()
    kv0 = torch.from_numpy(inp.kv_cache.view(np.int16)).view(torch.bfloat16).cuda()
    rot = max(2, math.ceil(4 * MALL_BYTES / kv0.numel() / 2))
    kvs = [kv0] + [kv0.clone() for _ in range(rot - 1)]
    lens = torch.from_numpy(inp.seq_lens).cuda()
    nranges, nbytes = gqa.gqa_decode_wide_plan(B, Hq, Hkv, T, cfg.d_k, cfg.d_v, args.split_tokens)
    ws = torch.empty(max(nbytes, 256), dtype=torch.uint8, device="cuda")
    out = torch.empty(B, Hq, cfg.d_v, dtype=torch.float32, device="cuda")

    def step(i):
        gqa.gqa_decode_wide(q, kvs[i % rot], lens, cfg.d_v, scale=cfg.scale, split_tokens=args.split_tokens,
                            out=out, workspace=ws)

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    ms = event_time_ms(step, args.steps, torch)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    gbs = kv_bytes / (ms * 1e-3) / 1e9
    tf = flops / (ms * 1e-3) / 1e12
    alg_bytes = kv_bytes + B * Hq * cfg.d_k * 2
    achieved = alg_bytes / (ms * 1e-3) / 1e9
    result = {
        "metric": METRIC, "value": round(gbs, 2), "unit": "GB/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms, 5), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": gi.describe(cfg), "global_batch": B, "seq_len": T, "num_q_heads": Hq,
                   "num_kv_heads": Hkv, "head_dim_qk": cfg.d_k, "head_dim_v": cfg.d_v,
                   "token_ranges": nranges, "kv_rotation_copies": rot, "parallelism": "single-gpu"},
        "pct_of_hbm_peak": round(100 * gbs / HBM_PEAK_GBS, 2),
        "decode_tokens_per_s": round(B / (ms * 1e-3), 1),
        "decode_tflops": round(tf, 2),
        "pct_of_mfma_peak": round(100 * tf / BF16_MFMA_PEAK_TFLOPS, 2),
        # intensity (d_k + d_v) * 2 * Hq / (2 d_k) = 242 FLOP/B is below the ridge
        # 2500 / 8 = 312 FLOP/B, so the roofline's attainable rate is the HBM one
        "roofline": {"kernel": "decode_wide_bf16 + decode_wide_merge", "bound": "hbm",
                     "achieved": round(achieved, 2), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": load_counters("decode_wide", "mla-decode"),
                     "algorithmic_bytes": alg_bytes, "algorithmic_flops": flops,
                     "flop_per_byte": round(flops / alg_bytes, 1), "ms_per_launch": round(ms, 5)},
        "timed_wall_s": round(wall, 4),
    }
    if args.calibration_copy:
        src = torch.ones(64 * 2 ** 20, dtype=torch.float32, device="cuda")
        torch.neg(src, out=torch.empty_like(src))
        torch.cuda.synchronize()
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline_wide(inp, args.cpu_budget)
    return result


def expanded_ab(args, torch, gi, gqa, q, ks, vs, lens, grouped_out, cfg, inp, grouped_ms):
    """The same decode kernel on an explicitly repeated cache: K and V
    repeated along the head axis (head h holds KV head h // g, the order of
    the oracle's repeat) and decoded with Hkv = Hq, each query head reading
    its own copy.  The result is the same attention; the step reads g times
    the bytes (study.greatitself.com, "Grouped-Query and Multi-Query
    Attention", section "Share keys and values without confusing query-head
    identity": expanding K/V keeps the arithmetic but loses the bandwidth
    advantage)."""
    B, Hq, Hkv, d = cfg.batch, cfg.num_q_heads, cfg.num_kv_heads, cfg.head_dim
    g = Hq // Hkv
    kx = [torch.repeat_interleave(k, g, dim=1).contiguous() for k in ks]
    vx = [torch.repeat_interleave(v, g, dim=1).contiguous() for v in vs]
    rot = len(kx)
    T = kx[0].shape[2]
    plan = gqa.gqa_decode_plan(B, Hq, Hq, d, T, gqa.GQA_BF16, 0)
    ws = torch.empty(plan.workspace_bytes, dtype=torch.uint8, device="cuda")
    xout = torch.empty_like(grouped_out)

    def xstep(i):
        gqa.gqa_decode(q, kx[i % rot], vx[i % rot], lens, scale=cfg.scale, out=xout, workspace=ws)

    for i in range(max(3, args.warmup // 2)):
        xstep(i)
    ms = event_time_ms(xstep, args.steps, torch)
    # both outputs from the same cache copy
    gqa.gqa_decode(q, ks[0], vs[0], lens, scale=cfg.scale, out=grouped_out)
    xstep(0)
    torch.cuda.synchronize()
    diff = float((xout - grouped_out).abs().max().item())
    xbytes = decode_kv_bytes(inp.seq_lens, Hq, d, 2)
    return {"workload": f"{gi.describe(cfg)}: K/V repeated to {Hq} KV heads, same kernel",
            "kv_bytes": xbytes, "ms_per_step": round(ms, 5),
            "kv_read_gb_per_s": round(xbytes / (ms * 1e-3) / 1e9, 2),
            "decode_tokens_per_s": round(B / (ms * 1e-3), 1),
            "grouped_ms_per_step": round(grouped_ms, 5),
            "slowdown_vs_grouped": round(ms / grouped_ms, 3),
            "max_abs_diff_vs_grouped": diff}


def cpu_baseline_wide(inp, budget_s: float, max_passes: int = 4):
    """The float64 oracle (oracle.decode_wide) on the host, one sequence per
    call, cycling over the batch until about `budget_s` seconds are spent."""
    from threadpoolctl import threadpool_info, threadpool_limits
    import gqa_inputs as gi
    import oracle
    cfg = inp.cfg
    cores = min(16, len(os.sched_getaffinity(0)))
    calls, t_used, bytes_done = 0, 0.0, 0
    with threadpool_limits(limits=cores):
        used = max([p.get("num_threads", 1) for p in threadpool_info()] or [1])
        while t_used < budget_s and calls < max_passes * cfg.batch:
            b = calls % cfg.batch
            q = gi.to_f64(inp.q[b:b + 1], "bf16")
            kv = gi.to_f64(inp.kv_cache[b:b + 1, :, :int(inp.seq_lens[b])], "bf16")
            t0 = time.perf_counter()
            oracle.decode_wide(q, kv, inp.seq_lens[b:b + 1], cfg.d_v, cfg.scale)
            t_used += time.perf_counter() - t0
            calls += 1
            bytes_done += int(inp.seq_lens[b]) * cfg.num_kv_heads * cfg.d_k * 2
    return {"value": round(bytes_done / t_used / 1e9, 4), "unit": "GB/s", "cores": int(used), "kind": "oracle",
            "sample": f"{calls} single-sequence oracle.decode_wide calls cycling over the {cfg.batch} sequences "
                      f"of mla-decode, {t_used:.1f} s of oracle time; value = cached-row bytes / oracle time"}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="llama3-8b",
                    choices=["llama3-8b", "wide-group", "mqa-128k", "group-32", "group-71", "paged-llama3-8b", "paged-wide-group",
                             "fp8-llama3-8b", "fp8-wide-group", "fp8-mqa-128k", "mla-decode"])
    ap.add_argument("--page-size", type=int, default=16, help="tokens per page for the paged-* workloads")
    ap.add_argument("--record-counters", nargs=2, metavar=("FETCH_CSV", "WRITE_CSV"),
                    help="write profiles/counters.json from two rocprofv3 --pmc counter CSVs and exit")
    ap.add_argument("--print-digests", action="store_true",
                    help="print the source digest of each measured kernel and exit")
    ap.add_argument("--split-tokens", type=int, default=0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-prefill", action="store_true")
    ap.add_argument("--expanded", action="store_true",
                    help="also run the same decode kernel on an explicitly repeated cache (Hkv = Hq) "
                         "and report it beside the grouped step in \"expanded_ab\"")
    ap.add_argument("--cpu-budget", type=float, default=12.0)
    ap.add_argument("--calibration-copy", action="store_true",
                    help="also run one plain 256 MiB device copy kernel (counter calibration)")
    args = ap.parse_args()
    if args.record_counters:
        data = record_counters(*args.record_counters, args.workload)
        with open(COUNTERS, "w") as f:
            json.dump(data, f, indent=1)
            f.write("\n")
        print(json.dumps(data))
        return
    if args.print_digests:
        print(json.dumps({k: kernel_source_digest(k) for k in KERNEL_SOURCES}))
        return
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: the GQA kernels here run on a single device "
              "and no multi-GPU path is built; run with --gpus 1.", file=sys.stderr)
        sys.exit(2)

    import torch
    import gqa_inputs as gi
    import grouped_query_attention_gqa_amd as gqa

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(2)
    gqa.load_library()   # fail loudly if the HIP library is missing
    torch.cuda.set_device(0)
    cus, khz = gqa.gqa_device_info(0)
    props = torch.cuda.get_device_properties(0)
    device = {"name": props.name, "arch": getattr(props, "gcnArchName", ""), "compute_units": cus,
              "max_clock_mhz": round(khz / 1000.0, 1),
              # gfx950 matrix cores: 4,096 dense bf16 FLOP per clock per compute unit
              "bf16_dense_peak_tflops_from_props": round(cus * 4096 * khz * 1e3 / 1e12, 1),
              "note": "the roofline peaks are the published 8 TB/s and 2.5 PFLOP/s"}

    if args.workload == "mla-decode":
        res = bench_wide(args, torch, gi, gqa)
        res["device"] = device
        print(json.dumps(res), flush=True)
        return

    paged = args.workload.startswith("paged-")
    fp8 = args.workload.startswith("fp8-")
    cfg = gi.CONFIGS[args.workload.split("-", 1)[1] if (paged or fp8) else args.workload]
    inp = gi.make_decode(cfg)
    elem = 1 if fp8 else (2 if cfg.dtype == "bf16" else 4)
    dt = gqa.GQA_FP8_E4M3 if fp8 else (gqa.GQA_BF16 if cfg.dtype == "bf16" else gqa.GQA_F32)
    B, Hq, Hkv, d, T = cfg.batch, cfg.num_q_heads, cfg.num_kv_heads, cfg.head_dim, cfg.max_seq_len
    kv_bytes = decode_kv_bytes(inp.seq_lens, Hkv, d, elem)
    alloc_kv = 2 * B * Hkv * T * d * elem
    rot = max(2, math.ceil(4 * MALL_BYTES / alloc_kv))

    def to_dev(a):
        if cfg.dtype == "bf16":
            return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).cuda()
        return torch.from_numpy(a).cuda()

    q = to_dev(inp.q)
    lens = torch.from_numpy(inp.seq_lens).cuda()
    pg = fq = None
    if fp8:
        # the same cache as E4M3 codes with per-KV-head scales
        fq = gi.make_fp8(inp)
        inp.k_cache = inp.v_cache = None
        k0, v0 = torch.from_numpy(fq.k_cache).cuda(), torch.from_numpy(fq.v_cache).cuda()
        k_scale, v_scale = torch.from_numpy(fq.k_scale).cuda(), torch.from_numpy(fq.v_scale).cuda()
    elif paged:
        # the same cache scattered into a permuted pool of pages
        pg = gi.make_paged(inp, page_size=args.page_size)
        inp.k_cache = inp.v_cache = None
        k0, v0 = to_dev(pg.k_pages), to_dev(pg.v_pages)
        table = torch.from_numpy(pg.block_table).cuda()
        T = pg.block_table.shape[1] * args.page_size
    else:
        k0, v0 = to_dev(inp.k_cache), to_dev(inp.v_cache)
    ks = [k0] + [k0.clone() for _ in range(rot - 1)]
    vs = [v0] + [v0.clone() for _ in range(rot - 1)]
    plan = gqa.gqa_decode_plan(B, Hq, Hkv, d, T, dt, args.split_tokens)
    ws = torch.empty(plan.workspace_bytes, dtype=torch.uint8, device="cuda")
    out = torch.empty(B, Hq, d, dtype=torch.float32, device="cuda")

    def step(i):
        if fp8:
            gqa.gqa_decode_fp8(q, ks[i % rot], vs[i % rot], k_scale, v_scale, lens, scale=cfg.scale, out=out,
                               workspace=ws, split_tokens=args.split_tokens)
        elif paged:
            gqa.gqa_decode_paged(q, ks[i % rot], vs[i % rot], table, lens, scale=cfg.scale, out=out,
                                 workspace=ws, split_tokens=args.split_tokens)
        else:
            gqa.gqa_decode(q, ks[i % rot], vs[i % rot], lens, scale=cfg.scale, out=out, workspace=ws,
                           split_tokens=args.split_tokens)

    def split_only(i):
        if fp8:
            gqa.gqa_decode_fp8(q, ks[i % rot], vs[i % rot], k_scale, v_scale, lens, scale=cfg.scale, out=out,
                               workspace=ws, split_tokens=args.split_tokens, stage="split")
        elif paged:
            gqa.gqa_decode_paged(q, ks[i % rot], vs[i % rot], table, lens, scale=cfg.scale, out=out,
                                 workspace=ws, split_tokens=args.split_tokens, stage="split")
        else:
            gqa.gqa_decode_split(q, ks[i % rot], vs[i % rot], lens, out, ws, scale=cfg.scale,
                                 split_tokens=args.split_tokens)

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    ms_step = event_time_ms(step, args.steps, torch)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_split = event_time_ms(split_only, args.steps, torch)
    value = kv_bytes / (ms_step * 1e-3) / 1e9
    split_bytes = decode_split_bytes(inp.seq_lens, Hq, Hkv, d, elem)
    if fp8:   # q is bf16 (2 B per element) and there are 2 * Hkv float scales
        split_bytes += B * Hq * d * (2 - elem) + 8 * Hkv
    if paged:   # plus one read of each block-table entry in use
        split_bytes += 4 * int(np.sum(-(-inp.seq_lens.astype(np.int64) // args.page_size)))
    achieved = split_bytes / (ms_split * 1e-3) / 1e9
    traffic = load_counters("decode_split", args.workload)

    result = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp8-e4m3 cache, bf16 compute" if fp8 else cfg.dtype,
        "data": "synthetic",
        "config": {"workload": (f"paged (page {args.page_size}) " if paged else "FP8 E4M3 cache, " if fp8 else "")
                   + gi.describe(cfg),
                   "global_batch": B, "seq_len": cfg.max_seq_len,
                   "num_q_heads": Hq, "num_kv_heads": Hkv, "head_dim": d,
                   "range_tokens": plan.range_tokens or "auto", "workgroups": plan.workgroups,
                   "kv_rotation_copies": rot, "parallelism": "single-gpu"},
        "pct_of_hbm_peak": round(100 * value / HBM_PEAK_GBS, 2),
        "decode_tokens_per_s": round(B / (ms_step * 1e-3), 1),
        "decode_tflops": round(decode_flops(inp.seq_lens, Hq, d) / (ms_step * 1e-3) / 1e12, 3),
        "roofline": {"kernel": ("decode_split_bf16 (paged)" if paged else "decode_split_bf16 (E4M3 cache)"
                                if fp8 else "decode_split_bf16") if cfg.dtype == "bf16" else "decode_split_f32",
                     "bound": "hbm", "achieved": round(achieved, 2), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "traffic": traffic, "algorithmic_bytes": split_bytes,
                     "ms_per_launch": round(ms_split, 5)},
        "timed_wall_s": round(wall, 4),
    }
    if not (paged or fp8) and cfg.dtype == "bf16" and bool(np.all(inp.seq_lens == cfg.max_seq_len)):
        step(0)   # out holds this library's result for the first cache copy
        vref = vendor_decode_reference(torch, q, ks, vs, out, cfg.scale, max(20, args.steps // 2), kv_bytes)
        if vref["value"]:
            vref["step_over_reference"] = round(value / vref["value"], 4)
        result["vendor_attention_reference"] = vref

    if args.expanded and cfg.dtype == "bf16" and not (paged or fp8) and Hq > Hkv:
        result["expanded_ab"] = expanded_ab(args, torch, gi, gqa, q, ks, vs, lens, out, cfg, inp, ms_step)

    if not args.no_prefill:
        pc = gi.CONFIGS["prefill-4k"]
        p = gi.make_prefill(pc)
        pq, pk, pv = (torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).cuda() for a in (p.q, p.k, p.v))
        pout = torch.empty(pc.batch, pc.num_q_heads, pc.seq_len, pc.head_dim, dtype=torch.float32,
                           device="cuda")

        def pstep(i):
            gqa.gqa_prefill_causal(pq, pk, pv, scale=pc.scale, out=pout)

        for i in range(max(3, args.warmup // 2)):
            pstep(i)
        pms = event_time_ms(pstep, max(100, args.steps), torch)
        fl = prefill_flops(pc.batch, pc.num_q_heads, pc.seq_len, pc.head_dim)
        tf = fl / (pms * 1e-3) / 1e12
        result["prefill"] = {
            "workload": gi.describe(pc), "value": round(tf, 2), "unit": "TFLOP/s",
            "ms_per_call": round(pms, 5), "tokens_per_s": round(pc.batch * pc.seq_len / (pms * 1e-3), 1),
            "pct_of_mfma_peak": round(100 * tf / BF16_MFMA_PEAK_TFLOPS, 2),
            "roofline": {"kernel": "prefill_causal_bf16", "bound": "mfma", "achieved": round(tf, 2),
                         "peak": BF16_MFMA_PEAK_TFLOPS, "unit": "TFLOP/s",
                         "frac": round(tf / BF16_MFMA_PEAK_TFLOPS, 4),
                         "traffic": load_counters("prefill_causal", "prefill-4k"),
                         "algorithmic_flops": fl,
                         "algorithmic_bytes": prefill_bytes(pc.batch, pc.num_q_heads, pc.num_kv_heads,
                                                            pc.seq_len, pc.head_dim)},
        }

        ref = matmul_reference(torch, max(100, args.steps))
        ref["prefill_over_reference"] = round(tf / ref["value"], 4)
        result["prefill"]["matmul_reference"] = ref
        att = vendor_attention_reference(torch, pq, pk, pv, pout, pc.scale, max(50, args.steps // 2), fl)
        if att["value"]:
            att["prefill_over_reference"] = round(tf / att["value"], 4)
        result["prefill"]["vendor_attention_reference"] = att

        # backward of the same prefill: dq, dk, dv from (q, k, v, out, lse, dout)
        pdo = torch.from_numpy(gi.make_dout(pc).view(np.int16)).view(torch.bfloat16).cuda()
        plse = torch.empty(pc.batch, pc.num_q_heads, pc.seq_len, dtype=torch.float32, device="cuda")
        gqa.gqa_prefill_causal(pq, pk, pv, scale=pc.scale, out=pout, lse=plse)
        grads = (torch.empty_like(pout),
                 torch.empty(pc.batch, pc.num_kv_heads, pc.seq_len, pc.head_dim, dtype=torch.float32,
                             device="cuda"),
                 torch.empty(pc.batch, pc.num_kv_heads, pc.seq_len, pc.head_dim, dtype=torch.float32,
                             device="cuda"))
        bws = torch.empty(gqa.gqa_prefill_backward_workspace(pc.batch, pc.num_q_heads, pc.num_kv_heads,
                                                             pc.seq_len, pc.head_dim),
                          dtype=torch.uint8, device="cuda")

        def bstep(i):
            gqa.gqa_prefill_causal_backward(pq, pk, pv, pout, plse, pdo, scale=pc.scale, workspace=bws,
                                            grads=grads)

        for i in range(max(3, args.warmup // 2)):
            bstep(i)
        bms = event_time_ms(bstep, max(100, args.steps), torch)
        bfl = prefill_backward_flops(pc.batch, pc.num_q_heads, pc.seq_len, pc.head_dim)
        btf = bfl / (bms * 1e-3) / 1e12
        result["prefill_backward"] = {
            "workload": gi.describe(pc) + " backward (dq, dk, dv)", "value": round(btf, 2),
            "unit": "TFLOP/s", "ms_per_call": round(bms, 5),
            "tokens_per_s": round(pc.batch * pc.seq_len / (bms * 1e-3), 1),
            "pct_of_mfma_peak": round(100 * btf / BF16_MFMA_PEAK_TFLOPS, 2),
            "roofline": {"kernel": "prefill_bwd_dq + prefill_bwd_dkdv", "bound": "mfma",
                         "achieved": round(btf, 2), "peak": BF16_MFMA_PEAK_TFLOPS, "unit": "TFLOP/s",
                         "frac": round(btf / BF16_MFMA_PEAK_TFLOPS, 4),
                         "traffic": {k: load_counters(k, "prefill-4k")
                                     for k in ("prefill_bwd_dq", "prefill_bwd_dkdv")},
                         "algorithmic_flops": bfl,
                         "executed_flops": 3.5 * prefill_flops(pc.batch, pc.num_q_heads, pc.seq_len,
                                                               pc.head_dim)},
        }
        batt = vendor_attention_backward_reference(torch, pq, pk, pv, pdo, grads, pc.scale, 25, bfl)
        if batt["value"]:
            batt["backward_over_reference"] = round(btf / batt["value"], 4)
        result["prefill_backward"]["vendor_attention_reference"] = batt

    if args.calibration_copy:
        # one elementwise kernel that reads 256 MiB and writes 256 MiB, the
        # known-size launch the FETCH_SIZE / WRITE_SIZE counters are scaled by
        src = torch.ones(64 * 2 ** 20, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        torch.neg(src, out=dst)
        torch.cuda.synchronize()

    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline_decode(inp, args.cpu_budget, pg, fq)
        if "prefill" in result:
            result["prefill"]["cpu_baseline"] = cpu_baseline_prefill(p, args.cpu_budget)
    result["context_from_pages"] = PAGE_FIGURES
    result["device"] = device

    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
