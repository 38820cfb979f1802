#!/usr/bin/env python3
"""Benchmark of the exact tiled attention hot path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W]

One step is one fa_fwd call (the whole prefill path: Q tile load, K/V tile
streaming, QK^T, masking, online softmax, PV, finalise) over the
Llama-3-8B-shaped long-context causal GQA workload (B=1, Hq=32, Hkv=8,
T=32768, d=128, bf16), the largest of the prefill workloads.  `value` is its
attention TFLOP/s (4*B*Hq*T*T*d/2 per call) over the wall-clock of K
back-to-back steps, inputs resident in HBM.  The same JSON line carries:

  roofline      achieved FLOP/s of the forward kernel (mean launch duration
                from HIP events recorded on the launch stream around every
                launch; median and min beside it) against the dense bf16
                matrix-core peak;
  also          the other workloads measured the same way, each with its own
                roofline block: Qwen3-0.6B GQA prefill and GPT-2-small MHA
                prefill (TFLOP/s), chunked prefill, 8-bit prefill, the
                backward pass, and split-KV decode over a 16-sequence cache
                (HBM GB/s) with a sweep of the split count;
  cpu_baseline  the fp64 CPU oracle timed on a bounded sample of the
                headline workload (whole heads, one per host thread).

Only rank 0 at one GPU is supported; more GPUs exit with a message.
"""
from __future__ import annotations

import argparse
import hashlib
import re
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2516.6   # MI355X dense bf16 matrix-core peak (256 CU x 2.4 GHz x 4096 FLOP/clk)
PEAK_HBM_GBS = 8000.0       # MI355X HBM3E peak
PEAK_FP8_TFLOPS = 5033.2    # MI355X dense fp8 matrix-core peak (twice the bf16 rate)
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic.json")
# Sources each workload's kernels are built from: a traffic figure counts
# only while they are unchanged since the counters were taken.
KERNEL_SOURCES = {
    "prefill": ["exact_tiled_attention_02_amd/csrc/fa_fwd.hip",
                "exact_tiled_attention_02_amd/csrc/fa_device.h",
                "exact_tiled_attention_02_amd/csrc/fa_lds.h",
                "exact_tiled_attention_02_amd/csrc/fa_launch.h"],
    "prefill_fp8": ["exact_tiled_attention_02_amd/csrc/fa_fwd_fp8.hip",
                    "exact_tiled_attention_02_amd/csrc/fa_device.h",
                    "exact_tiled_attention_02_amd/csrc/fa_lds.h",
                    "exact_tiled_attention_02_amd/csrc/fa_launch.h"],
    "decode": ["exact_tiled_attention_02_amd/csrc/fa_decode.hip",
               "exact_tiled_attention_02_amd/csrc/fa_device.h",
               "exact_tiled_attention_02_amd/csrc/fa_launch.h"],
}


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def _code_only(text: str) -> str:
    """Source text without comments and blank lines, so that an edit to a
    comment does not invalidate counters taken from the same code."""
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    lines = (re.sub(r"//.*$", "", ln).rstrip() for ln in text.splitlines())
    return "\n".join(ln for ln in lines if ln)


def kernel_source_hash(kind: str) -> str:
    h = hashlib.sha256()
    for rel in KERNEL_SOURCES[kind]:
        with open(os.path.join(ROOT, rel), encoding="utf-8") as f:
            h.update(_code_only(f.read()).encode())
    return h.hexdigest()[:16]


def measured_traffic(workload: str):
    """HBM bytes per launch of the workload's dominant kernel from the
    committed counter summary (FETCH_SIZE and WRITE_SIZE scaled by what they
    read for a copy of known size), or None when the kernel sources changed
    since the counters were taken."""
    try:
        with open(TRAFFIC_FILE, encoding="utf-8") as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None
    w = t.get("workloads", {}).get(workload)
    if w is None:
        return None
    from exact_tiled_attention_02_amd import inputs
    wk = inputs.WORKLOADS[workload]
    kind = ("decode" if isinstance(wk, inputs.Decode)
            else "prefill_fp8" if wk.dtype == "fp8" else "prefill")
    if w.get("kernel_source_hash") != kernel_source_hash(kind):
        return None
    return w.get("hbm_bytes_per_launch")


# ----------------------------------------------------------------------------
# Synthetic device inputs: N(0,1) fp32 from a seeded generator, optional
# query multiplier, one round-to-nearest-even conversion to bf16.
# ----------------------------------------------------------------------------

def dev_normal(torch, shape, gen, mult=1.0):
    x = torch.randn(shape, generator=gen, device="cuda", dtype=torch.float32)
    if mult != 1.0:
        x.mul_(mult)
    return x.to(torch.bfloat16)


def time_calls(torch, launch, steps: int, warmup: int) -> dict:
    """Run `launch` warmup times, then `steps` times back to back, bracketed
    by device synchronisation.  HIP events recorded on the launch stream
    (torch's current stream, which every launch here uses) before each timed
    call and after the last give each call's duration.  Returns wall
    seconds per call and the mean, median and min event duration in ms."""
    for _ in range(warmup):
        launch()
    torch.cuda.synchronize()
    events = [torch.cuda.Event(enable_timing=True) for _ in range(steps + 1)]
    t0 = time.perf_counter()
    for i in range(steps):
        events[i].record()
        launch()
    events[steps].record()
    torch.cuda.synchronize()
    wall = (time.perf_counter() - t0) / steps
    per = sorted(events[i].elapsed_time(events[i + 1]) for i in range(steps))
    mid = per[steps // 2] if steps % 2 else 0.5 * (per[steps // 2 - 1] + per[steps // 2])
    return {"wall_s": wall, "mean_ms": events[0].elapsed_time(events[steps]) / steps,
            "median_ms": mid, "min_ms": per[0]}


def prefill_case(torch, fa, w, steps, warmup, seed=0):
    gen = torch.Generator(device="cuda")
    gen.manual_seed(seed)
    stream = torch.cuda.current_stream()
    lse = torch.empty((w.B, w.Hq, w.Tq), dtype=torch.float32, device="cuda")
    if w.dtype == "fp8":
        # fp32 N(0,1) draws stored as E4M3 codes with block scales: one per
        # query row, one per (batch, kv head) for k and v.
        def quant(x, dims):
            sc = x.abs().amax(dim=dims, keepdim=True) / 448.0
            return (x / sc).to(torch.float8_e4m3fn).view(torch.uint8), sc.reshape(
                [n for i, n in enumerate(x.shape) if i - x.dim() not in dims]).contiguous()
        qf = torch.randn((w.B, w.Hq, w.Tq, w.d), generator=gen, device="cuda") * w.q_mult
        kf = torch.randn((w.B, w.Hkv, w.Tk, w.d), generator=gen, device="cuda")
        vf = torch.randn((w.B, w.Hkv, w.Tk, w.d), generator=gen, device="cuda")
        q, qs = quant(qf, (-1,))
        k, ks = quant(kf, (-2, -1))
        v, vs = quant(vf, (-2, -1))
        del qf, kf, vf
        o = torch.empty((w.B, w.Hq, w.Tq, w.d), dtype=torch.bfloat16, device="cuda")
        launch = fa.prepared("fa_fwd_fp8", q, k, v, qs, ks, vs, o, lse, w.B, w.Hq, w.Hkv, w.Tq,
                             w.Tk, w.d, w.causal_mode, w.scale, stream=stream)
        t = time_calls(torch, launch, steps, warmup)
        del q, k, v, qs, ks, vs, o, lse
        return t
    q = dev_normal(torch, (w.B, w.Hq, w.Tq, w.d), gen, w.q_mult)
    k = dev_normal(torch, (w.B, w.Hkv, w.Tk, w.d), gen)
    v = dev_normal(torch, (w.B, w.Hkv, w.Tk, w.d), gen)
    o = torch.empty_like(q)

    launch = fa.prepared("fa_fwd", q, k, v, o, lse, w.B, w.Hq, w.Hkv, w.Tq, w.Tk, w.d,
                         w.causal_mode, w.scale, stream=stream)
    t = time_calls(torch, launch, steps, warmup)
    del q, k, v, o, lse
    return t


def backward_case(torch, fa, w, steps, warmup, seed=0):
    """fa_bwd on the workload's shapes: q, k, v and dout N(0,1) (q times the
    workload's multiplier), o and lse from one fa_fwd call.  Times the whole
    call (row-term, dQ and dK/dV kernels)."""
    gen = torch.Generator(device="cuda")
    gen.manual_seed(seed)
    q = dev_normal(torch, (w.B, w.Hq, w.Tq, w.d), gen, w.q_mult)
    k = dev_normal(torch, (w.B, w.Hkv, w.Tk, w.d), gen)
    v = dev_normal(torch, (w.B, w.Hkv, w.Tk, w.d), gen)
    do = dev_normal(torch, (w.B, w.Hq, w.Tq, w.d), gen)
    o = torch.empty_like(q)
    lse = torch.empty((w.B, w.Hq, w.Tq), dtype=torch.float32, device="cuda")
    stream = torch.cuda.current_stream()
    fa.fa_fwd(q, k, v, o, lse, w.B, w.Hq, w.Hkv, w.Tq, w.Tk, w.d, w.causal_mode, w.scale, stream)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    launch = fa.prepared("fa_bwd", q, k, v, o, lse, do, dq, dk, dv, w.B, w.Hq, w.Hkv, w.Tq,
                         w.Tk, w.d, w.causal_mode, w.scale, stream=stream)
    t = time_calls(torch, launch, steps, warmup)
    del q, k, v, do, o, lse, dq, dk, dv
    return t


def decode_case(torch, fa, w, steps, warmup, splits_list, copies=4, seed=0):
    """Decode timed over `copies` independent caches used in rotation, so the
    last-level cache cannot serve one call's reads from the previous call.
    Each requested split count in `splits_list` is timed on the same caches.
    Returns ({num_splits: timing}, algorithmic bytes per call, cached tokens)."""
    import numpy as np
    from exact_tiled_attention_02_amd import inputs
    seqlens = inputs.decode_seqlens(w, seed=seed)
    gen = torch.Generator(device="cuda")
    gen.manual_seed(seed)
    q = dev_normal(torch, (w.B, w.Hq, w.d), gen)
    caches = []
    for _ in range(copies):
        kc = dev_normal(torch, (w.B, w.Hkv, w.Tk_max, w.d), gen)
        vc = dev_normal(torch, (w.B, w.Hkv, w.Tk_max, w.d), gen)
        caches.append((kc, vc))
    sl = torch.from_numpy(seqlens).cuda()
    o = torch.empty_like(q)
    stream = torch.cuda.current_stream()
    if w.kv_dtype in ("fp8", "int8"):
        # Codes of N(0,1) rows scaled to the code range (E4M3 by torch's
        # conversion, int8 by rounding and clamping): the byte pattern of a
        # quantised cache; uniform random scales of the same order.
        coded = []
        for kc, vc in caches:
            ks = torch.rand((w.B, w.Hkv, w.Tk_max), generator=gen, device="cuda") * 0.01 + 0.005
            vs = torch.rand((w.B, w.Hkv, w.Tk_max), generator=gen, device="cuda") * 0.01 + 0.005
            if w.kv_dtype == "fp8":
                k8 = (kc * 40).to(torch.float8_e4m3fn).view(torch.uint8)
                v8 = (vc * 40).to(torch.float8_e4m3fn).view(torch.uint8)
            else:
                k8 = (kc * 40).round().clamp(-127, 127).to(torch.int8).view(torch.uint8)
                v8 = (vc * 40).round().clamp(-127, 127).to(torch.int8).view(torch.uint8)
            coded.append((k8, v8, ks, vs))
        del caches
        caches = coded
        entry = "fa_decode_fp8" if w.kv_dtype == "fp8" else "fa_decode_int8"

        def make(ns):
            return [fa.prepared(entry, q, k8, v8, ks, vs, sl, o, w.B, w.Hq, w.Hkv,
                                w.Tk_max, w.d, ns, stream=stream) for k8, v8, ks, vs in caches]
        row_bytes = w.d + 4   # codes plus the fp32 row scale, per tensor
    else:
        def make(ns):
            return [fa.prepared("fa_decode", q, kc, vc, sl, o, w.B, w.Hq, w.Hkv, w.Tk_max, w.d,
                                ns, stream=stream) for kc, vc in caches]
        row_bytes = w.d * 2
    out = {}
    for ns in splits_list:
        calls = make(ns)
        it = [0]

        def launch():
            calls[it[0] % copies]()
            it[0] += 1

        out[ns] = time_calls(torch, launch, steps, warmup)
    kv_bytes = int(seqlens.astype(np.int64).sum()) * w.Hkv * row_bytes * 2
    io_bytes = 2 * w.B * w.Hq * w.d * 2 + w.B * 4
    del caches, q, o
    torch.cuda.empty_cache()
    return out, kv_bytes + io_bytes, int(seqlens.sum())


def read_ceiling(torch, fa, nbytes=1 << 30, copies=2, steps=50, warmup=10):
    """Achievable read bandwidth of the device: the library's read probe
    streaming `nbytes` once per call (buffers used in rotation), GB/s."""
    bufs = [torch.ones(nbytes // 4, dtype=torch.int32, device="cuda") for _ in range(copies)]
    sink = torch.zeros(1, dtype=torch.int32, device="cuda")
    stream = torch.cuda.current_stream()
    calls = [fa.prepared("fa_read_probe", b, nbytes, sink, stream=stream) for b in bufs]
    it = [0]

    def launch():
        calls[it[0] % copies]()
        it[0] += 1

    t = time_calls(torch, launch, steps, warmup)
    del bufs
    torch.cuda.empty_cache()
    return nbytes / (t["mean_ms"] * 1e-3) / 1e9


def cpu_baseline(w, heads=None, max_s=60.0):
    """Time the fp64 oracle on whole (batch, head) pairs of the workload, one
    pair per host thread at a time (one-threaded BLAS in each), and scale to
    TFLOP/s.  By default twice as many pairs as threads; pairs not yet
    started after about `max_s` seconds of wall-clock are skipped."""
    import numpy as np
    from concurrent.futures import ThreadPoolExecutor
    import oracle
    from exact_tiled_attention_02_amd import inputs
    try:
        ncpu = len(os.sched_getaffinity(0))
    except (AttributeError, OSError):
        ncpu = os.cpu_count() or 1
    threads = max(1, min(16, ncpu))
    heads = 2 * threads if heads is None else heads
    q, k, v = inputs.prefill_inputs(w)
    g = w.Hq // w.Hkv
    per_head = 4.0 * w.Tq * w.Tk * w.d / (2 if w.causal else 1)
    order = [(b, h) for b in range(w.B) for h in range(w.Hq)][:heads]
    t0 = time.perf_counter()

    def one(bh):
        b, h = bh
        if time.perf_counter() - t0 > max_s:
            return 0
        oracle.softmax_attention(q[b:b + 1, h:h + 1], k[b:b + 1, h // g:h // g + 1],
                                 v[b:b + 1, h // g:h // g + 1], causal=w.causal, scale=w.scale)
        return 1

    try:
        from threadpoolctl import threadpool_limits
        limit = threadpool_limits(1)
    except Exception:
        limit = None
    try:
        with ThreadPoolExecutor(threads) as ex:
            done = sum(ex.map(one, order))
    finally:
        if limit is not None:
            limit.restore_original_limits()
    el = time.perf_counter() - t0
    return {
        "value": round(done * per_head / el / 1e12, 6),
        "unit": "TFLOP/s",
        "cores": threads,
        "kind": "oracle",
        "sample": f"{done} of {w.B * w.Hq} (batch, head) pairs of {w.name}, all {w.Tq} rows each, "
                  f"fp64 numpy three-pass, one pair per thread on {threads} threads, {el:.1f} s",
    }


def inputs_names():
    from exact_tiled_attention_02_amd import inputs
    names = list(inputs.WORKLOADS.keys())
    return names + ["bwd_" + n for n, w in inputs.WORKLOADS.items()
                    if isinstance(w, inputs.Prefill) and w.dtype == "bf16"]


def timing_fields(t):
    return {"kernel_ms": round(t["mean_ms"], 4), "kernel_ms_median": round(t["median_ms"], 4),
            "kernel_ms_min": round(t["min_ms"], 4)}


def prefill_entry(torch, fa, w, name, steps, warmup, kernel):
    """Time one prefill workload; its roofline block against its dtype's peak."""
    t = prefill_case(torch, fa, w, steps, warmup)
    peak = PEAK_FP8_TFLOPS if w.dtype == "fp8" else PEAK_BF16_TFLOPS
    ach = w.flops / (t["mean_ms"] * 1e-3) / 1e12
    return t, {"value": round(w.flops / t["wall_s"] / 1e12, 2), "unit": "TFLOP/s",
               "ms_per_call": round(t["wall_s"] * 1e3, 4), **timing_fields(t),
               "steps": steps, "dtype": w.dtype,
               "roofline": {"bound": "mfma", "achieved": round(ach, 2), "peak": peak,
                            "unit": "TFLOP/s", "frac": round(ach / peak, 4),
                            "frac_at_min": round(w.flops / (t["min_ms"] * 1e-3) / 1e12 / peak, 4),
                            "traffic": measured_traffic(name), "kernel": kernel}}


# Dominant kernel of each prefill workload (the grid choice of the launcher).
PREFILL_KERNELS = {
    "llama3_8b_long": "fwd_bf16_kernel<128, causal, 4, no key split>",
    "qwen3_0p6b_gqa": "fwd_bf16_kernel<128, causal, 2, key split>",
    "gpt2_small_mha": "fwd_bf16_kernel<64, causal, 1, no key split>",
    "llama3_8b_chunk": "fwd_bf16_kernel<128, causal, 4, no key split> (bottom-right)",
    "gpt2_small_mha_fp8": "fwd_fp8_kernel<64, causal, 1, no key split>",
    "qwen3_0p6b_gqa_fp8": "fwd_fp8_kernel<128, causal, 2, key split>",
    "llama3_8b_long_fp8": "fwd_fp8_kernel<128, causal, 4, no key split>",
}


def run_only(torch, fa, inputs, args):
    """One workload, `steps` timed calls, a one-line JSON summary."""
    if args.calib_copy_mib > 0:
        n = args.calib_copy_mib * (1 << 20) // 4
        a = torch.ones(n, dtype=torch.float32, device="cuda")
        b = torch.empty_like(a)
        torch.cuda.synchronize()
        b.copy_(a)
        torch.cuda.synchronize()
        del a, b
    if args.only.startswith("bwd_"):
        w = inputs.WORKLOADS[args.only[4:]]
        t = backward_case(torch, fa, w, args.steps, args.warmup)
        out = {"workload": "backward, " + w.name,
               "TFLOP/s": round(w.bwd_flops / t["wall_s"] / 1e12, 2), **timing_fields(t),
               "frac_of_mfma_peak": round(w.bwd_flops / (t["mean_ms"] * 1e-3) / 1e12 /
                                          PEAK_BF16_TFLOPS, 4)}
        print(json.dumps(out), flush=True)
        return
    w = inputs.WORKLOADS[args.only]
    if isinstance(w, inputs.Prefill):
        t = prefill_case(torch, fa, w, args.steps, args.warmup)
        peak = PEAK_FP8_TFLOPS if w.dtype == "fp8" else PEAK_BF16_TFLOPS
        out = {"workload": w.name, "TFLOP/s": round(w.flops / t["wall_s"] / 1e12, 2),
               **timing_fields(t),
               "frac_of_mfma_peak": round(w.flops / (t["mean_ms"] * 1e-3) / 1e12 / peak, 4)}
    else:
        res, nbytes, _ = decode_case(torch, fa, w, args.steps, args.warmup, [args.decode_splits])
        t = res[args.decode_splits]
        out = {"workload": w.name, "GB/s": round(nbytes / (t["mean_ms"] * 1e-3) / 1e9, 1),
               "call_us": round(t["mean_ms"] * 1e3, 2), "num_splits": args.decode_splits}
    print(json.dumps(out), flush=True)


def decode_entry(fa, w, res, nbytes, ntok, auto, ceil_gbs, plan, key):
    """JSON block of one decode workload: the automatic split count's
    roofline and, for the bf16 cache, every timed split count."""
    t = res[0]
    gbs = nbytes / (t["mean_ms"] * 1e-3) / 1e9
    blk = {"value": round(nbytes / t["wall_s"] / 1e9, 1), "unit": "GB/s",
           "read_probe_gbs": round(ceil_gbs, 1), "frac_of_read_probe": round(gbs / ceil_gbs, 4),
           "us_per_call": round(t["wall_s"] * 1e6, 2), "call_us_events": round(t["mean_ms"] * 1e3, 2),
           "call_us_median": round(t["median_ms"] * 1e3, 2),
           "call_us_min": round(t["min_ms"] * 1e3, 2),
           "num_splits": auto, "algorithmic_bytes": nbytes, "kv_tokens": ntok,
           "roofline": {"bound": "hbm", "achieved": round(gbs, 1), "peak": PEAK_HBM_GBS,
                        "unit": "GB/s", "frac": round(gbs / PEAK_HBM_GBS, 4),
                        "traffic": measured_traffic(key)}}
    if len(res) > 1:
        sweep = {}
        for ns, ts in res.items():
            if ns == 0:
                continue
            g = nbytes / (ts["mean_ms"] * 1e-3) / 1e9
            sweep[str(ns)] = {"key_ranges": plan(w.B, w.Hq, w.Hkv, w.Tk_max, w.d, ns),
                              "call_us_events": round(ts["mean_ms"] * 1e3, 2),
                              "call_us_median": round(ts["median_ms"] * 1e3, 2),
                              "call_us_min": round(ts["min_ms"] * 1e3, 2),
                              "GB/s": round(g, 1), "frac_of_hbm_peak": round(g / PEAK_HBM_GBS, 4)}
        blk["num_splits_sweep"] = {
            "note": "num_splits is the number of equal key ranges the whole batch's key space "
                    f"(all {w.B} sequences x {w.Hkv} kv heads) is cut into, one workgroup each; "
                    f"the automatic choice ({auto}) is the device's resident workgroup count",
            **sweep}
    return blk


def main():
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--no-extra", action="store_true", help="skip the other workloads")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--decode-splits", type=int, default=0, help="num_splits for decode (0 = library choice)")
    ap.add_argument("--only", choices=sorted(inputs_names()), default=None,
                    help="time one workload only and print its numbers (for profiling runs)")
    ap.add_argument("--calib-copy-mib", type=int, default=0,
                    help="with --only: first run one device-to-device copy of this many MiB "
                         "(the reference kernel for scaling traffic counters)")
    args = ap.parse_args()

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU only: the library has no multi-GPU path "
              "(its kernels compute one GPU's share of a sharded job).",
              file=sys.stderr)
        sys.exit(2)

    import torch
    from exact_tiled_attention_02_amd import fa, inputs
    fa.load()
    torch.cuda.set_device(0)

    if args.only is not None:
        run_only(torch, fa, inputs, args)
        return

    w = inputs.LLAMA3_8B_LONG
    log(f"[bench] {w.name}: warmup {args.warmup}, steps {args.steps}")
    t, blk = prefill_entry(torch, fa, w, "llama3_8b_long", args.steps, args.warmup,
                           PREFILL_KERNELS["llama3_8b_long"])
    roof = dict(blk["roofline"])
    roof.update(timing_fields(t))
    result = {
        "metric": "causal prefill attn TFLOP/s (% MFMA peak); decode HBM GB/s (% peak)",
        "value": blk["value"],
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(t["wall_s"] * 1e3, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": w.name, "B": w.B, "Hq": w.Hq, "Hkv": w.Hkv, "Tq": w.Tq,
                   "Tk": w.Tk, "d": w.d, "causal": w.causal, "parallelism": "none (1 GPU)"},
        "roofline": roof,
    }
    log(f"[bench] headline {blk['value']:.1f} TFLOP/s, kernel {t['mean_ms']:.3f} ms "
        f"(median {t['median_ms']:.3f}, min {t['min_ms']:.3f})")

    if not args.no_extra:
        also = {}
        for name, steps in (("qwen3_0p6b_gqa", 200), ("gpt2_small_mha", 100),
                            ("llama3_8b_chunk", 30), ("gpt2_small_mha_fp8", 100),
                            ("qwen3_0p6b_gqa_fp8", 200), ("llama3_8b_long_fp8", 10)):
            wk = inputs.WORKLOADS[name]
            log(f"[bench] {wk.name}")
            _, also[name] = prefill_entry(torch, fa, wk, name, steps, 10, PREFILL_KERNELS[name])
            log(f"[bench]   {also[name]}")
        for name, steps in (("gpt2_small_mha", 20), ("qwen3_0p6b_gqa", 20), ("llama3_8b_long", 3)):
            wk = inputs.WORKLOADS[name]
            log(f"[bench] backward, {wk.name}")
            tb = backward_case(torch, fa, wk, steps, 2)
            ach = wk.bwd_flops / (tb["mean_ms"] * 1e-3) / 1e12
            also["bwd_" + name] = {"value": round(wk.bwd_flops / tb["wall_s"] / 1e12, 2),
                                   "unit": "TFLOP/s",
                                   "flops": "10*B*Hq*Tq*Tk*d/2 (five products, causal)",
                                   "ms_per_call": round(tb["wall_s"] * 1e3, 4),
                                   "call_ms_events": round(tb["mean_ms"], 4),
                                   "call_ms_median": round(tb["median_ms"], 4),
                                   "call_ms_min": round(tb["min_ms"], 4),
                                   "frac_of_mfma_peak": round(ach / PEAK_BF16_TFLOPS, 4)}
            log(f"[bench]   {also['bwd_' + name]}")
        ceil_gbs = read_ceiling(torch, fa)
        log(f"[bench] read probe (1 GiB streamed once): {ceil_gbs:.1f} GB/s")
        wd = inputs.FLASH_DECODE
        auto = fa.fa_decode_workgroups(wd.B, wd.Hq, wd.Hkv, wd.Tk_max, wd.d, args.decode_splits)
        log(f"[bench] {wd.name}, {auto} key ranges, and a sweep of num_splits")
        splits = [args.decode_splits] + [n for n in (8, 16, 32, 64, 128, 256, 1024)
                                         if n != args.decode_splits]
        res, nbytes, ntok = decode_case(torch, fa, wd, 100, 20, splits)
        res = {(0 if ns == args.decode_splits else ns): r for ns, r in res.items()}
        also["flash_decode"] = decode_entry(fa, wd, res, nbytes, ntok, auto, ceil_gbs,
                                            fa.fa_decode_workgroups, "flash_decode")
        log(f"[bench]   {also['flash_decode']}")
        for key, w8, plan in (("flash_decode_fp8", inputs.FLASH_DECODE_FP8, fa.fa_decode_fp8_workgroups),
                              ("flash_decode_int8", inputs.FLASH_DECODE_INT8, fa.fa_decode_int8_workgroups)):
            a8 = plan(w8.B, w8.Hq, w8.Hkv, w8.Tk_max, w8.d, args.decode_splits)
            log(f"[bench] {w8.name}, {a8} key ranges")
            r8, nb8, nt8 = decode_case(torch, fa, w8, 200, 50, [args.decode_splits])
            r8 = {0: r8[args.decode_splits]}
            also[key] = decode_entry(fa, w8, r8, nb8, nt8, a8, ceil_gbs, plan, key)
            also[key]["speedup_vs_bf16_cache"] = round(res[0]["mean_ms"] / r8[0]["mean_ms"], 3)
            log(f"[bench]   {also[key]}")
        result["also"] = also

    if not args.no_cpu_baseline:
        log("[bench] cpu_baseline: fp64 oracle on a sample of the headline workload")
        result["cpu_baseline"] = cpu_baseline(w)
        log(f"[bench]   {result['cpu_baseline']}")

    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
