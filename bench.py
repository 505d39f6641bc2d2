"""Benchmark of biased paged-attention decode on one MI355X.

Default workload: the large biased decode (256 sequences x 32 heads,
head_dim 128, bf16 q/K/V, fp32 bias [256,32,4096], L ~ U[1024,4096], random
block permutation). One step = one paged_attn_decode call = one decode step of
one attention layer for all 256 sequences; throughput is decode tokens/s
(sequences served per second) and the achieved HBM bandwidth of the call.

Timing: W untimed warm-up steps, further untimed steps until 0.3 s of warm-up
have passed (the GPU's clocks ramp over the first ~0.1 s of load), then exactly
K steps between two HIP events on the stream the library launches on, with a
device synchronisation on both sides. The CPU baseline times the float64
oracle on the same workload (repeated to ~10 s of CPU work).

Prints ONE JSON line. Options:
  --gpus N        only 1 is supported (the path runs on one GPU)
  --steps K       timed steps (default 20)
  --warmup W      untimed warm-up steps (default 5)
  --workload X    large_biased_decode_bf16 (default) | modernbert_prefill_f32 |
                  modernbert_prefill_bf16 | modernbert_chunked_prefill_f32 |
                  modernbert_chunked_prefill_bf16 (one layer, 128-token chunks) |
                  t5_small_self_decode_bf16 | t5_large_cross_decode_bf16 (cold-cache
                  median of single calls) | kv_write_modernbert_f32 | copy_probe (a plain device copy of
                  known size, for calibrating the rocprofv3 byte counters)
  --no-cpu-baseline   skip the oracle timing
  --no-variants       skip the window / chunk / null-bias / no-bias-build variants
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time

import numpy as np
import torch

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import sliding_window_mask_amd as pa  # noqa: E402
import workloads  # noqa: E402

METRIC = "decode tokens/s and achieved HBM GB/s (% of MI355X peak), biased paged attn"
HBM_PEAK_GBPS = 8000.0
FP32_MFMA_PEAK_TFLOPS = 157.3
PROFILES = os.path.join(ROOT, "profiles")


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def source_sha(name):
    p = os.path.join(ROOT, "sliding_window_mask_amd", "csrc", name)
    return hashlib.sha256(open(p, "rb").read()).hexdigest()[:16]


def read_traffic(workload, kernel_src, key="hbm_bytes_per_launch"):
    """HBM bytes (per launch, or the given key) from the committed rocprofv3
    counter summary, if it was taken on the current kernel source; otherwise
    None."""
    path = os.path.join(PROFILES, "%s_traffic.txt" % workload)
    if not os.path.exists(path):
        return None
    kv = {}
    for ln in open(path):
        if "=" in ln and not ln.startswith("#"):
            k, v = ln.split("=", 1)
            kv[k.strip()] = v.strip()
    if kv.get("kernel_source_sha") != source_sha(kernel_src):
        return None
    try:
        return float(kv[key])
    except (KeyError, ValueError):
        return None


SETTLE_S = 0.3     # untimed run time before the timed steps, for the clocks to ramp


def time_steps(fn, steps, warmup):
    """W untimed warmup steps, then more untimed steps until SETTLE_S seconds
    of warmup have passed (an idle MI355X ramps its clocks over the first
    ~0.1 s of sustained work; short steps otherwise get timed at low clock),
    then exactly `steps` timed steps between two events."""
    t0 = time.perf_counter()
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    while time.perf_counter() - t0 < SETTLE_S:
        fn()
        torch.cuda.synchronize()
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    start.record()
    for _ in range(steps):
        fn()
    end.record()
    torch.cuda.synchronize()
    return start.elapsed_time(end) / steps          # ms per step


def per_call_ms(fn, n):
    """Distribution of single-call times (each call between its own pair of
    events, after the timed region): median, p10, p90."""
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(n)]
    for s, e in ev:
        s.record()
        fn()
        e.record()
    torch.cuda.synchronize()
    t = np.array([s.elapsed_time(e) for s, e in ev])
    return {"calls": n, "median": float(np.median(t)), "p10": float(np.percentile(t, 10)),
            "p90": float(np.percentile(t, 90))}


# ----------------------------------------------------------------------------
# decode
# ----------------------------------------------------------------------------
def decode_bytes(lens, H, D, esize, window, with_bias, chunk=0):
    """Algorithmic HBM bytes of one decode call: for every (sequence, head)
    the visible tokens' K and V rows (2*D*e bytes) and bias entries (4 bytes),
    plus the q read and out write (2*D*e). Visible: all L tokens, the W newest
    with a window, or with chunked local attention the query's chunk up to it,
    ((L-1) mod C) + 1 tokens. Block-table and length reads (< 0.1%) are not
    counted."""
    L = lens.astype(np.int64)
    if chunk > 0:
        n_vis = np.where(L > 0, (L - 1) % chunk + 1, 0)
    else:
        n_vis = np.minimum(L, window) if window > 0 else L
    per_tok = 2 * D * esize + (4 if with_bias else 0)
    return int(H * np.sum(n_vis * per_tok + 2 * D * esize))


def compact_sample(case, seqs):
    """Host copies of the inputs of a subset of sequences, with a compact cache
    holding only the blocks they reference (for the oracle)."""
    idx = torch.as_tensor(seqs, dtype=torch.long, device=case.block_tables.device)
    bt = case.block_tables[idx].cpu()
    used = torch.unique(bt)
    remap = torch.full((case.num_blocks,), -1, dtype=torch.int32)
    remap[used] = torch.arange(used.numel(), dtype=torch.int32)
    dev_used = used.to(case.k_cache.device)
    return dict(q=case.q[idx].cpu(), k=case.k_cache[dev_used].cpu(),
                v=case.v_cache[dev_used].cpu(), bt=remap[bt.long()],
                cl=case.context_lens[idx].cpu(),
                bias=None if case.attn_bias is None else case.attn_bias[idx].cpu())


def cpu_baseline_decode(case, out_gpu):
    """Time the float64 oracle (as it stands) on a bounded sample of the same
    workload; also report the GPU-vs-oracle error on that sample."""
    import oracle
    oracle.build(force=False)
    rng = np.random.default_rng(12345)

    target_s = 15.0

    def run(n, min_s=0.0):
        """Oracle on n sequences, repeated (same inputs) until min_s seconds."""
        seqs = np.sort(rng.choice(case.num_seqs, size=n, replace=False))
        s = compact_sample(case, seqs)
        reps, t0 = 0, time.perf_counter()
        while True:
            ref = oracle.decode(s["q"], s["k"], s["v"], s["bt"], s["cl"], s["bias"],
                                case.sliding_window, case.scale, case.max_seq_len)
            reps += 1
            dt = time.perf_counter() - t0
            if dt >= min_s or reps >= 100:
                break
        g = out_gpu[torch.as_tensor(seqs, device=out_gpu.device)].float().cpu().double().numpy()
        return n, reps, dt, float(np.max(np.abs(g - ref)))

    n, _, dt, _ = run(4)                                  # rate estimate
    n = int(min(case.num_seqs, max(4, math.floor(target_s / max(dt / n, 1e-6)))))
    # the whole workload can take well under the target: repeat it, so the
    # rate comes from ~10 s of CPU work
    n, reps, dt, err = run(n, min_s=10.0 if n == case.num_seqs else 0.0)
    threads = oracle.num_threads()
    # the same oracle on one thread, on a smaller sample (~5 s)
    n1 = max(1, min(case.num_seqs, int(5.0 * n * reps / dt / max(threads, 1))))
    oracle.set_num_threads(1)
    try:
        n1, reps1, dt1, _ = run(n1)
    finally:
        oracle.set_num_threads(threads)
    return {"value": n * reps / dt, "unit": "tokens/s", "cores": threads,
            "kind": "oracle",
            "sample": "%d of the %d sequences (all 32 heads, their full contexts), "
                      "float64 C loop over the block table, %d pass(es) in %.1f s"
                      % (n, case.num_seqs, reps, dt),
            "single_thread": {"value": n1 * reps1 / dt1, "unit": "tokens/s", "cores": 1,
                              "sample": "%d sequences, %d pass(es) in %.1f s"
                                        % (n1, reps1, dt1)},
            "gpu_vs_oracle_max_abs_err_on_sample": err}


def bench_decode(args):
    t0 = time.time()
    case = workloads.large_biased_decode_bf16(device="cuda")
    torch.cuda.synchronize()
    log("inputs ready in %.1f s (%d blocks)" % (time.time() - t0, case.num_blocks))
    B, H, D = case.q.shape
    lib = pa.lib()
    out = torch.empty_like(case.q)
    P = lib.pa_decode_default_partition(B, H, D, case.max_seq_len, case.sliding_window)
    ws = lib.workspace_for(case.q, case.max_seq_len, case.sliding_window)

    def step(window=-1, bias="case", which=lib, o=out, w=ws):
        which.paged_attn_decode(case.q, case.k_cache, case.v_cache, case.block_tables,
                                case.context_lens, case.attn_bias if bias == "case" else bias,
                                window, case.scale, max_seq_len=case.max_seq_len, out=o,
                                workspace=w)

    ms = time_steps(step, args.steps, args.warmup)
    nbytes = decode_bytes(case.lens, H, D, 2, -1, True)
    gbps = nbytes / (ms * 1e-3) / 1e9
    tokens_per_s = B / (ms * 1e-3)
    log("decode: %.4f ms/step, %.0f tokens/s, %.1f GB/s" % (ms, tokens_per_s, gbps))
    traffic = read_traffic("decode_large_biased_bf16", "pa_decode.hip")
    line = {
        "metric": METRIC, "value": tokens_per_s, "unit": "tokens/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": ms,
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "large_biased_decode_bf16", "num_seqs": B, "num_heads": H,
                   "head_dim": D, "block_size": 16, "context_lens": "uniform [1024, 4096]",
                   "num_blocks": case.num_blocks, "max_seq_len": case.max_seq_len,
                   "attn_bias": "fp32 [256, 32, 4096] N(0,1)", "sliding_window": -1,
                   "partition_tokens": P, "parallelism": "single GPU"},
        "achieved_GBps": gbps,
        "algorithmic_bytes_per_step": nbytes,
        "roofline": {"bound": "hbm", "achieved": gbps, "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                     "frac": gbps / HBM_PEAK_GBPS,
                     "traffic": traffic,
                     "kernel": "paged_attn_decode call: pa_decode_partition" +
                               ("" if ws is None else " + pa_decode_merge")},
    }
    line["per_call_ms"] = per_call_ms(step, max(args.steps, 20))
    if not args.no_variants:
        var = {}
        msw = time_steps(lambda: step(window=1024), args.steps, args.warmup)
        bw = decode_bytes(case.lens, H, D, 2, 1024, True)
        var["window_1024"] = {"ms_per_step": msw, "tokens_per_s": B / (msw * 1e-3),
                              "GBps": bw / (msw * 1e-3) / 1e9}
        # chunked local attention, 1024-token chunks (the query sees its chunk's
        # first ((L-1) mod 1024) + 1 tokens)
        msc = time_steps(lambda: lib.paged_attn_decode_chunked(
            case.q, case.k_cache, case.v_cache, case.block_tables, case.context_lens,
            case.attn_bias, 1024, case.scale, max_seq_len=case.max_seq_len, out=out),
            args.steps, args.warmup)
        bc = decode_bytes(case.lens, H, D, 2, -1, True, chunk=1024)
        var["chunk_1024"] = {"ms_per_step": msc, "tokens_per_s": B / (msc * 1e-3),
                             "GBps": bc / (msc * 1e-3) / 1e9}
        msn = time_steps(lambda: step(bias=None), args.steps, args.warmup)
        bn = decode_bytes(case.lens, H, D, 2, -1, False)
        var["null_bias"] = {"ms_per_step": msn, "tokens_per_s": B / (msn * 1e-3),
                            "GBps": bn / (msn * 1e-3) / 1e9}
        # the same shape with a T5 bias computed in the kernel (32 buckets,
        # max distance 128) instead of the materialised [256, 32, 4096] stream
        t5_tab = torch.randn(H, 32, device="cuda") * 0.5
        msr = time_steps(lambda: lib.paged_attn_decode_relpos(
            case.q, case.k_cache, case.v_cache, case.block_tables, case.context_lens, t5_tab,
            32, 128, 0, -1, case.scale, max_seq_len=case.max_seq_len, out=out, workspace=ws),
            args.steps, args.warmup)
        var["t5_bias_in_kernel"] = {"ms_per_step": msr, "tokens_per_s": B / (msr * 1e-3),
                                    "GBps": bn / (msr * 1e-3) / 1e9}
        # the same bias values in the packed (unpadded) layout
        Lt = torch.from_numpy(case.lens.astype(np.int64))
        starts = torch.zeros(B, dtype=torch.int64)
        starts[1:] = torch.cumsum(Lt * H, 0)[:-1]
        packed = torch.cat([case.attn_bias[b, :, :int(case.lens[b])].reshape(-1)
                            for b in range(B)]).contiguous()
        starts = starts.to("cuda")
        msg = time_steps(lambda: lib.paged_attn_decode_ragged_bias(
            case.q, case.k_cache, case.v_cache, case.block_tables, case.context_lens, packed,
            starts, -1, case.scale, max_seq_len=case.max_seq_len, out=out, workspace=ws),
            args.steps, args.warmup)
        var["ragged_bias"] = {"ms_per_step": msg, "tokens_per_s": B / (msg * 1e-3),
                              "GBps": nbytes / (msg * 1e-3) / 1e9,
                              "bias_MiB_packed": packed.numel() * 4 / 2**20,
                              "bias_MiB_padded": case.attn_bias.numel() * 4 / 2**20}
        del packed
        if os.path.exists(pa.LIB_NOBIAS_PATH):
            nob = pa.PagedAttnLib(pa.LIB_NOBIAS_PATH)
            msb = time_steps(lambda: step(bias=None, which=nob), args.steps, args.warmup)
            var["null_bias_in_no_bias_build"] = {"ms_per_step": msb,
                                                 "tokens_per_s": B / (msb * 1e-3),
                                                 "GBps": bn / (msb * 1e-3) / 1e9}
            var["null_bias_slowdown_vs_no_bias_build"] = msn / msb - 1.0
        line["variants"] = var
        log("variants: %s" % json.dumps(var))
    if not args.no_cpu_baseline:
        step()
        torch.cuda.synchronize()
        line["cpu_baseline"] = cpu_baseline_decode(case, out)
    return line


# ----------------------------------------------------------------------------
# prefill (12-layer ModernBERT-shaped encoder)
# ----------------------------------------------------------------------------
def prefill_flops(lens, H, D, window, chunk=0):
    """Algorithmic flops of a bidirectional prefill layer: 4*D per visible
    (query, key) pair, every pair of a sequence, |i - j| < W with a window, or
    pairs inside one chunk of C positions with chunked local attention."""
    L = lens.astype(np.int64)
    if chunk > 0:
        full, rem = L // chunk, L % chunk
        return int(4 * D * H * np.sum(full * chunk * chunk + rem * rem))
    if window > 0:
        W = np.minimum(window, L)
        pairs = L * (2 * W - 1) - W * (W - 1)
    else:
        pairs = L * L
    return int(4 * D * H * np.sum(pairs))


BF16_MFMA_PEAK_TFLOPS = 2500.0


def bench_prefill(args, dtype=torch.float32):
    if dtype == torch.float32:
        layers = [workloads.modernbert_prefill_f32(l, device="cuda")
                  for l in range(workloads.MODERNBERT_LAYERS)]
    else:
        layers = [workloads.prefill_case(4, num_seqs=32, num_heads=12, head_dim=64,
                                         lens=(64, 1024), max_seq_len=1024, dtype=dtype,
                                         sliding_window=workloads.modernbert_window(l),
                                         device="cuda", layer_seed=[4, l])
                  for l in range(workloads.MODERNBERT_LAYERS)]
    torch.cuda.synchronize()
    outs = [torch.empty_like(c.q) for c in layers]
    lib = pa.lib()

    def step():
        for c, o in zip(layers, outs):
            lib.paged_attn_prefill(c.q, c.k_cache, c.v_cache, c.block_tables, c.context_lens,
                                   c.query_start_loc, None, c.sliding_window, False, c.scale,
                                   max_seq_len=c.max_seq_len, out=o)

    ms = time_steps(step, args.steps, args.warmup)
    c0 = layers[0]
    flops = sum(prefill_flops(c.lens, 12, 64, c.sliding_window) for c in layers)
    tflops = flops / (ms * 1e-3) / 1e12
    tokens = int(c0.lens.sum())
    peak = FP32_MFMA_PEAK_TFLOPS if dtype == torch.float32 else BF16_MFMA_PEAK_TFLOPS
    tag = "f32" if dtype == torch.float32 else "bf16"
    line = {
        "metric": "encoder prefill tokens/s (12 layers) and MFMA TFLOP/s", "value":
        tokens / (ms * 1e-3), "unit": "tokens/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": ms, "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": tag, "data": "synthetic",
        "config": {"workload": "modernbert_prefill_" + tag, "layers": 12, "num_seqs": 32,
                   "num_heads": 12, "head_dim": 64, "context_lens": "uniform [64, 1024]",
                   "windows": [workloads.modernbert_window(l) for l in range(12)]},
        "roofline": {"bound": "mfma", "achieved": tflops, "peak": peak,
                     "unit": "TFLOP/s", "frac": tflops / peak,
                     # HBM bytes of one step (the 12 launches), from the counters
                     "traffic": read_traffic("modernbert_prefill_" + tag,
                                             "pa_prefill.hip" if tag == "f32"
                                             else "pa_prefill_bf16.hip", "hbm_bytes_per_step"),
                     "kernel": "pa_prefill_%s (12 launches per step)" % tag},
        "algorithmic_flops_per_step": flops,
    }
    return line


def bench_chunked_prefill(args, dtype=torch.float32):
    """One ModernBERT-shaped layer (32 sequences of U[64,1024], 12 heads,
    head_dim 64) with bidirectional chunked local attention in 128-token
    chunks, through paged_attn_prefill_chunked."""
    c = workloads.prefill_case(4, num_seqs=32, num_heads=12, head_dim=64, lens=(64, 1024),
                               max_seq_len=1024, dtype=dtype, device="cuda", layer_seed=[4, 1])
    torch.cuda.synchronize()
    out = torch.empty_like(c.q)
    lib = pa.lib()
    ms = time_steps(lambda: lib.paged_attn_prefill_chunked(
        c.q, c.k_cache, c.v_cache, c.block_tables, c.context_lens, c.query_start_loc, None,
        128, False, c.scale, max_seq_len=c.max_seq_len, out=out), args.steps, args.warmup)
    flops = prefill_flops(c.lens, 12, 64, -1, chunk=128)
    tflops = flops / (ms * 1e-3) / 1e12
    peak = FP32_MFMA_PEAK_TFLOPS if dtype == torch.float32 else BF16_MFMA_PEAK_TFLOPS
    tag = "f32" if dtype == torch.float32 else "bf16"
    return {
        "metric": "chunked-local prefill tokens/s (one layer) and MFMA TFLOP/s",
        "value": int(c.lens.sum()) / (ms * 1e-3), "unit": "tokens/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": ms,
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": tag,
        "data": "synthetic",
        "config": {"workload": "modernbert_chunked_prefill_" + tag, "layers": 1,
                   "num_seqs": 32, "num_heads": 12, "head_dim": 64,
                   "context_lens": "uniform [64, 1024]", "chunk_size": 128},
        "roofline": {"bound": "mfma", "achieved": tflops, "peak": peak, "unit": "TFLOP/s",
                     "frac": tflops / peak, "traffic": None,
                     "kernel": "pa_prefill_%s (banded variant, one launch)" % tag},
        "algorithmic_flops_per_step": flops,
    }


def bench_copy(args):
    """A plain device-to-device copy of known size (256 MiB read + 256 MiB
    written per launch), used to calibrate the rocprofv3 byte counters."""
    n = 256 << 20
    src = torch.empty(n, dtype=torch.uint8, device="cuda").random_(0, 255)
    dst = torch.empty_like(src)
    ms = time_steps(lambda: dst.copy_(src), args.steps, args.warmup)
    return {"metric": "copy probe GB/s", "value": 2 * n / (ms * 1e-3) / 1e9, "unit": "GB/s",
            "bytes_read_per_launch": n, "bytes_written_per_launch": n, "ms_per_step": ms,
            "steps": args.steps, "warmup": args.warmup, "n_gpus": 1}


def bench_small_decode(args, name):
    """T5-shaped decode workloads (small working sets: an L2 + Infinity Cache
    flush precedes every timed call, and each call is timed on its own)."""
    if name == "t5_small_self_decode_bf16":
        case = workloads.t5_small_self_decode_bf16(device="cuda")
    else:
        case = workloads.t5_large_cross_decode_bf16(device="cuda", bias=None)
    B, H, D = case.q.shape
    lib = pa.lib()
    out = torch.empty_like(case.q)
    ws = lib.workspace_for(case.q, case.max_seq_len, case.sliding_window)
    flush = torch.empty(1 << 30, dtype=torch.uint8, device="cuda")

    def call():
        lib.paged_attn_decode(case.q, case.k_cache, case.v_cache, case.block_tables,
                              case.context_lens, case.attn_bias, case.sliding_window,
                              case.scale, max_seq_len=case.max_seq_len, out=out, workspace=ws)

    for _ in range(args.warmup):
        call()
    times = []
    for _ in range(args.steps):
        flush.zero_()
        s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        s.record()
        call()
        e.record()
        torch.cuda.synchronize()
        times.append(s.elapsed_time(e))
    ms = float(np.median(times))
    nbytes = decode_bytes(case.lens, H, D, 2, -1, case.attn_bias is not None)
    extra = {}
    if case.t5_table is not None:
        # the same T5 bias computed in the kernel from the [8, 32] bucket table
        rt = []
        for _ in range(args.steps):
            flush.zero_()
            s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            s.record()
            lib.paged_attn_decode_relpos(case.q, case.k_cache, case.v_cache, case.block_tables,
                                         case.context_lens, case.t5_table, 32, 128, 0, -1,
                                         case.scale, max_seq_len=case.max_seq_len, out=out,
                                         workspace=ws)
            e.record()
            torch.cuda.synchronize()
            rt.append(s.elapsed_time(e))
        mr = float(np.median(rt))
        extra["t5_bias_in_kernel"] = {"ms_per_step": mr, "tokens_per_s": B / (mr * 1e-3),
                                      "GBps": decode_bytes(case.lens, H, D, 2, -1, False) /
                                      (mr * 1e-3) / 1e9}
    gbps = nbytes / (ms * 1e-3) / 1e9
    return {"metric": "decode tokens/s and achieved HBM GB/s (cold caches, median call)",
            "value": B / (ms * 1e-3), "unit": "tokens/s", "n_gpus": 1, "steps": args.steps,
            "warmup": args.warmup, "ms_per_step": ms, "p10_ms": float(np.percentile(times, 10)),
            "p90_ms": float(np.percentile(times, 90)), "higher_is_better": True,
            "scaling": "weak", "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
            "config": {"workload": name, "num_seqs": B, "num_heads": H, "head_dim": D,
                       "partition_tokens": lib.pa_decode_default_partition(
                           B, H, D, case.max_seq_len, -1),
                       "attn_bias": None if case.attn_bias is None else "fp32 (T5 buckets)"},
            "roofline": {"bound": "hbm", "achieved": gbps, "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                         "frac": gbps / HBM_PEAK_GBPS,
                         "traffic": read_traffic(name, "pa_decode.hip"),
                         "kernel": "paged_attn_decode call"},
            "algorithmic_bytes_per_step": nbytes, "variants": extra}


def bench_kv_write(args):
    """KV-cache write of a whole ModernBERT-shaped prompt batch (32 sequences,
    L ~ U[64,1024], 12 heads, D = 64, fp32) into a randomly permuted block
    pool: algorithmic bytes = k_new + v_new read + the same written."""
    case = workloads.modernbert_prefill_f32(0, device="cuda")
    T, H, D = case.q.shape
    L = case.lens
    bt = case.block_tables.cpu()
    slots = torch.cat([bt[b, torch.arange(int(L[b])) // 16].long() * 16 +
                       torch.arange(int(L[b])) % 16 for b in range(case.num_seqs)]).to("cuda")
    kn = torch.randn(T, H, D, device="cuda")
    vn = torch.randn(T, H, D, device="cuda")
    lib = pa.lib()
    ms = time_steps(lambda: lib.paged_kv_write(case.k_cache, case.v_cache, kn, vn, slots),
                    args.steps, args.warmup)
    nbytes = 2 * 2 * T * H * D * 4
    gbps = nbytes / (ms * 1e-3) / 1e9
    return {"metric": "KV-cache write GB/s", "value": gbps, "unit": "GB/s", "n_gpus": 1,
            "steps": args.steps, "warmup": args.warmup, "ms_per_step": ms,
            "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "f32",
            "data": "synthetic",
            "config": {"workload": "kv_write_modernbert_f32", "tokens": T, "num_heads": H,
                       "head_dim": D},
            "roofline": {"bound": "hbm", "achieved": gbps, "peak": HBM_PEAK_GBPS,
                         "unit": "GB/s", "frac": gbps / HBM_PEAK_GBPS,
                         "traffic": read_traffic("kv_write_modernbert_f32", "pa_cache.hip"),
                         "kernel": "pa_kv_write"},
            "algorithmic_bytes_per_step": nbytes}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="large_biased_decode_bf16")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-variants", action="store_true")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py runs on one GPU only: the paged-attention path is measured on a "
              "single MI355X (--gpus 1).", file=sys.stderr)
        sys.exit(2)
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(2)
    if args.workload == "large_biased_decode_bf16":
        line = bench_decode(args)
    elif args.workload == "modernbert_prefill_f32":
        line = bench_prefill(args)
    elif args.workload == "modernbert_prefill_bf16":
        line = bench_prefill(args, torch.bfloat16)
    elif args.workload == "modernbert_chunked_prefill_f32":
        line = bench_chunked_prefill(args)
    elif args.workload == "modernbert_chunked_prefill_bf16":
        line = bench_chunked_prefill(args, torch.bfloat16)
    elif args.workload in ("t5_small_self_decode_bf16", "t5_large_cross_decode_bf16"):
        line = bench_small_decode(args, args.workload)
    elif args.workload == "kv_write_modernbert_f32":
        line = bench_kv_write(args)
    elif args.workload == "copy_probe":
        line = bench_copy(args)
    else:
        raise SystemExit("unknown workload %s" % args.workload)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
