"""Benchmark of biased paged-attention decode on one MI355X.

Default workload: the large biased decode (256 sequences x 32 heads,
head_dim 128, bf16 q/K/V, fp32 bias [256,32,4096], L ~ U[1024,4096], random
block permutation). One step = one paged_attn_decode call = one decode step of
one attention layer for all 256 sequences; throughput is decode tokens/s
(sequences served per second) and the achieved HBM bandwidth of the call.

The default run also measures the other workloads of the path and reports each
as an entry of "configs" in the same line: T5-small self-attention decode and
T5-large cross-attention decode (back-to-back calls over rotating copies of
their inputs, so that every call reads from HBM), and the
12-layer ModernBERT-shaped encoder prefill in fp32 and in bf16. Every entry
carries its time per step, its roofline fraction and its own CPU baseline.

Timing: W untimed warm-up steps, further untimed steps until 0.3 s of warm-up
have passed (the GPU's clocks ramp over the first ~0.1 s of load), then exactly
K steps between two HIP events on the stream the library launches on, with a
device synchronisation on both sides. The CPU baseline times the float64
oracle, as it stands, on a bounded sample of the same inputs, at all the
threads it gets and at one thread, and names the host CPU.

Prints ONE JSON line. Options:
  --gpus N        only 1 is supported (the path runs on one GPU)
  --steps K       timed steps (default 20)
  --warmup W      untimed warm-up steps (default 5)
  --workload X    large_biased_decode_bf16 (default) | modernbert_prefill_f32 |
                  modernbert_prefill_bf16 | modernbert_chunked_prefill_f32 |
                  modernbert_chunked_prefill_bf16 (one layer, 128-token chunks) |
                  t5_small_self_decode_bf16 | t5_large_cross_decode_bf16 (calls rotating
                  over input copies > 1 GiB) | kv_write_modernbert_f32 | copy_probe (a plain
                  device copy of known size, for calibrating the rocprofv3 byte counters) |
                  prefill_layer (one layer: --layer-dtype, --layer-window, --layer-causal) |
                  prefill_window_sweep | probe_mfma | probe_lds | probe_stream |
                  probe_gather | probe_gather_t5 | probe_bias | probe_mix | probe_valu | probe_clock (hardware rates from
                  bench_probes.hip: matrix instructions, LDS reads, a streaming read, the
                  decode's K/V gather without arithmetic)
  --no-cpu-baseline   skip the oracle timing
  --no-variants       skip the window / chunk / null-bias / no-bias-build variants
  --no-configs        default workload only: skip the other workloads' entries
  --profile-run       warm-up, settle and the K timed steps only, nothing after them
                      (no variants, single-call timings or baselines): under
                      rocprofv3 the last K steps' dispatches are the timed ones
  --write-profiles X  write profiles/X_kernel_trace.md and profiles/X_traffic.txt
                      from rocprofv3 output of --profile-run runs of workload X
                      (see write_profiles for the arguments)
"""
from __future__ import annotations

import argparse
import csv
import glob
import hashlib
import json
import math
import os
import statistics
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "decode tokens/s and achieved HBM GB/s (% of MI355X peak), biased paged attn"
HBM_PEAK_GBPS = 8000.0
FP32_MFMA_PEAK_TFLOPS = 157.3
BF16_MFMA_PEAK_TFLOPS = 2500.0
PROFILES = os.path.join(ROOT, "profiles")

# kernel source each workload's dominant kernels are built from
KERNEL_SOURCE = {
    "large_biased_decode_bf16": "pa_decode.hip",
    "t5_small_self_decode_bf16": "pa_decode.hip",
    "t5_large_cross_decode_bf16": "pa_decode.hip",
    "modernbert_prefill_f32": ("pa_prefill.hip", "pa_prefill_f32x3.hip"),
    "modernbert_prefill_bf16": "pa_prefill_bf16.hip",
    "kv_write_modernbert_f32": "pa_cache.hip",
    "prefill_layer_f32": ("pa_prefill.hip", "pa_prefill_f32x3.hip"),
    "prefill_layer_bf16": "pa_prefill_bf16.hip",
}


def kernel_source_of(wl):
    """Kernel sources of a workload; `<workload>_w<W>` names one window of it
    and `<workload>_causal` its causal form."""
    if wl in KERNEL_SOURCE:
        return KERNEL_SOURCE[wl]
    if wl.endswith("_causal"):
        return kernel_source_of(wl[:-len("_causal")])
    return KERNEL_SOURCE[wl.rsplit("_w", 1)[0]]


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def source_sha(names):
    """First 16 hex digits of the sha256 of a kernel source file, or of the
    concatenation of several (a tuple of names)."""
    if isinstance(names, str):
        names = (names,)
    h = hashlib.sha256()
    for name in names:
        h.update(open(os.path.join(ROOT, "sliding_window_mask_amd", "csrc", name), "rb").read())
    return h.hexdigest()[:16]


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


def cpu_model():
    """Model name of the host CPU: lscpu's "Model name", else /proc/cpuinfo's."""
    import subprocess
    try:
        out = subprocess.run(["lscpu"], capture_output=True, text=True, timeout=10).stdout
        for ln in out.splitlines():
            if ln.strip().lower().startswith("model name"):
                return ln.split(":", 1)[1].strip()
    except (OSError, subprocess.SubprocessError):
        pass
    try:
        for ln in open("/proc/cpuinfo"):
            if ln.lower().startswith("model name"):
                return ln.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


SETTLE_S = 0.3     # untimed run time before the timed steps, for the clocks to ramp


def time_steps(fn, steps, warmup):
    """W untimed warmup steps, then more untimed steps until SETTLE_S seconds
    of warmup have passed (an idle MI355X ramps its clocks over the first
    ~0.1 s of sustained work; short steps otherwise get timed at low clock),
    then exactly `steps` timed steps between two events."""
    import torch
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
    import torch
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


def cold_call_times(fn, steps, warmup, flush):
    """Single calls after an L2 + Infinity Cache flush (a 1 GiB write, outside
    the timed interval), each between its own pair of events."""
    import torch
    for _ in range(warmup):
        fn()
    times = []
    for _ in range(steps):
        flush.zero_()
        s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        s.record()
        fn()
        e.record()
        torch.cuda.synchronize()
        times.append(s.elapsed_time(e))
    return times


# ----------------------------------------------------------------------------
# algorithmic work
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


def prefill_flops(lens, H, D, window, chunk=0, causal=False):
    """Algorithmic flops of a prefill layer: 4*D per visible (query, key)
    pair, every pair of a sequence, |i - j| < W with a window, or pairs inside
    one chunk of C positions with chunked local attention; causal (without a
    window or chunks): the pairs j <= i."""
    L = lens.astype(np.int64)
    if causal:
        assert window <= 0 and chunk <= 0
        return int(4 * D * H * np.sum(L * (L + 1) // 2))
    if chunk > 0:
        full, rem = L // chunk, L % chunk
        return int(4 * D * H * np.sum(full * chunk * chunk + rem * rem))
    if window > 0:
        W = np.minimum(window, L)
        pairs = L * (2 * W - 1) - W * (W - 1)
    else:
        pairs = L * L
    return int(4 * D * H * np.sum(pairs))


def prefill_bytes(lens, H, D, esize):
    """Algorithmic HBM bytes of an encoder prefill layer: q, K and V read once
    and out written once over the valid tokens."""
    return int(4 * int(np.sum(lens.astype(np.int64))) * H * D * esize)


# ----------------------------------------------------------------------------
# the oracle beside the GPU
# ----------------------------------------------------------------------------
def _sample_rates(prepare, n_total, target_s, single_s, describe):
    """Time the oracle as it stands. `prepare(seqs)` makes host copies of the
    inputs of the sequences `seqs` (not timed) and returns a function that
    runs the oracle on them and returns (units of work, max |gpu - oracle|).
    A one-sequence run estimates the cost, the sample is sized to ~target_s of
    oracle time at the oracle's thread count (the whole workload, repeated on
    the same inputs, when it takes less), then at one thread to ~single_s."""
    import oracle
    oracle.build(force=False)
    rng = np.random.default_rng(12345)

    def size_for(sec, per_seq):
        return int(min(n_total, max(1, math.floor(sec / max(per_seq, 1e-9)))))

    def go(n, min_s):
        seqs = np.sort(rng.choice(n_total, size=n, replace=False))
        run = prepare(seqs)
        reps, units, err, dt = 0, 0, 0.0, 0.0
        while True:
            t0 = time.perf_counter()
            u, e = run()
            dt += time.perf_counter() - t0
            units, err, reps = units + u, max(err, e), reps + 1
            if dt >= min_s or reps >= 1000:
                return n, reps, units, dt, err

    _, _, _, dt, _ = go(1, 0.0)
    n = size_for(target_s, dt)
    n, reps, units, dt, err = go(n, target_s if n == n_total else 0.0)
    threads = oracle.num_threads()
    oracle.set_num_threads(1)
    try:
        _, _, _, dt1, _ = go(1, 0.0)
        n1 = size_for(single_s, dt1)
        n1, reps1, units1, dt1, _ = go(n1, single_s if n1 == n_total else 0.0)
    finally:
        oracle.set_num_threads(threads)
    return {"value": units / dt, "cores": threads, "kind": "oracle",
            "cpu_model": cpu_model(), "host_logical_cpus": os.cpu_count(),
            "sample": "%s; %d of the %d sequences, %d pass(es), %.1f s of oracle time "
                      "(host copies of the inputs made beforehand, not timed)"
                      % (describe, n, n_total, reps, dt),
            "single_thread": {"value": units1 / dt1, "cores": 1,
                              "sample": "%d sequences, %d pass(es), %.1f s"
                                        % (n1, reps1, dt1)},
            "gpu_vs_oracle_max_abs_err_on_sample": err}


def compact_decode_sample(case, seqs):
    """Host copies of the inputs of a subset of sequences, with a compact cache
    holding only the blocks they reference (for the oracle)."""
    import torch
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


def cpu_baseline_decode(case, out_gpu, target_s=10.0, single_s=5.0):
    """The float64 oracle (as it stands) on a bounded sample of a decode
    workload's sequences (all heads, whole contexts); the rate is decode
    tokens/s (sequences per second), like the GPU line."""
    import torch
    import oracle

    def prepare(seqs):
        s = compact_decode_sample(case, seqs)
        g = out_gpu[torch.as_tensor(seqs, device=out_gpu.device)].float().cpu().double().numpy()

        def run():
            ref = oracle.decode(s["q"], s["k"], s["v"], s["bt"], s["cl"], s["bias"],
                                case.sliding_window, case.scale, case.max_seq_len)
            return len(seqs), float(np.max(np.abs(g - ref)))
        return run

    r = _sample_rates(prepare, case.num_seqs, target_s, single_s,
                      "float64 C loop over the block table, all %d heads and whole contexts"
                      % case.num_heads)
    r["unit"] = r["single_thread"]["unit"] = "tokens/s"
    return r


def cpu_baseline_prefill(layers, outs, target_s=8.0, single_s=4.0):
    """The float64 oracle on a bounded sample of the encoder batch: every
    layer of the step for the sampled sequences (all heads, all queries); the
    rate is tokens through the 12 layers per second, like the GPU line."""
    import torch
    import oracle
    qsl = layers[0].query_start_loc.cpu()

    def prepare(seqs):
        rows = torch.cat([torch.arange(int(qsl[s]), int(qsl[s + 1])) for s in seqs])
        nq = torch.tensor([int(qsl[s + 1] - qsl[s]) for s in seqs], dtype=torch.int32)
        new_qsl = torch.zeros(len(seqs) + 1, dtype=torch.int32)
        new_qsl[1:] = torch.cumsum(nq, 0)
        idx = torch.as_tensor(seqs, dtype=torch.long)
        host = []
        for c, o in zip(layers, outs):
            bt = c.block_tables.cpu()[idx]
            used = torch.unique(bt)
            remap = torch.full((c.num_blocks,), -1, dtype=torch.int32)
            remap[used] = torch.arange(used.numel(), dtype=torch.int32)
            dev_used = used.to(c.k_cache.device)
            host.append((c, c.q[rows.to(c.q.device)].cpu(), c.k_cache[dev_used].cpu(),
                         c.v_cache[dev_used].cpu(), remap[bt.long()], c.context_lens.cpu()[idx],
                         o[rows.to(o.device)].float().cpu().double().numpy()))

        def run():
            err = 0.0
            for c, q, k, v, bt, cl, g in host:
                ref = oracle.prefill(q, k, v, bt, cl, new_qsl, None, c.sliding_window, 0,
                                     c.scale, c.max_seq_len)
                err = max(err, float(np.max(np.abs(g - ref))) if g.size else 0.0)
            return int(nq.sum()), err
        return run

    r = _sample_rates(prepare, layers[0].num_seqs, target_s, single_s,
                      "float64 C loop over the block table, all %d layers, heads and queries "
                      "of each sampled sequence" % len(layers))
    r["unit"] = r["single_thread"]["unit"] = "tokens/s (12 layers)"
    return r


def _line(metric, value, unit, ms, args, dtype, config, **extra):
    d = {"metric": metric, "value": value, "unit": unit, "n_gpus": 1, "steps": args.steps,
         "warmup": args.warmup, "ms_per_step": ms, "higher_is_better": True,
         "scaling": "weak", "vs_baseline": None, "dtype": dtype, "data": "synthetic",
         "config": config}
    d.update(extra)
    return d


# ----------------------------------------------------------------------------
# decode
# ----------------------------------------------------------------------------
def bench_decode(args):
    import torch
    import sliding_window_mask_amd as pa
    import workloads
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
    traffic = read_traffic("large_biased_decode_bf16", "pa_decode.hip")
    line = _line(
        METRIC, tokens_per_s, "tokens/s", ms, args, "bf16",
        {"workload": "large_biased_decode_bf16", "num_seqs": B, "num_heads": H,
         "head_dim": D, "block_size": 16, "context_lens": "uniform [1024, 4096]",
         "num_blocks": case.num_blocks, "max_seq_len": case.max_seq_len,
         "attn_bias": "fp32 [256, 32, 4096] N(0,1)", "sliding_window": -1,
         "partition_tokens": P, "parallelism": "single GPU"},
        achieved_GBps=gbps, algorithmic_bytes_per_step=nbytes,
        launches_per_step=1 if ws is None else 2,
        roofline={"bound": "hbm", "achieved": gbps, "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                  "frac": gbps / HBM_PEAK_GBPS, "traffic": traffic,
                  "kernel": "paged_attn_decode call: pa_decode_partition" +
                            ("" if ws is None else " + pa_decode_merge")})
    if args.profile_run:
        return line
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
        t5_tab = torch.randn(H, 32, device="cuda",
                             generator=torch.Generator(device="cuda").manual_seed(5)) * 0.5
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


def bench_small_decode(args, name):
    """T5-shaped decode workloads. Their working sets (38 and 339 MB) would
    sit in the caches if one call were repeated, so the timed steps rotate
    over copies of the inputs totalling over 1 GiB (as the layers of a decode
    step do); the single-call time after a cache flush is reported beside."""
    import torch
    import sliding_window_mask_amd as pa
    import workloads
    if name == "t5_small_self_decode_bf16":
        case = workloads.t5_small_self_decode_bf16(device="cuda")
    else:
        case = workloads.t5_large_cross_decode_bf16(device="cuda", bias=None)
    B, H, D = case.q.shape
    lib = pa.lib()
    out = torch.empty_like(case.q)
    ws = lib.workspace_for(case.q, case.max_seq_len, case.sliding_window)
    flush = torch.empty(1 << 30, dtype=torch.uint8, device="cuda")

    def call(bias="case", o=out):
        lib.paged_attn_decode(case.q, case.k_cache, case.v_cache, case.block_tables,
                              case.context_lens, case.attn_bias if bias == "case" else bias,
                              case.sliding_window, case.scale, max_seq_len=case.max_seq_len,
                              out=o, workspace=ws)

    # The timed steps: back-to-back calls as in a decode step over many layers,
    # each call reading its own copy of q, K, V (and bias) while the layers
    # share the block tables and lengths. The copies total over 1 GiB, so no
    # call finds its data in the 256 MB Infinity Cache or the L2s.
    per_copy = sum(t.numel() * t.element_size() for t in
                   (case.q, case.k_cache, case.v_cache, case.attn_bias) if t is not None)
    ncopy = max(4, -(-(1 << 30) // per_copy))
    layers = [(case.q.clone(), case.k_cache.clone(), case.v_cache.clone(),
               None if case.attn_bias is None else case.attn_bias.clone(),
               torch.empty_like(out)) for _ in range(ncopy)]

    def rotating_ms(fn):
        """ms per call of fn(q, k, v, bias, out) over the copies in turn. The
        K calls (a ~10-60 us kernel each, shorter than the binding's host
        work per call) are captured once in a HIP graph and the graph is
        replayed, as a serving loop would launch them; a replay's outputs are
        checked bit for bit against eager calls."""
        if args.profile_run:
            # under a profiler the calls are launched one by one (no graph):
            # the kernels are the same, the host launch gaps are not timed
            it = [0]

            def step():
                fn(*layers[it[0] % ncopy])
                it[0] += 1
            return time_steps(step, args.steps, args.warmup)
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            for c in layers:
                fn(*c)
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        eager = [c[4].clone() for c in layers[:min(args.steps, ncopy)]]
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for i in range(args.steps):
                fn(*layers[i % ncopy])

        def check():
            for i, e in enumerate(eager):
                if not torch.equal(layers[i][4].view(torch.int16), e.view(torch.int16)):
                    raise RuntimeError("graph replay differs from the eager call")
        for c in layers:
            c[4].zero_()
        g.replay()
        torch.cuda.synchronize()
        check()
        t = time_steps(g.replay, 1, args.warmup) / args.steps
        if not args.profile_run:
            check()                      # the last of the timed replays
        return t

    ms = rotating_ms(lambda q, k, v, bias, o: lib.paged_attn_decode(
        q, k, v, case.block_tables, case.context_lens, bias, case.sliding_window, case.scale,
        max_seq_len=case.max_seq_len, out=o, workspace=ws))
    with_bias = case.attn_bias is not None
    nbytes = decode_bytes(case.lens, H, D, 2, -1, with_bias)
    gbps = nbytes / (ms * 1e-3) / 1e9
    if name == "t5_small_self_decode_bf16":
        cfg = {"workload": name, "config": "T5-small-shaped decoder self-attention decode",
               "num_seqs": B, "num_heads": H, "head_dim": D, "context_lens": "uniform [32, 512]",
               "attn_bias": "fp32 [64, 8, 512] materialised from a 32-bucket T5 table "
                            "(max distance 128)"}
    else:
        cfg = {"workload": name, "config": "T5-large-shaped cross-attention decode",
               "num_seqs": B, "num_heads": H, "head_dim": D,
               "context_lens": "encoder lengths uniform [128, 512], separate cross table",
               "attn_bias": "null (and a zero bias, bit-identical)"}
    cfg["partition_tokens"] = lib.pa_decode_default_partition(B, H, D, case.max_seq_len, -1)
    line = _line("decode tokens/s and achieved HBM GB/s (cold caches)",
                 B / (ms * 1e-3), "tokens/s", ms, args, "bf16", cfg,
                 timing="%d back-to-back calls (one HIP graph, replayed) between two "
                        "events, rotating over %d copies of q, K, V and bias (%.0f MB each, "
                        "as the layers of a decode step sharing block tables and lengths): "
                        "every call reads from HBM" % (args.steps, ncopy, per_copy / 1e6),
                 algorithmic_bytes_per_step=nbytes, launches_per_step=1 if ws is None else 2,
                 roofline={"bound": "hbm", "achieved": gbps, "peak": HBM_PEAK_GBPS,
                           "unit": "GB/s", "frac": gbps / HBM_PEAK_GBPS,
                           "traffic": read_traffic(name, "pa_decode.hip"),
                           "kernel": "paged_attn_decode call"})
    if args.profile_run:
        return line
    times = cold_call_times(call, args.steps, args.warmup, flush)
    line["single_call_cold_ms"] = {
        "median": float(np.median(times)), "p10": float(np.percentile(times, 10)),
        "p90": float(np.percentile(times, 90)),
        "timing": "one call between its own pair of events after a 1 GiB cache flush "
                  "(includes the per-call event and launch overhead)"}
    extra = {}
    if case.t5_table is not None:
        # the same T5 bias computed in the kernel from the [8, 32] bucket table
        mr = rotating_ms(lambda q, k, v, bias, o: lib.paged_attn_decode_relpos(
            q, k, v, case.block_tables, case.context_lens, case.t5_table, 32, 128, 0, -1,
            case.scale, max_seq_len=case.max_seq_len, out=o, workspace=ws))
        extra["t5_bias_in_kernel"] = {"ms_per_step": mr, "tokens_per_s": B / (mr * 1e-3),
                                      "GBps": decode_bytes(case.lens, H, D, 2, -1, False) /
                                      (mr * 1e-3) / 1e9}
    else:
        # the zero-bias run of the cross-attention workload: identical output
        zero = torch.zeros(B, H, case.max_seq_len, device="cuda")
        out_zero = torch.empty_like(out)
        mz = rotating_ms(lambda q, k, v, bias, o: lib.paged_attn_decode(
            q, k, v, case.block_tables, case.context_lens, zero, case.sliding_window,
            case.scale, max_seq_len=case.max_seq_len, out=o, workspace=ws))
        call(bias=zero, o=out_zero)
        call()
        torch.cuda.synchronize()
        extra["zero_bias"] = {"ms_per_step": mz, "tokens_per_s": B / (mz * 1e-3),
                              "GBps": decode_bytes(case.lens, H, D, 2, -1, True) /
                              (mz * 1e-3) / 1e9,
                              "bit_identical_to_null_bias": bool(torch.equal(
                                  out.view(torch.int16), out_zero.view(torch.int16)))}
    line["variants"] = extra
    del layers
    if not args.no_cpu_baseline:
        call()
        torch.cuda.synchronize()
        line["cpu_baseline"] = cpu_baseline_decode(case, out, target_s=6.0, single_s=3.0)
    return line


# ----------------------------------------------------------------------------
# prefill (12-layer ModernBERT-shaped encoder)
# ----------------------------------------------------------------------------
def modernbert_layers(dtype):
    import workloads
    return [workloads.prefill_case(4, num_seqs=32, num_heads=12, head_dim=64,
                                   lens=(64, 1024), max_seq_len=1024, dtype=dtype,
                                   sliding_window=workloads.modernbert_window(l),
                                   device="cuda", layer_seed=[4, l])
            for l in range(workloads.MODERNBERT_LAYERS)]


def bench_prefill(args, dtype_name="f32"):
    import torch
    import sliding_window_mask_amd as pa
    import workloads
    dtype = torch.float32 if dtype_name == "f32" else torch.bfloat16
    layers = modernbert_layers(dtype)
    torch.cuda.synchronize()
    outs = [torch.empty_like(c.q) for c in layers]
    lib = pa.lib()

    def run_layer(c, o, bias=None):
        lib.paged_attn_prefill(c.q, c.k_cache, c.v_cache, c.block_tables, c.context_lens,
                               c.query_start_loc, bias, c.sliding_window, False, c.scale,
                               max_seq_len=c.max_seq_len, out=o)

    def step():
        for c, o in zip(layers, outs):
            run_layer(c, o)

    ms = time_steps(step, args.steps, args.warmup)
    c0 = layers[0]
    esize = 4 if dtype_name == "f32" else 2
    flops = sum(prefill_flops(c.lens, 12, 64, c.sliding_window) for c in layers)
    nbytes = sum(prefill_bytes(c.lens, 12, 64, esize) for c in layers)
    tflops = flops / (ms * 1e-3) / 1e12
    tokens = int(c0.lens.sum())
    peak = FP32_MFMA_PEAK_TFLOPS if dtype_name == "f32" else BF16_MFMA_PEAK_TFLOPS
    wl = "modernbert_prefill_" + dtype_name
    line = _line(
        "encoder prefill tokens/s (12 layers) and MFMA TFLOP/s", tokens / (ms * 1e-3),
        "tokens/s", ms, args, dtype_name,
        {"workload": wl,
         "config": "ModernBERT-base-shaped encoder-only bidirectional prefill" +
                   ("" if dtype_name == "f32" else " (bf16 variant)"),
         "layers": 12, "num_seqs": 32, "num_heads": 12, "head_dim": 64,
         "context_lens": "uniform [64, 1024]", "attn_bias": None,
         "windows": [workloads.modernbert_window(l) for l in range(12)]},
        algorithmic_flops_per_step=flops, algorithmic_bytes_per_step=nbytes,
        launches_per_step=len(layers),
        roofline={"bound": "mfma", "achieved": tflops, "peak": peak, "unit": "TFLOP/s",
                  "frac": tflops / peak,
                  # HBM bytes of one step (the 12 launches), from the counters
                  "traffic": read_traffic(wl, KERNEL_SOURCE[wl], "hbm_bytes_per_step"),
                  "kernel": ("pa_prefill_f32x3 (4 full-attention launches) + "
                             "pa_prefill_f32x3_band (8 window-64 launches), both with fp32 "
                             "operands split into three bf16 parts on "
                             "v_mfma_f32_16x16x32_bf16; achieved and peak count fp32 flops"
                             if dtype_name == "f32" else
                             "pa_prefill_bf16_32 (4 full-attention launches) + pa_prefill_bf16 "
                             "(8 window-64 launches)")})
    if args.profile_run:
        return line
    # per layer kind, and one full-attention layer with a materialised bias
    full = [i for i, c in enumerate(layers) if c.sliding_window < 0]
    win = [i for i, c in enumerate(layers) if c.sliding_window > 0]
    var = {}
    for kind, ids in (("full_attention_layer", full), ("window_64_layer", win)):
        c, o = layers[ids[0]], outs[ids[0]]
        msl = time_steps(lambda: run_layer(c, o), args.steps, args.warmup)
        fl = prefill_flops(c.lens, 12, 64, c.sliding_window)
        by = prefill_bytes(c.lens, 12, 64, esize)
        var[kind] = {"ms_per_layer": msl, "TFLOPs": fl / (msl * 1e-3) / 1e12,
                     "mfma_frac": fl / (msl * 1e-3) / 1e12 / peak,
                     "GBps": by / (msl * 1e-3) / 1e9,
                     "hbm_frac": by / (msl * 1e-3) / 1e9 / HBM_PEAK_GBPS}
        if dtype_name == "f32" and kind == "window_64_layer":
            var[kind]["kernel"] = "pa_prefill_f32x3_band (v_mfma_f32_16x16x32_bf16, split operands)"
        if dtype_name == "f32" and kind == "full_attention_layer":
            # these launches run on the bf16 matrix cores, six bf16 products
            # per fp32 product (operands split into three bf16 parts)
            var[kind]["kernel"] = "pa_prefill_f32x3 (v_mfma_f32_16x16x32_bf16, split operands)"
            var[kind]["bf16_mfma_TFLOPs_executed"] = 6 * fl / (msl * 1e-3) / 1e12
            var[kind]["bf16_mfma_frac_executed"] = 6 * fl / (msl * 1e-3) / 1e12 / \
                BF16_MFMA_PEAK_TFLOPS
    c, o = layers[full[0]], outs[full[0]]
    bias = torch.randn(c.num_seqs, 12, c.max_seq_len, c.max_seq_len, device="cuda",
                       generator=torch.Generator(device="cuda").manual_seed(12))
    msb = time_steps(lambda: run_layer(c, o, bias), args.steps, args.warmup)
    fl = prefill_flops(c.lens, 12, 64, -1)
    bias_bytes = 4 * 12 * int(np.sum(c.lens.astype(np.int64) ** 2))
    var["full_attention_layer_with_bias"] = {
        "ms_per_layer": msb, "TFLOPs": fl / (msb * 1e-3) / 1e12,
        "attn_bias": "fp32 [32, 12, 1024, 1024] N(0,1), %d visible entries read"
                     % (bias_bytes // 4),
        "bias_GBps": bias_bytes / (msb * 1e-3) / 1e9,
        "slowdown_vs_no_bias": msb / var["full_attention_layer"]["ms_per_layer"] - 1.0}
    # the same bias under a causal mask (a T5 decoder's prompt with a
    # materialised bias): only the entries j <= i are read
    mscb = time_steps(lambda: lib.paged_attn_prefill(
        c.q, c.k_cache, c.v_cache, c.block_tables, c.context_lens, c.query_start_loc, bias, -1,
        True, c.scale, max_seq_len=c.max_seq_len, out=o), args.steps, args.warmup)
    cbias_bytes = 4 * 12 * int(np.sum(c.lens.astype(np.int64) * (c.lens + 1) // 2))
    var["causal_layer_with_bias"] = {
        "ms_per_layer": mscb,
        "TFLOPs": prefill_flops(c.lens, 12, 64, -1, causal=True) / (mscb * 1e-3) / 1e12,
        "bias_GBps": cbias_bytes / (mscb * 1e-3) / 1e9}
    # a window-64 layer with the same bias (sliding window and bias together):
    # only the entries |i - j| < 64 are read
    cw, ow = layers[win[0]], outs[win[0]]
    mswb = time_steps(lambda: run_layer(cw, ow, bias), args.steps, args.warmup)
    fw = prefill_flops(cw.lens, 12, 64, cw.sliding_window)
    wpairs = fw // (4 * 64 * 12)   # visible (query, key) pairs per head
    var["window_64_layer_with_bias"] = {
        "ms_per_layer": mswb, "TFLOPs": fw / (mswb * 1e-3) / 1e12,
        "bias_GBps": 4 * 12 * wpairs / (mswb * 1e-3) / 1e9,
        "slowdown_vs_no_bias": mswb / var["window_64_layer"]["ms_per_layer"] - 1.0}
    del bias
    # the same layer under a causal mask (decoder-style prefill: the queries
    # see the keys at or before their own position)
    msc = time_steps(lambda: lib.paged_attn_prefill(
        c.q, c.k_cache, c.v_cache, c.block_tables, c.context_lens, c.query_start_loc, None, -1,
        True, c.scale, max_seq_len=c.max_seq_len, out=o), args.steps, args.warmup)
    flc = prefill_flops(c.lens, 12, 64, -1, causal=True)
    var["causal_layer"] = {
        "ms_per_layer": msc, "TFLOPs": flc / (msc * 1e-3) / 1e12,
        "mfma_frac": flc / (msc * 1e-3) / 1e12 / peak,
        "kernel": "pa_prefill_f32x3_band (causal)" if dtype_name == "f32" else
                  "pa_prefill_bf16_32 (32x32x16, causal)"}
    # and with the in-kernel T5 bias of a decoder (32 buckets, max distance
    # 128, one direction): a T5 decoder's prompt
    t5_tab = torch.randn(12, 32, device="cuda",
                         generator=torch.Generator(device="cuda").manual_seed(5)) * 0.5
    mst = time_steps(lambda: lib.paged_attn_prefill_relpos(
        c.q, c.k_cache, c.v_cache, c.block_tables, c.context_lens, c.query_start_loc, t5_tab,
        32, 128, 0, -1, True, c.scale, max_seq_len=c.max_seq_len, out=o), args.steps, args.warmup)
    var["causal_layer_t5_bias"] = {
        "ms_per_layer": mst, "TFLOPs": flc / (mst * 1e-3) / 1e12,
        "slowdown_vs_causal_no_bias": mst / msc - 1.0,
        "t5_bias": "[12, 32] N(0, 0.25) bucket table, unidirectional, max distance 128"}
    line["variants"] = var
    if not args.no_cpu_baseline:
        step()
        torch.cuda.synchronize()
        line["cpu_baseline"] = cpu_baseline_prefill(layers, outs)
    return line


def bench_chunked_prefill(args, dtype_name="f32"):
    """One ModernBERT-shaped layer (32 sequences of U[64,1024], 12 heads,
    head_dim 64) with bidirectional chunked local attention in 128-token
    chunks, through paged_attn_prefill_chunked."""
    import torch
    import sliding_window_mask_amd as pa
    import workloads
    dtype = torch.float32 if dtype_name == "f32" else torch.bfloat16
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
    peak = FP32_MFMA_PEAK_TFLOPS if dtype_name == "f32" else BF16_MFMA_PEAK_TFLOPS
    return _line("chunked-local prefill tokens/s (one layer) and MFMA TFLOP/s",
                 int(c.lens.sum()) / (ms * 1e-3), "tokens/s", ms, args, dtype_name,
                 {"workload": "modernbert_chunked_prefill_" + dtype_name, "layers": 1,
                  "num_seqs": 32, "num_heads": 12, "head_dim": 64,
                  "context_lens": "uniform [64, 1024]", "chunk_size": 128},
                 launches_per_step=1, algorithmic_flops_per_step=flops,
                 roofline={"bound": "mfma", "achieved": tflops, "peak": peak,
                           "unit": "TFLOP/s", "frac": tflops / peak, "traffic": None,
                           "kernel": "pa_prefill_f32x3_band (one launch, split bf16 operands)"
                           if dtype_name == "f32" else "pa_prefill_bf16 (banded variant, one launch)"})


def bench_copy(args):
    """A plain device-to-device copy of known size (256 MiB read + 256 MiB
    written per launch), used to calibrate the rocprofv3 byte counters."""
    import torch
    n = 256 << 20
    src = torch.empty(n, dtype=torch.uint8, device="cuda").random_(0, 255)
    dst = torch.empty_like(src)
    ms = time_steps(lambda: dst.copy_(src), args.steps, args.warmup)
    return {"metric": "copy probe GB/s", "value": 2 * n / (ms * 1e-3) / 1e9, "unit": "GB/s",
            "bytes_read_per_launch": n, "bytes_written_per_launch": n, "ms_per_step": ms,
            "steps": args.steps, "warmup": args.warmup, "n_gpus": 1, "launches_per_step": 1}


def bench_kv_write(args):
    """KV-cache write of a whole ModernBERT-shaped prompt batch (32 sequences,
    L ~ U[64,1024], 12 heads, D = 64, fp32) into a randomly permuted block
    pool: algorithmic bytes = k_new + v_new read + the same written."""
    import torch
    import sliding_window_mask_amd as pa
    import workloads
    case = workloads.modernbert_prefill_f32(0, device="cuda")
    T, H, D = case.q.shape
    L = case.lens
    bt = case.block_tables.cpu()
    slots = torch.cat([bt[b, torch.arange(int(L[b])) // 16].long() * 16 +
                       torch.arange(int(L[b])) % 16 for b in range(case.num_seqs)]).to("cuda")
    gen = torch.Generator(device="cuda").manual_seed(7)
    kn = torch.randn(T, H, D, device="cuda", generator=gen)
    vn = torch.randn(T, H, D, device="cuda", generator=gen)
    lib = pa.lib()
    ms = time_steps(lambda: lib.paged_kv_write(case.k_cache, case.v_cache, kn, vn, slots),
                    args.steps, args.warmup)
    nbytes = 2 * 2 * T * H * D * 4
    gbps = nbytes / (ms * 1e-3) / 1e9
    return _line("KV-cache write GB/s", gbps, "GB/s", ms, args, "f32",
                 {"workload": "kv_write_modernbert_f32", "tokens": T, "num_heads": H,
                  "head_dim": D},
                 algorithmic_bytes_per_step=nbytes, launches_per_step=1,
                 roofline={"bound": "hbm", "achieved": gbps, "peak": HBM_PEAK_GBPS,
                           "unit": "GB/s", "frac": gbps / HBM_PEAK_GBPS,
                           "traffic": read_traffic("kv_write_modernbert_f32", "pa_cache.hip"),
                           "kernel": "pa_kv_write"})


def bench_configs(args):
    """Every other workload of the path, each as it is printed by its own
    --workload run (roofline and CPU baseline included)."""
    import torch
    out = {}
    for name, fn in (("t5_small_self_decode_bf16",
                      lambda: bench_small_decode(args, "t5_small_self_decode_bf16")),
                     ("t5_large_cross_decode_bf16",
                      lambda: bench_small_decode(args, "t5_large_cross_decode_bf16")),
                     ("modernbert_prefill_f32", lambda: bench_prefill(args, "f32")),
                     ("modernbert_prefill_bf16", lambda: bench_prefill(args, "bf16"))):
        t0 = time.time()
        line = fn()
        for k in ("n_gpus", "scaling", "data", "steps", "warmup"):
            line.pop(k, None)
        out[name] = line
        torch.cuda.empty_cache()
        log("%s: %.4f ms/step, roofline %.3f (%.1f s)"
            % (name, line["ms_per_step"], line["roofline"]["frac"], time.time() - t0))
    return out


def bench_prefill_layer(args):
    """One ModernBERT-shaped prefill layer (32 sequences, lengths U[64, 1024],
    12 heads, head_dim 64, no bias) at --layer-window, in --layer-dtype,
    causal with --layer-causal: the unit the counter passes of single layers
    are taken over."""
    import torch
    import sliding_window_mask_amd as pa
    lib = pa.lib()
    dn = args.layer_dtype
    dt = torch.float32 if dn == "f32" else torch.bfloat16
    c = modernbert_layers(dt)[0]
    o = torch.empty_like(c.q)
    torch.cuda.synchronize()
    w, causal = args.layer_window, args.layer_causal
    ms = time_steps(lambda: lib.paged_attn_prefill(
        c.q, c.k_cache, c.v_cache, c.block_tables, c.context_lens, c.query_start_loc,
        None, w, causal, c.scale, max_seq_len=c.max_seq_len, out=o), args.steps, args.warmup)
    fl = prefill_flops(c.lens, 12, 64, w, causal=causal)
    by = prefill_bytes(c.lens, 12, 64, 4 if dn == "f32" else 2)
    return {"metric": "one prefill layer", "workload": "prefill_layer_" + dn,
            "sliding_window": w, "causal": causal, "steps": args.steps, "warmup": args.warmup,
            "launches_per_step": 1, "ms_per_step": ms, "us_per_layer": ms * 1e3,
            "TFLOPs": fl / (ms * 1e-3) / 1e12, "GBps": by / (ms * 1e-3) / 1e9}


def bench_prefill_window_sweep(args):
    """One ModernBERT-shaped layer (32 sequences, lengths U[64, 1024], 12
    heads, head_dim 64) through the product prefill call at a range of
    sliding windows, in both dtypes, without a bias and with a materialised
    fp32 bias [32, 12, 1024, 1024] N(0, 1) (its visible entries read)."""
    import torch
    import sliding_window_mask_amd as pa
    lib = pa.lib()
    rows = []
    bias = None
    for dtype_name, dtype, esize in (("f32", torch.float32, 4), ("bf16", torch.bfloat16, 2)):
        c = modernbert_layers(dtype)[0]
        o = torch.empty_like(c.q)
        if bias is None:
            bias = torch.randn(c.num_seqs, 12, c.max_seq_len, c.max_seq_len, device="cuda",
                               generator=torch.Generator(device="cuda").manual_seed(12))
        torch.cuda.synchronize()
        by = prefill_bytes(c.lens, 12, 64, esize)
        for w in (1, 16, 32, 64, 128, 256, 512, -1):
            fl = prefill_flops(c.lens, 12, 64, w)
            row = {"dtype": dtype_name, "sliding_window": w}
            for tag, bb in (("", None), ("_with_bias", bias)):
                msl = time_steps(lambda: lib.paged_attn_prefill(
                    c.q, c.k_cache, c.v_cache, c.block_tables, c.context_lens,
                    c.query_start_loc, bb, w, False, c.scale, max_seq_len=c.max_seq_len, out=o),
                    args.steps, args.warmup)
                row["us_per_layer" + tag] = msl * 1e3
                row["TFLOPs" + tag] = fl / (msl * 1e-3) / 1e12
            row["GBps"] = by / (row["us_per_layer"] * 1e-6) / 1e9
            # visible bias entries: one per visible (query, key) pair and head
            row["bias_GBps"] = fl // (4 * 64) * 4 / (row["us_per_layer_with_bias"] * 1e-6) / 1e9
            rows.append(row)
        del c, o
    return {"metric": "prefill layer time by sliding window", "rows": rows,
            "note": "one layer of the 12-layer ModernBERT-shaped step; GBps counts q, K, V "
                    "read once and the output written once; bias_GBps the visible bias "
                    "entries over the biased layer's time"}


# ----------------------------------------------------------------------------
# hardware probes (bench_probes.hip, built by __graft_entry__.build())
# ----------------------------------------------------------------------------
def _probe_lib():
    import ctypes
    path = os.path.join(ROOT, "bench_probes.so")
    if not os.path.exists(path):
        raise SystemExit("bench_probes.so is not built: run __graft_entry__.build()")
    lib = ctypes.CDLL(path)
    P, I, I64 = ctypes.c_void_p, ctypes.c_int, ctypes.c_int64
    lib.pb_mfma.argtypes = [I, I, I, I, I, P, P]
    lib.pb_lds.argtypes = [I, I, I, P, P]
    lib.pb_stream.argtypes = [P, I64, I, P, P]
    lib.pb_gather.argtypes = [I, P, P, P, P, I, I, I, I, P, P]
    lib.pb_bias.argtypes = [P, P, I, I, I, I, I, P, P]
    lib.pb_mix.argtypes = [I, I, I, P, P]
    lib.pb_valu.argtypes = [I, I, I, P, P]
    lib.pb_clock.argtypes = [I, I, I, P, P]
    for f in (lib.pb_mfma, lib.pb_lds, lib.pb_stream, lib.pb_gather, lib.pb_bias, lib.pb_mix,
              lib.pb_valu, lib.pb_clock):
        f.restype = I
    return lib


def _probe_call(rc):
    if rc != 0:
        raise RuntimeError("probe launch failed (%d)" % rc)


def bench_probe_mfma(args):
    """Rate each matrix instruction sustains with independent accumulator
    chains in every wave (registers only), at several waves per SIMD, and
    with v_exp_f32 work interleaved."""
    import torch
    lib = _probe_lib()
    stream = torch.cuda.current_stream().cuda_stream
    kinds = {0: ("v_mfma_f32_16x16x32_bf16", 2 * 16 * 16 * 32, BF16_MFMA_PEAK_TFLOPS),
             1: ("v_mfma_f32_32x32x16_bf16", 2 * 32 * 32 * 16, BF16_MFMA_PEAK_TFLOPS),
             2: ("v_mfma_f32_16x16x4_f32", 2 * 16 * 16 * 4, FP32_MFMA_PEAK_TFLOPS),
             3: ("v_mfma_f32_32x32x2_f32", 2 * 32 * 32 * 2, FP32_MFMA_PEAK_TFLOPS)}
    cases = [(k, wps, ch, 0) for k in kinds for wps, ch in ((2, 4), (4, 4), (8, 4), (4, 8))]
    cases += [(k, 4, ch, e) for k in (0, 1) for ch, e in ((4, 1), (4, 2), (2, 2), (2, 4))]
    iters = 8000
    rows = []
    out = torch.empty(256 * 8 * 256, dtype=torch.float32, device="cuda")
    for kind, wps, ch, ex in cases:
        grid = 256 * wps                    # 4-wave workgroups: wps waves per SIMD
        ms = time_steps(lambda: _probe_call(lib.pb_mfma(kind, ch, ex, grid, iters,
                                                        out.data_ptr(), stream)),
                        args.steps, args.warmup)
        name, flops, peak = kinds[kind]
        tf = flops * ch * iters * grid * 4 / (ms * 1e-3) / 1e12
        rows.append({"instruction": name, "waves_per_simd": wps, "chains_per_wave": ch,
                     "exp_per_product": ex, "ms": ms, "TFLOPs": tf, "frac_of_peak": tf / peak})
    return {"metric": "probe: sustained matrix-instruction rates", "rows": rows,
            "note": "independent accumulator chains per wave, registers only; grid = 256 "
                    "CUs x waves_per_simd 4-wave workgroups, %d iterations" % iters}


def bench_probe_clock(args):
    """The shader clock while every SIMD runs matrix (four 32x32x16 chains per
    wave) or vector (v_exp_f32 chains) work at 4 waves per SIMD: s_memtime
    cycles over s_memrealtime's constant 100 MHz ticks, per workgroup."""
    import torch
    lib = _probe_lib()
    stream = torch.cuda.current_stream().cuda_stream
    grid = 256 * 4
    out = torch.zeros(2 * grid, dtype=torch.float32, device="cuda")
    rows = []
    for kind, name, iters in ((0, "v_mfma_f32_32x32x16_bf16 x4 chains", 20000),
                              (1, "v_exp_f32 x8 chains", 40000)):
        ms = time_steps(lambda: _probe_call(lib.pb_clock(kind, grid, iters, out.data_ptr(),
                                                         stream)), args.steps, args.warmup)
        v = out.view(grid, 2).double().cpu().numpy()
        ghz = v[:, 0] / np.maximum(v[:, 1], 1.0) * 0.1
        row = {"work": name, "us": ms * 1e3, "clock_GHz_median": float(np.median(ghz)),
               "clock_GHz_min": float(np.min(ghz)), "clock_GHz_max": float(np.max(ghz))}
        if kind == 0:
            tf = 2 * 32 * 32 * 16 * 4 * iters * grid * 4 / (ms * 1e-3) / 1e12
            row["TFLOPs"] = tf
            row["cycles_per_mfma_at_measured_clock"] = (ms * 1e-3 * row["clock_GHz_median"] * 1e9 /
                                                        (4 * iters))
        rows.append(row)
    return {"metric": "probe: shader clock under load", "rows": rows}


def bench_probe_valu(args):
    """SIMD cycles per wave64 vector instruction: 8 independent chains per
    thread of v_add_f32, v_fma_f32 or v_exp_f32, 8192 workgroups of 4 waves
    (cycles at 2.4 GHz over the chip's 1024 SIMDs)."""
    import torch
    lib = _probe_lib()
    stream = torch.cuda.current_stream().cuda_stream
    grid, iters = 8192, 1024
    out = torch.empty(grid * 256, dtype=torch.float32, device="cuda")
    rows = []
    for kind, name in ((0, "v_add_f32"), (1, "v_fma_f32"), (2, "v_exp_f32")):
        ms = time_steps(lambda: _probe_call(lib.pb_valu(kind, grid, iters, out.data_ptr(),
                                                        stream)), args.steps, args.warmup)
        insts = grid * 4 * iters * 8
        rows.append({"instruction": name, "us": ms * 1e3,
                     "simd_cycles_per_wave_instruction": ms * 1e-3 * 2.4e9 * 1024 / insts})
    return {"metric": "probe: vector instruction rate", "rows": rows}


def bench_probe_mix(args):
    """Whether matrix-core work of some waves overlaps vector work of other
    waves on the same SIMD: 8-wave workgroups whose waves 0-3 run MFMA
    chains (four independent ones, or one dependent chain) and waves 4-7 an
    exp/fma loop, timed alone and together."""
    import torch
    lib = _probe_lib()
    stream = torch.cuda.current_stream().cuda_stream
    rows = []
    for wgs in (1, 2):
        grid = 256 * wgs
        out = torch.empty(grid * 512, dtype=torch.float32, device="cuda")
        t = {}
        for mode, name in ((0, "mfma_waves_only"), (1, "valu_waves_only"), (2, "both"),
                           (3, "chained_mfma_waves_only"), (4, "chained_mfma_and_valu")):
            t[name] = time_steps(lambda: _probe_call(lib.pb_mix(mode, grid, 4000, out.data_ptr(),
                                                               stream)),
                                 args.steps, args.warmup) * 1e3
        rows.append({"workgroups_per_cu": wgs, **{k + "_us": v for k, v in t.items()},
                     "both_over_max": t["both"] / max(t["mfma_waves_only"], t["valu_waves_only"]),
                     "both_over_sum": t["both"] / (t["mfma_waves_only"] + t["valu_waves_only"]),
                     "chained_both_over_sum": t["chained_mfma_and_valu"] / (
                         t["chained_mfma_waves_only"] + t["valu_waves_only"])})
    return {"metric": "probe: matrix/vector overlap across waves of one SIMD", "rows": rows}


def bench_probe_lds(args):
    """LDS read rate per CU: conflict-free 16-byte reads (ds_read_b128) and
    transposing 8-byte reads (ds_read_b64_tr_b16)."""
    import torch
    lib = _probe_lib()
    stream = torch.cuda.current_stream().cuda_stream
    iters = 4000
    out = torch.empty(256 * 8 * 256, dtype=torch.float32, device="cuda")
    rows = []
    for wgs in (2, 4, 8):
        for kind, name, size in ((0, "ds_read_b128", 16), (1, "ds_read_b64_tr_b16", 8)):
            grid = 256 * wgs
            ms = time_steps(lambda: _probe_call(lib.pb_lds(kind, grid, iters, out.data_ptr(),
                                                           stream)), args.steps, args.warmup)
            nbytes = grid * 256 * iters * 8 * size
            rows.append({"read": name, "workgroups_per_cu": wgs, "ms": ms,
                         "TBps": nbytes / (ms * 1e-3) / 1e12,
                         "bytes_per_clk_per_cu_at_2.4GHz": nbytes / (ms * 1e-3) / 256 / 2.4e9})
    return {"metric": "probe: LDS read rate", "rows": rows,
            "note": "4-wave workgroups, each wave reading 1 KiB LDS rows; %d x 8 reads per "
                    "thread" % iters}


def bench_probe_stream(args):
    """A streaming read of 8 GiB with non-temporal 16-byte loads."""
    import torch
    lib = _probe_lib()
    stream = torch.cuda.current_stream().cuda_stream
    nbytes = 8 << 30
    src = torch.zeros(nbytes, dtype=torch.uint8, device="cuda")
    rows = []
    for grid in (256 * 8, 256 * 16, 256 * 32):
        out = torch.empty(grid * 256, dtype=torch.float32, device="cuda")
        ms = time_steps(lambda: _probe_call(lib.pb_stream(src.data_ptr(), nbytes, grid,
                                                          out.data_ptr(), stream)),
                        args.steps, args.warmup)
        gbps = nbytes / (ms * 1e-3) / 1e9
        rows.append({"workgroups": grid, "ms": ms, "GBps": gbps, "hbm_frac": gbps / HBM_PEAK_GBPS})
    return {"metric": "probe: streaming read GB/s", "value": max(r["GBps"] for r in rows),
            "rows": rows, "bytes": nbytes,
            "note": "non-temporal 16-byte loads, 4 in flight per thread, 256-thread workgroups"}


def bench_probe_bias(args):
    """The materialised prefill bias of one ModernBERT-shaped full-attention
    layer ([32, 12, 1024, 1024] fp32, lengths U[64, 1024]) read with no
    arithmetic in the order the prefill kernels walk it (each wave its 32
    query rows, advancing along the keys), at several widths per row and
    iteration (W bytes, G contiguous bytes per row and load)."""
    import torch
    lib = _probe_lib()
    stream = torch.cuda.current_stream().cuda_stream
    c = modernbert_layers(torch.bfloat16)[0]
    H, M = 12, c.max_seq_len
    bias = torch.randn(c.num_seqs, H, M, M, device="cuda",
                       generator=torch.Generator(device="cuda").manual_seed(13))
    lens = c.context_lens
    out = torch.empty((M // 128) * H * c.num_seqs * 256, dtype=torch.float32, device="cuda")
    torch.cuda.synchronize()
    rows = []
    for w, g in ((128, 128), (256, 256), (512, 128), (512, 512)):
        ms = time_steps(lambda: _probe_call(lib.pb_bias(
            bias.data_ptr(), lens.data_ptr(), c.num_seqs, H, M, w, g, out.data_ptr(), stream)),
            args.steps, args.warmup)
        L = c.lens.astype(np.int64)
        nbytes = int(np.sum(L * ((L + w // 4 - 1) // (w // 4) * (w // 4)))) * 4 * H
        rows.append({"W_bytes_per_row_per_iteration": w, "G_contiguous_bytes_per_load": g,
                     "us": ms * 1e3, "GBps": nbytes / (ms * 1e-3) / 1e9, "bytes": nbytes})
    return {"metric": "probe: prefill bias access pattern", "rows": rows,
            "note": "one workgroup of 4 waves per (128-query tile, head, sequence); wave w "
                    "reads rows 32w..32w+31 of its tile, W/32 non-temporal 16-byte loads per "
                    "lane in flight per iteration"}


def bench_probe_gather_t5(args):
    """The T5-large cross-attention decode's K/V gather without arithmetic
    (pb_gather, the decode kernel's order and loads), next to the decode call,
    both as back-to-back calls over rotating copies of the inputs (over 1 GiB)
    replayed from a HIP graph, as the T5 decode lines time them."""
    import torch
    import sliding_window_mask_amd as pa
    import workloads
    lib = _probe_lib()
    dec = pa.lib()
    case = workloads.t5_large_cross_decode_bf16(device="cuda", bias=None)
    B, H, D = case.q.shape
    block_bytes = 16 * D * case.k_cache.element_size()
    per_copy = sum(t.numel() * t.element_size() for t in (case.q, case.k_cache, case.v_cache))
    ncopy = max(4, -(-(1 << 30) // per_copy))
    layers = [(case.q.clone(), case.k_cache.clone(), case.v_cache.clone(),
               torch.empty_like(case.q)) for _ in range(ncopy)]
    ws = dec.workspace_for(case.q, case.max_seq_len, case.sliding_window)
    pout = torch.empty(B * H * 256, dtype=torch.float32, device="cuda")
    torch.cuda.synchronize()

    def graph_ms(fn):
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            for c in layers:
                fn(*c)
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for i in range(args.steps):
                fn(*layers[i % ncopy])
        return time_steps(g.replay, 1, args.warmup) / args.steps

    def gather(mode):
        def fn(q, k, v, o):
            _probe_call(lib.pb_gather(mode, k.data_ptr(), v.data_ptr(),
                                      case.block_tables.data_ptr(),
                                      case.context_lens.data_ptr(), B, H, block_bytes,
                                      case.block_tables.shape[1], pout.data_ptr(),
                                      torch.cuda.current_stream().cuda_stream))
        return fn
    kv = 2 * H * block_bytes * int(np.sum((case.lens + 15) // 16))
    res = {}
    for mode, name in ((0, "k_then_v_nontemporal"), (2, "k_and_v_together_nontemporal")):
        ms = graph_ms(gather(mode))
        res[name] = {"us": ms * 1e3, "kv_GBps": kv / (ms * 1e-3) / 1e9}
    msd = graph_ms(lambda q, k, v, o: dec.paged_attn_decode(
        q, k, v, case.block_tables, case.context_lens, None, case.sliding_window, case.scale,
        max_seq_len=case.max_seq_len, out=o, workspace=ws))
    # a contiguous read of the same number of bytes per call, over as many
    # rotating buffers
    nbytes = (kv + 15) // 16 * 16
    bufs = [torch.zeros(nbytes, dtype=torch.uint8, device="cuda") for _ in range(ncopy)]
    sgrid = 256 * 16
    sout = torch.empty(sgrid * 256, dtype=torch.float32, device="cuda")
    layers_bak = layers
    layers = [(b_, None, None, None) for b_ in bufs]

    def stream_fn(buf, *_):
        _probe_call(lib.pb_stream(buf.data_ptr(), nbytes, sgrid, sout.data_ptr(),
                                  torch.cuda.current_stream().cuda_stream))
    mss = graph_ms(stream_fn)
    layers = layers_bak
    return {"metric": "probe: T5-large cross decode K/V gather without arithmetic",
            "orders": res, "us_decode_call": msd * 1e3,
            "us_contiguous_read_same_bytes": mss * 1e3,
            "contiguous_GBps": nbytes / (mss * 1e-3) / 1e9,
            "decode_kv_GBps": kv / (msd * 1e-3) / 1e9, "kv_bytes": kv, "copies": ncopy,
            "note": "256 sequences x 16 heads, head_dim 64, bf16, encoder lengths U[128, 512]; "
                    "graph-replayed back-to-back calls over rotating input copies"}


def bench_probe_gather(args):
    """The large decode's K/V gather (same block tables, 4 blocks in flight
    per wave, K pass then V pass, non-temporal loads) with no arithmetic and
    no bias, next to the decode call on the same inputs."""
    import torch
    import sliding_window_mask_amd as pa
    import workloads
    lib = _probe_lib()
    stream = torch.cuda.current_stream().cuda_stream
    case = workloads.large_biased_decode_bf16(device="cuda")
    torch.cuda.synchronize()
    B, H, D = case.q.shape
    block_bytes = 16 * D * case.k_cache.element_size()
    out = torch.empty(B * H * 256, dtype=torch.float32, device="cuda")
    kv = 2 * H * block_bytes * int(np.sum((case.lens + 15) // 16))
    modes = {}
    for mode, name in ((0, "k_then_v_nontemporal"), (1, "k_then_v_ordinary_loads"),
                       (2, "k_and_v_together_nontemporal")):
        msm = time_steps(lambda: _probe_call(lib.pb_gather(
            mode, case.k_cache.data_ptr(), case.v_cache.data_ptr(),
            case.block_tables.data_ptr(), case.context_lens.data_ptr(), B, H, block_bytes,
            case.block_tables.shape[1], out.data_ptr(), stream)), args.steps, args.warmup)
        modes[name] = {"ms": msm, "kv_GBps": kv / (msm * 1e-3) / 1e9}
    ms = modes["k_then_v_nontemporal"]["ms"]
    o = torch.empty_like(case.q)
    dec = pa.lib()
    ws = dec.workspace_for(case.q, case.max_seq_len, case.sliding_window)
    ms_dec = time_steps(lambda: dec.paged_attn_decode(
        case.q, case.k_cache, case.v_cache, case.block_tables, case.context_lens,
        case.attn_bias, -1, case.scale, max_seq_len=case.max_seq_len, out=o, workspace=ws),
        args.steps, args.warmup)
    return {"metric": "probe: decode K/V gather without arithmetic", "ms_gather": ms,
            "kv_GBps": kv / (ms * 1e-3) / 1e9, "orders": modes, "ms_decode_call": ms_dec,
            "decode_kv_GBps": kv / (ms_dec * 1e-3) / 1e9, "kv_bytes": kv,
            "note": "large biased decode inputs (256 x 32 heads, head_dim 128, bf16); the "
                    "decode call also reads the bias and q and writes the output"}


# ----------------------------------------------------------------------------
# profile summaries (rocprofv3 output -> profiles/)
# ----------------------------------------------------------------------------
def _rows(path):
    with open(path, newline="") as f:
        return list(csv.DictReader(f))


def _find(path, suffix):
    """A rocprofv3 output file: `path` itself, or the one file under the
    directory `path` whose name ends in `suffix`."""
    if os.path.isfile(path):
        return path
    hits = sorted(glob.glob(os.path.join(path, "**", "*" + suffix), recursive=True))
    if len(hits) != 1:
        raise SystemExit("expected one *%s under %s, found %d" % (suffix, path, len(hits)))
    return hits[0]


def kernel_tag(name):
    """Short key for a kernel name: 'pa_prefill_f32<64, 1, 0, false, 1>' ->
    'pa_prefill_f32_64_1_0_false_1'."""
    import re
    m = re.search(r"(pa_\w+)(<[^>]*>)?", name)
    if not m:
        return re.sub(r"\W+", "_", name).strip("_")
    args = re.sub(r"[^\w]+", "_", m.group(2) or "").strip("_")
    return m.group(1) + ("_" + args if args else "")


def _ours(name):
    return " pa::" in (" " + name) or name.startswith("pa::")


def timed_dispatches(rows, n):
    """The last n dispatches of the library's kernels, in dispatch order."""
    mine = [r for r in rows if _ours(r["Kernel_Name"])]
    mine.sort(key=lambda r: int(r["Dispatch_Id"]))
    if len(mine) < n:
        raise SystemExit("only %d dispatches of the library's kernels, %d expected"
                         % (len(mine), n))
    return mine[-n:]


def trace_table(trace_csv, n):
    """Per kernel name over the last n dispatches: count and mean / min / max
    duration in microseconds (from the kernel trace's timestamps)."""
    per = {}
    for r in timed_dispatches(_rows(trace_csv), n):
        d = (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1000.0
        per.setdefault(r["Kernel_Name"], []).append(d)
    return per


def counter_table(counter_csv, n):
    """Per kernel name over the last n dispatches: the summed counter value of
    each dispatch (rows of one dispatch are summed), as a list."""
    rows = _rows(counter_csv)
    by_disp = {}
    for r in rows:
        if not _ours(r["Kernel_Name"]):
            continue
        k = int(r["Dispatch_Id"])
        by_disp.setdefault(k, [r["Kernel_Name"], 0.0])
        by_disp[k][1] += float(r["Counter_Value"])
    ids = sorted(by_disp)[-n:]
    if len(ids) < n:
        raise SystemExit("only %d counted dispatches, %d expected" % (len(ids), n))
    per = {}
    for k in ids:
        per.setdefault(by_disp[k][0], []).append(by_disp[k][1])
    return per


def copy_counter(counter_csv):
    """Median counter value (KiB) per dispatch of the calibration copy."""
    vals = {}
    for r in _rows(counter_csv):
        if "copy" in r["Kernel_Name"].lower():
            vals[r["Dispatch_Id"]] = vals.get(r["Dispatch_Id"], 0.0) + float(r["Counter_Value"])
    if not vals:
        raise SystemExit("no copy kernel in %s" % counter_csv)
    return statistics.median(vals.values())


def write_profiles(a):
    """Write profiles/<workload>_kernel_trace.md (and, with the counter runs,
    profiles/<workload>_traffic.txt) from rocprofv3 output of --profile-run
    runs. --trace DIR: a `--kernel-trace --stats` run; --bench-line FILE: its
    printed JSON line (steps and launches per step say which dispatches were
    timed); --fetch/--write DIR: `--pmc FETCH_SIZE` / `--pmc WRITE_SIZE` runs
    with --counter-line FILE their JSON line; --copy-fetch/--copy-write DIR:
    the same passes over --workload copy_probe (the byte calibration)."""
    wl = a.write_profiles
    src = KERNEL_SOURCE[wl]
    sha = source_sha(src)
    line = json.loads(open(a.bench_line).read().strip().splitlines()[-1])
    n = line["steps"] * line["launches_per_step"]
    trace = _find(a.trace, "_kernel_trace.csv")
    per = trace_table(trace, n)
    step_us = sum(sum(v) for v in per.values()) / line["steps"]
    cmd = a.command or "(command not recorded)"
    md = ["# Kernel trace: %s (timed steps only)" % wl, "",
          "Command (on the MI355X box, from the repository root):", "",
          "    " + cmd, "",
          "%s sha256[:16] = %s" % (" + ".join(src) if isinstance(src, tuple) else src, sha), "",
          "Averages over the last %d dispatches of the library's kernels: the %d timed "
          "steps of `--profile-run` (%d launch(es) per step); warm-up and clock-settling "
          "launches are excluded." % (n, line["steps"], line["launches_per_step"]), "",
          "| kernel | calls | average (us) | min (us) | max (us) |", "|---|---|---|---|---|"]
    for k, v in sorted(per.items(), key=lambda kv: -sum(kv[1])):
        md.append("| `%s` | %d | %.1f | %.1f | %.1f |" % (k, len(v), sum(v) / len(v),
                                                           min(v), max(v)))
    md += ["", "Sum of kernel durations per step: %.1f us. The bench line of the same run "
           "(HIP events around the %d timed steps): %.1f us per step, roofline frac %.4f."
           % (step_us, line["steps"], line["ms_per_step"] * 1000, line["roofline"]["frac"])]
    if wl.startswith("t5_") and line["ms_per_step"] * 1000 > 1.2 * step_us:
        md.append("Under --profile-run the T5 calls are launched one by one from the host (the "
                  "default run replays them from a HIP graph), so the events of this run also "
                  "time the host's launch gaps under the profiler; the kernel durations above "
                  "are the figure to compare with the default bench line.")
    if "algorithmic_bytes_per_step" in line:
        md.append("Algorithmic bytes per step: %d (%.1f GB/s over the summed kernel time)."
                  % (line["algorithmic_bytes_per_step"],
                     line["algorithmic_bytes_per_step"] / (step_us * 1e-6) / 1e9))
    if "algorithmic_flops_per_step" in line:
        md.append("Algorithmic flops per step: %d (%.1f TFLOP/s over the summed kernel time)."
                  % (line["algorithmic_flops_per_step"],
                     line["algorithmic_flops_per_step"] / (step_us * 1e-6) / 1e12))
    open(os.path.join(PROFILES, "%s_kernel_trace.md" % wl), "w").write("\n".join(md) + "\n")
    if not a.fetch:
        return
    cl = json.loads(open(a.counter_line).read().strip().splitlines()[-1])
    nc = cl["steps"] * cl["launches_per_step"]
    cf = copy_counter(_find(a.copy_fetch, "_counter_collection.csv"))
    cw = copy_counter(_find(a.copy_write, "_counter_collection.csv"))
    fs, ws = 262144.0 / cf, 262144.0 / cw
    fpk = counter_table(_find(a.fetch, "_counter_collection.csv"), nc)
    wpk = counter_table(_find(a.write, "_counter_collection.csv"), nc)
    hb_step = (sum(sum(v) for v in fpk.values()) * fs +
               sum(sum(v) for v in wpk.values()) * ws) * 1024 / cl["steps"]
    alg = cl["algorithmic_bytes_per_step"]
    txt = ["# HBM traffic: %s (counter passes over the timed steps of --profile-run)" % wl,
           "#", "# Commands (each its own run, on the MI355X box, from the repository root):"]
    txt += ["#   " + c for c in (a.counter_commands or [])]
    txt += ["# Counter values are KiB per dispatch, scaled so that the same counter reads",
            "# 262144 KiB for a plain 256 MiB device copy (read and written once).",
            "# Bytes per step = summed scaled FETCH_SIZE + WRITE_SIZE of the last %d"
            % nc, "# dispatches (%d steps of %d launch(es)), divided by %d."
            % (cl["steps"], cl["launches_per_step"], cl["steps"]),
            "kernel_source_sha = %s" % sha,
            "copy_FETCH_SIZE_KiB = %.1f" % cf, "copy_WRITE_SIZE_KiB = %.1f" % cw,
            "fetch_scale = %.5f" % fs, "write_scale = %.5f" % ws]
    for k in sorted(fpk):
        tag = kernel_tag(k)
        f_med = statistics.median(fpk[k])
        w_med = statistics.median(wpk.get(k, [0.0]))
        txt += ["# kernel %s" % k,
                "%s_FETCH_SIZE_KiB_median = %.1f" % (tag, f_med),
                "%s_WRITE_SIZE_KiB_median = %.1f" % (tag, w_med),
                "%s_hbm_bytes_median = %.0f" % (tag, (f_med * fs + w_med * ws) * 1024)]
    txt += ["hbm_bytes_per_step = %.0f" % hb_step,
            "hbm_bytes_per_launch = %.0f" % (hb_step / cl["launches_per_step"]),
            "algorithmic_bytes_per_step = %d" % alg,
            "ratio_hbm_to_algorithmic = %.4f" % (hb_step / alg)]
    open(os.path.join(PROFILES, "%s_traffic.txt" % wl), "w").write("\n".join(txt) + "\n")


def write_counter_summary(a):
    """profiles/<workload>_counters.md: the median per dispatch of every
    counter of one `--pmc` run over the timed dispatches, per kernel."""
    wl = a.counter_summary
    line = json.loads(open(a.counter_line).read().strip().splitlines()[-1])
    n = line["steps"] * line["launches_per_step"]
    rows = _rows(_find(a.counters, "_counter_collection.csv"))
    by = {}
    for r in rows:
        if _ours(r["Kernel_Name"]):
            by.setdefault(int(r["Dispatch_Id"]), {"k": r["Kernel_Name"]})
            d = by[int(r["Dispatch_Id"])]
            d[r["Counter_Name"]] = d.get(r["Counter_Name"], 0.0) + float(r["Counter_Value"])
    ids = sorted(by)[-n:]
    names = sorted({c for i in ids for c in by[i] if c != "k"})
    kernels = sorted({by[i]["k"] for i in ids})
    path = os.path.join(PROFILES, "%s_counters.md" % wl)
    old = open(path).read() if os.path.exists(path) and a.append else ""
    ks = kernel_source_of(wl)
    md = [old.rstrip() + "\n"] if old else ["# Counters: %s (timed steps of --profile-run)" % wl,
                                            "", "%s sha256[:16] = %s" % (
                                                " + ".join(ks) if isinstance(ks, tuple) else ks,
                                                source_sha(ks)), ""]
    md += ["Command: `%s`" % (a.command or "(not recorded)"), "",
           "| kernel | " + " | ".join(names) + " |", "|---|" + "---|" * len(names)]
    med = {}
    for k in kernels:
        vals = [statistics.median([by[i][c] for i in ids if by[i]["k"] == k and c in by[i]])
                if any(by[i]["k"] == k and c in by[i] for i in ids) else float("nan")
                for c in names]
        med[k] = dict(zip(names, vals))
        md.append("| `%s` | " % k + " | ".join("%.4g" % v for v in vals) + " |")
    md += ["", "Medians per dispatch over the last %d dispatches (%d timed steps). Each "
           "counter is summed by rocprofv3 over the chip; GRBM_GUI_ACTIVE over the 8 XCDs, so "
           "GRBM_GUI_ACTIVE / 8 is the launch duration in cycles." % (n, line["steps"])]
    derived = []
    for k, v in med.items():
        row = []
        cyc = v.get("GRBM_GUI_ACTIVE", float("nan")) / 8
        if "SQ_VALU_MFMA_BUSY_CYCLES" in v:
            row.append(("MFMA busy (per SIMD per launch cycle)",
                        "%.1f%%" % (100 * v["SQ_VALU_MFMA_BUSY_CYCLES"] / (cyc * 1024))))
        if "SQ_INSTS_MFMA" in v and "SQ_INSTS_VALU" in v:
            row.append(("other VALU insts per MFMA inst",
                        "%.2f" % ((v["SQ_INSTS_VALU"] - v["SQ_INSTS_MFMA"]) / v["SQ_INSTS_MFMA"])))
        if "SQ_INSTS_MFMA" in v and "SQ_INSTS_LDS" in v:
            row.append(("LDS insts per MFMA inst", "%.2f" % (v["SQ_INSTS_LDS"] / v["SQ_INSTS_MFMA"])))
        if "SQ_WAIT_INST_ANY" in v and "SQ_WAVE_CYCLES" in v:
            row.append(("SQ_WAIT_INST_ANY / SQ_WAVE_CYCLES",
                        "%.2f" % (v["SQ_WAIT_INST_ANY"] / v["SQ_WAVE_CYCLES"])))
        if "TCC_HIT_sum" in v and "TCC_MISS_sum" in v:
            row.append(("L2 hit rate (TCC_HIT / (TCC_HIT + TCC_MISS))", "%.1f%%" % (
                100 * v["TCC_HIT_sum"] / max(1.0, v["TCC_HIT_sum"] + v["TCC_MISS_sum"]))))
        if "TCP_TCC_READ_REQ_LATENCY_sum" in v and "TCP_TCC_READ_REQ_sum" in v:
            row.append(("mean L1-to-L2 read latency (cycles per request)", "%.0f" % (
                v["TCP_TCC_READ_REQ_LATENCY_sum"] / max(1.0, v["TCP_TCC_READ_REQ_sum"]))))
        if "TA_BUSY_avr" in v:
            row.append(("TA busy (per TA, share of the launch)",
                        "%.1f%%" % (100 * v["TA_BUSY_avr"] / cyc)))
        if "TD_TD_BUSY_sum" in v:
            row.append(("TD busy (per CU, share of the launch)",
                        "%.1f%%" % (100 * v["TD_TD_BUSY_sum"] / (cyc * 256))))
        if "SQ_WAIT_ANY" in v and "SQ_WAVE_CYCLES" in v:
            row.append(("SQ_WAIT_ANY / SQ_WAVE_CYCLES",
                        "%.2f" % (v["SQ_WAIT_ANY"] / v["SQ_WAVE_CYCLES"])))
        if "SQ_VALU_MFMA_COEXEC_CYCLES" in v:
            row.append(("VALU-MFMA co-exec (per SIMD per launch cycle)",
                        "%.1f%%" % (100 * v["SQ_VALU_MFMA_COEXEC_CYCLES"] / (cyc * 1024))))
        if row:
            derived.append((k, row))
        if v.get("SQ_LDS_BANK_CONFLICT") == v.get("SQ_INSTS_MFMA") and "SQ_INSTS_MFMA" in v:
            md.append("`%s`: SQ_LDS_BANK_CONFLICT reads exactly SQ_INSTS_MFMA in this pass, so it "
                      "is not taken as a measurement of bank conflicts." % k)
    for k, row in derived:
        md += ["", "Derived, `%s`:" % k, ""] + ["- %s: %s" % kv for kv in row]
    open(path, "w").write("\n".join(md) + "\n")


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="large_biased_decode_bf16")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--layer-dtype", default="f32", choices=("f32", "bf16"))
    ap.add_argument("--layer-window", type=int, default=-1)
    ap.add_argument("--layer-causal", action="store_true")
    ap.add_argument("--no-variants", action="store_true")
    ap.add_argument("--no-configs", action="store_true")
    ap.add_argument("--profile-run", action="store_true")
    ap.add_argument("--write-profiles", metavar="WORKLOAD")
    ap.add_argument("--counter-summary", metavar="WORKLOAD")
    ap.add_argument("--trace")
    ap.add_argument("--bench-line")
    ap.add_argument("--fetch")
    ap.add_argument("--write")
    ap.add_argument("--copy-fetch")
    ap.add_argument("--copy-write")
    ap.add_argument("--counters")
    ap.add_argument("--counter-line")
    ap.add_argument("--command")
    ap.add_argument("--counter-commands", nargs="*")
    ap.add_argument("--append", action="store_true")
    args = ap.parse_args()
    if args.write_profiles:
        write_profiles(args)
        return
    if args.counter_summary:
        write_counter_summary(args)
        return
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py runs on one GPU only: the paged-attention path is measured on a "
              "single MI355X (--gpus 1).", file=sys.stderr)
        sys.exit(2)
    import torch
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(2)
    if args.profile_run:
        args.no_variants = args.no_cpu_baseline = args.no_configs = True
    if args.workload == "large_biased_decode_bf16":
        line = bench_decode(args)
        if not args.no_configs:
            line["configs"] = bench_configs(args)
    elif args.workload in ("modernbert_prefill_f32", "modernbert_prefill_bf16"):
        line = bench_prefill(args, args.workload.rsplit("_", 1)[1])
    elif args.workload in ("modernbert_chunked_prefill_f32", "modernbert_chunked_prefill_bf16"):
        line = bench_chunked_prefill(args, args.workload.rsplit("_", 1)[1])
    elif args.workload in ("t5_small_self_decode_bf16", "t5_large_cross_decode_bf16"):
        line = bench_small_decode(args, args.workload)
    elif args.workload == "kv_write_modernbert_f32":
        line = bench_kv_write(args)
    elif args.workload == "copy_probe":
        line = bench_copy(args)
    elif args.workload == "prefill_layer":
        line = bench_prefill_layer(args)
    elif args.workload == "prefill_window_sweep":
        line = bench_prefill_window_sweep(args)
    elif args.workload == "probe_mfma":
        line = bench_probe_mfma(args)
    elif args.workload == "probe_clock":
        line = bench_probe_clock(args)
    elif args.workload == "probe_valu":
        line = bench_probe_valu(args)
    elif args.workload == "probe_mix":
        line = bench_probe_mix(args)
    elif args.workload == "probe_lds":
        line = bench_probe_lds(args)
    elif args.workload == "probe_stream":
        line = bench_probe_stream(args)
    elif args.workload == "probe_gather":
        line = bench_probe_gather(args)
    elif args.workload == "probe_gather_t5":
        line = bench_probe_gather_t5(args)
    elif args.workload == "probe_bias":
        line = bench_probe_bias(args)
    else:
        raise SystemExit("unknown workload %s" % args.workload)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
