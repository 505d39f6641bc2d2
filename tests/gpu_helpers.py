"""Shared glue for the GPU parity tests: run the HIP library through its
binding, run the float64 oracle on host copies of the same inputs, compare.

Tolerances (max absolute error against the float64 oracle): 1e-5 for fp32,
2e-2 for bf16 outputs (fp32 accumulation inside the kernels)."""
import os
import sys
from types import SimpleNamespace

import numpy as np
import torch

os.environ.setdefault("PA_VALIDATE", "1")      # range-check metadata before each launch

import oracle                                   # noqa: E402
import parity_log                               # noqa: E402
import sliding_window_mask_amd as pa            # noqa: E402

TOL = {torch.float32: 1e-5, torch.bfloat16: 2e-2}
BS = 16


def log(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def to_device(case, device="cuda"):
    d = {}
    for k, v in vars(case).items():
        d[k] = v.to(device) if isinstance(v, torch.Tensor) else v
    return SimpleNamespace(**d)


def to_host(case):
    return to_device(case, "cpu")


def gpu_decode(case, bias="case", window=None, partition=0, lib=None):
    lib = lib or pa.lib()
    out = lib.paged_attn_decode(case.q, case.k_cache, case.v_cache, case.block_tables,
                                case.context_lens, case.attn_bias if bias == "case" else bias,
                                case.sliding_window if window is None else window, case.scale,
                                max_seq_len=case.max_seq_len, partition_tokens=partition)
    torch.cuda.synchronize()
    return out


def oracle_decode(case, bias="case", window=None):
    h = to_host(case)
    b = h.attn_bias if bias == "case" else (None if bias is None else bias.cpu())
    return oracle.decode(h.q, h.k_cache, h.v_cache, h.block_tables, h.context_lens, b,
                         h.sliding_window if window is None else window, h.scale,
                         h.max_seq_len)


def gpu_prefill(case, bias="case", window=None, causal=None):
    out = pa.paged_attn_prefill(case.q, case.k_cache, case.v_cache, case.block_tables,
                                case.context_lens, case.query_start_loc,
                                case.attn_bias if bias == "case" else bias,
                                case.sliding_window if window is None else window,
                                case.causal if causal is None else causal, case.scale,
                                max_seq_len=case.max_seq_len)
    torch.cuda.synchronize()
    return out


def oracle_prefill(case, bias="case", window=None, causal=None):
    h = to_host(case)
    b = h.attn_bias if bias == "case" else (None if bias is None else bias.cpu())
    return oracle.prefill(h.q, h.k_cache, h.v_cache, h.block_tables, h.context_lens,
                          h.query_start_loc, b, h.sliding_window if window is None else window,
                          int(h.causal if causal is None else causal), h.scale, h.max_seq_len)


def max_err(gpu_out, ref):
    g = gpu_out.float().cpu().double().numpy()
    assert np.all(np.isfinite(g)), "non-finite GPU output"
    return float(np.max(np.abs(g - ref))) if g.size else 0.0


def assert_close(gpu_out, ref, dtype, what=""):
    e = max_err(gpu_out, ref)
    log("  %s max|err| = %.3e (tol %.0e)" % (what, e, TOL[dtype]))
    parity_log.add(what, e, TOL[dtype])
    assert e <= TOL[dtype], "%s: max abs error %.3e > %.0e" % (what, e, TOL[dtype])


def sample_decode(case, seqs):
    """Oracle inputs for a subset of sequences: the sampled rows of q, the
    tables, lengths and bias, and a compact host cache holding only the blocks
    those rows reference (tables remapped to it)."""
    seqs = torch.as_tensor(seqs, dtype=torch.long)
    bt = case.block_tables[seqs.to(case.block_tables.device)].cpu()
    used = torch.unique(bt)
    remap = torch.full((case.num_blocks,), -1, dtype=torch.int32)
    remap[used] = torch.arange(used.numel(), dtype=torch.int32)
    dev_used = used.to(case.k_cache.device)
    sub = SimpleNamespace(**vars(case))
    sub.q = case.q[seqs.to(case.q.device)].cpu()
    sub.k_cache = case.k_cache[dev_used].cpu()
    sub.v_cache = case.v_cache[dev_used].cpu()
    sub.block_tables = remap[bt.long()]
    sub.context_lens = case.context_lens[seqs.to(case.context_lens.device)].cpu()
    sub.attn_bias = (None if case.attn_bias is None else
                     case.attn_bias[seqs.to(case.attn_bias.device)].cpu())
    sub.num_blocks = int(used.numel())
    return sub


def sample_prefill(case, seqs):
    """Oracle inputs for a subset of sequences of a prefill case (packed q
    rows re-packed, a compact cache, remapped tables)."""
    seqs = [int(s) for s in seqs]
    qsl = case.query_start_loc.cpu()
    rows = torch.cat([torch.arange(int(qsl[s]), int(qsl[s + 1])) for s in seqs])
    nq = torch.tensor([int(qsl[s + 1] - qsl[s]) for s in seqs], dtype=torch.int32)
    new_qsl = torch.zeros(len(seqs) + 1, dtype=torch.int32)
    new_qsl[1:] = torch.cumsum(nq, 0)
    idx = torch.tensor(seqs, dtype=torch.long)
    bt = case.block_tables.cpu()[idx]
    used = torch.unique(bt)
    remap = torch.full((case.num_blocks,), -1, dtype=torch.int32)
    remap[used] = torch.arange(used.numel(), dtype=torch.int32)
    sub = SimpleNamespace(**vars(case))
    sub.q = case.q[rows.to(case.q.device)].cpu()
    sub.k_cache = case.k_cache[used.to(case.k_cache.device)].cpu()
    sub.v_cache = case.v_cache[used.to(case.v_cache.device)].cpu()
    sub.block_tables = remap[bt.long()]
    sub.context_lens = case.context_lens.cpu()[idx]
    sub.query_start_loc = new_qsl
    sub.attn_bias = None if case.attn_bias is None else case.attn_bias[idx.to(
        case.attn_bias.device)].cpu()
    sub.num_seqs = len(seqs)
    sub.rows = rows
    return sub
