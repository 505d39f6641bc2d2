"""Seeded synthetic inputs for paged attention (shared by the tests and the bench).

This module only draws and lays out inputs; it holds none of the attention
arithmetic. Both sides of every comparison (the HIP library and the float64
oracle) consume exactly the tensors built here.

Recipe (all five workloads follow it):

1. ``context_lens`` = ``numpy.random.default_rng(seed).integers(lo, hi,
   endpoint=True)``: uniform lengths.
2. Physical blocks: ``rng.permutation(num_blocks)``; sequence b takes the next
   ``ceil(L_b / 16)`` ids in order, then any decoy sequences (a second,
   never-passed table), then one *poison* block. Block-table padding points at
   the poison block. This mimics a block-table KV cache whose blocks are
   scattered over the pool (the paged layout of the T5 encoder-decoder work,
   "Add Encoder-decoder model support and T5 Model support", block-table
   discussion).
3. Dense values from ``torch.Generator(device).manual_seed(seed)``: q, then K,
   then V (``standard normal`` in fp32, rounded to bf16 with round-to-nearest-
   even when the workload is bf16), then the bias.
4. Poisoning: every cache slot that holds no valid token (the tail of a
   sequence's last block, unused blocks, the poison block, decoy blocks) and
   every bias entry past a sequence's length is NaN, so any over-read shows.
   With ``evict_before`` a decode workload also NaN-fills the blocks that lie
   wholly before the window (and the bias there) and points their table
   entries at the poison block: the situation of a cache that has evicted
   out-of-window blocks ("[V1] Add sliding window support to Flex Attention
   backend", review remark that in-window iteration may skip evicted blocks).

KV cache layout: ``[num_blocks, num_heads, 16, head_dim]`` for K and V.
Bias layout: decode ``[B, H, max_seq_len]``, prefill ``[B, H, max_seq_len,
max_seq_len]``, fp32, indexed by logical positions.
"""
from __future__ import annotations

import math
from types import SimpleNamespace

import numpy as np
import torch

BLOCK_SIZE = 16


# ----------------------------------------------------------------------------
# T5 relative-position buckets (input synthesis for the T5-shaped workload)
# ----------------------------------------------------------------------------
T5_NUM_BUCKETS = 32
T5_MAX_DISTANCE = 128


def t5_bucket(distance) -> np.ndarray:
    """Unidirectional T5 relative-position bucket of ``distance = i - j``.

    Half of the 32 buckets hold the exact distances 0..15; the other half are
    logarithmically spaced up to the maximum distance 128, beyond which every
    distance shares the last bucket (the clamp described in the custom-bias
    thread, "PagedAttention: Support custom attention bias for T5 model",
    T5 max-distance remark). Negative distances (future keys) map to bucket 0.
    Evaluated in float64."""
    n = np.maximum(np.asarray(distance, dtype=np.int64), 0)
    exact = T5_NUM_BUCKETS // 2
    with np.errstate(divide="ignore"):
        logb = exact + np.floor(
            np.log(np.maximum(n, 1) / exact) / math.log(T5_MAX_DISTANCE / exact) * exact)
    logb = np.minimum(logb, T5_NUM_BUCKETS - 1).astype(np.int64)
    return np.where(n < exact, n, logb)


def t5_decode_bias(table: torch.Tensor, lens: np.ndarray, max_seq_len: int) -> torch.Tensor:
    """Materialise a decode bias [B,H,max_seq_len] from a bucket table [H,32]:
    bias[b,h,j] = table[h, bucket(L_b - 1 - j)] for j < L_b, NaN beyond."""
    H = table.shape[0]
    B = len(lens)
    j = np.arange(max_seq_len)
    dist = (lens[:, None].astype(np.int64) - 1) - j[None, :]
    bucket = torch.from_numpy(t5_bucket(dist)).to(table.device)          # [B, MS]
    bias = table[:, bucket].permute(1, 0, 2).contiguous()               # [B, H, MS]
    pad = torch.from_numpy(j[None, :] >= lens[:, None]).to(table.device)
    bias.masked_fill_(pad[:, None, :].expand(B, H, max_seq_len), float("nan"))
    return bias


# ----------------------------------------------------------------------------
# generic builders
# ----------------------------------------------------------------------------
def _torch_seed(seed) -> int:
    return int(np.random.default_rng(seed).integers(0, 2**62))


def _randn(shape, gen, device, dtype, chunk_rows=None):
    """fp32 standard normals rounded to `dtype`, drawn in chunks along dim 0."""
    out = torch.empty(shape, dtype=dtype, device=device)
    n = shape[0]
    step = max(1, n) if chunk_rows is None else max(1, chunk_rows)   # n = 0: empty
    for s in range(0, n, step):
        e = min(n, s + step)
        out[s:e] = torch.randn((e - s,) + tuple(shape[1:]), generator=gen, device=device,
                               dtype=torch.float32).to(dtype)
    return out


def _assign_blocks(rng, lens, max_blocks, num_blocks=None, decoy_lens=None):
    need = -(-lens // BLOCK_SIZE)
    dneed = np.zeros(0, np.int64) if decoy_lens is None else -(-decoy_lens // BLOCK_SIZE)
    used = int(need.sum() + dneed.sum()) + 1
    if num_blocks is None:
        num_blocks = used
    if num_blocks < used:
        raise ValueError("block pool too small")
    perm = rng.permutation(num_blocks).astype(np.int32)
    cur = 0
    table = np.empty((len(lens), max_blocks), np.int32)
    owned = []
    for b, n in enumerate(need):
        owned.append(perm[cur:cur + n])
        cur += int(n)
    dtable = None
    if decoy_lens is not None:
        dtable = np.empty((len(decoy_lens), max_blocks), np.int32)
        downed = []
        for b, n in enumerate(dneed):
            downed.append(perm[cur:cur + n])
            cur += int(n)
    poison = int(perm[cur])
    for b, ids in enumerate(owned):
        table[b, :] = poison
        table[b, :len(ids)] = ids
    if decoy_lens is not None:
        for b, ids in enumerate(downed):
            dtable[b, :] = poison
            dtable[b, :len(ids)] = ids
    return table, dtable, poison, num_blocks


def _valid_slots(table, lens, num_blocks, first_block=None):
    """Boolean [num_blocks, 16]: slot holds a token some sequence may read."""
    valid = np.zeros((num_blocks, BLOCK_SIZE), dtype=bool)
    for b, L in enumerate(lens):
        L = int(L)
        if L == 0:
            continue
        nb = -(-L // BLOCK_SIZE)
        n0 = 0 if first_block is None else int(first_block[b])
        for n in range(n0, nb):
            cnt = min(BLOCK_SIZE, L - n * BLOCK_SIZE)
            valid[table[b, n], :cnt] = True
    return valid


def _poison(cache, valid_np):
    valid = torch.from_numpy(valid_np).to(cache.device)
    cache.masked_fill_(~valid[:, None, :, None], float("nan"))


def decode_case(seed, *, num_seqs, num_heads, head_dim, lens, max_seq_len, dtype,
                bias="normal", sliding_window=-1, num_blocks=None, decoy_lens=None,
                evict_before=None, device="cpu", scale=None, chunk_rows=4096):
    """Build one decode workload.

    lens: (lo, hi) inclusive range for the uniform lengths, or an explicit
    sequence of lengths. bias: "normal" (N(0,1)), "t5" (bucket table
    N(0, sd 0.5)), "zero", or None. evict_before: a window size W whose
    out-of-window blocks are poisoned and unmapped (see module docstring)."""
    rng = np.random.default_rng(seed)
    if isinstance(lens, tuple) and len(lens) == 2:
        L = rng.integers(lens[0], lens[1], endpoint=True, size=num_seqs).astype(np.int32)
    else:
        L = np.asarray(lens, dtype=np.int32)
        assert L.shape == (num_seqs,)
    dl = None
    if decoy_lens is not None:
        dl = rng.integers(decoy_lens[0], decoy_lens[1], endpoint=True,
                          size=num_seqs).astype(np.int32)
    max_blocks = -(-max_seq_len // BLOCK_SIZE)
    table, dtable, poison, nb = _assign_blocks(rng, L.astype(np.int64), max_blocks,
                                               num_blocks, None if dl is None else
                                               dl.astype(np.int64))
    first = None
    if evict_before is not None:
        lo = np.maximum(L.astype(np.int64) - int(evict_before), 0)
        first = lo // BLOCK_SIZE
        for b in range(num_seqs):
            table[b, :first[b]] = poison
    g = torch.Generator(device=device).manual_seed(_torch_seed(seed))
    q = _randn((num_seqs, num_heads, head_dim), g, device, dtype)
    kv_shape = (nb, num_heads, BLOCK_SIZE, head_dim)
    k = _randn(kv_shape, g, device, dtype, chunk_rows)
    v = _randn(kv_shape, g, device, dtype, chunk_rows)
    valid = _valid_slots(table, L, nb, first)
    _poison(k, valid)
    _poison(v, valid)
    pad = np.arange(max_seq_len)[None, :] >= L[:, None]
    if first is not None:
        pad |= np.arange(max_seq_len)[None, :] < (first * BLOCK_SIZE)[:, None]
    pad_t = torch.from_numpy(pad).to(device)[:, None, :].expand(num_seqs, num_heads,
                                                                 max_seq_len)
    attn_bias = None
    t5_table = None
    if bias == "normal":
        attn_bias = torch.randn((num_seqs, num_heads, max_seq_len), generator=g, device=device,
                                dtype=torch.float32)
        attn_bias.masked_fill_(pad_t, float("nan"))
    elif bias == "zero":
        attn_bias = torch.zeros((num_seqs, num_heads, max_seq_len), device=device)
        attn_bias.masked_fill_(pad_t, float("nan"))
    elif bias == "t5":
        t5_table = torch.randn((num_heads, T5_NUM_BUCKETS), generator=g, device=device,
                               dtype=torch.float32) * 0.5
        attn_bias = t5_decode_bias(t5_table, L, max_seq_len)
        if first is not None:
            attn_bias.masked_fill_(pad_t, float("nan"))
    elif bias is not None:
        raise ValueError(bias)
    return SimpleNamespace(
        kind="decode", q=q, k_cache=k, v_cache=v,
        block_tables=torch.from_numpy(table).to(device),
        context_lens=torch.from_numpy(L).to(device),
        attn_bias=attn_bias, sliding_window=int(sliding_window),
        scale=float(np.float32(1.0 / math.sqrt(head_dim)) if scale is None else
                    np.float32(scale)),
        max_seq_len=int(max_seq_len), num_blocks=int(nb), poison_block=poison,
        lens=L, decoy_table=None if dtable is None else torch.from_numpy(dtable).to(device),
        decoy_lens=dl, t5_table=t5_table, num_seqs=num_seqs, num_heads=num_heads,
        head_dim=head_dim, dtype=dtype)


def prefill_case(seed, *, num_seqs, num_heads, head_dim, lens, max_seq_len, dtype,
                 bias=None, sliding_window=-1, causal=False, q_lens=None, device="cpu",
                 scale=None, layer_seed=None):
    """Build one prefill workload: packed queries [total_q,H,D] with
    query_start_loc; by default every sequence queries all of its positions
    (encoder-only). q_lens (optional, explicit) gives fewer queries: the last
    n_q positions. layer_seed: seed for the dense tensors (lengths and block
    assignment still come from `seed`), so layers can share one layout."""
    rng = np.random.default_rng(seed)
    if isinstance(lens, tuple) and len(lens) == 2:
        L = rng.integers(lens[0], lens[1], endpoint=True, size=num_seqs).astype(np.int32)
    else:
        L = np.asarray(lens, dtype=np.int32)
        assert L.shape == (num_seqs,)
    nq = L.copy() if q_lens is None else np.asarray(q_lens, dtype=np.int32)
    assert np.all(nq <= L) and np.all(nq >= 0)
    max_blocks = -(-max_seq_len // BLOCK_SIZE)
    table, _, poison, nb = _assign_blocks(rng, L.astype(np.int64), max_blocks)
    qsl = np.zeros(num_seqs + 1, np.int32)
    qsl[1:] = np.cumsum(nq)
    total_q = int(qsl[-1])
    g = torch.Generator(device=device).manual_seed(
        _torch_seed(seed if layer_seed is None else layer_seed))
    q = _randn((total_q, num_heads, head_dim), g, device, dtype)
    kv_shape = (nb, num_heads, BLOCK_SIZE, head_dim)
    k = _randn(kv_shape, g, device, dtype)
    v = _randn(kv_shape, g, device, dtype)
    valid = _valid_slots(table, L, nb)
    _poison(k, valid)
    _poison(v, valid)
    attn_bias = None
    if bias == "normal":
        attn_bias = torch.randn((num_seqs, num_heads, max_seq_len, max_seq_len), generator=g,
                                device=device, dtype=torch.float32)
        pos = np.arange(max_seq_len)
        pad = (pos[None, :, None] >= L[:, None, None]) | (pos[None, None, :] >= L[:, None, None])
        attn_bias.masked_fill_(torch.from_numpy(pad).to(device)[:, None], float("nan"))
    elif bias is not None:
        raise ValueError(bias)
    return SimpleNamespace(
        kind="prefill", q=q, k_cache=k, v_cache=v,
        block_tables=torch.from_numpy(table).to(device),
        context_lens=torch.from_numpy(L).to(device),
        query_start_loc=torch.from_numpy(qsl).to(device),
        attn_bias=attn_bias, sliding_window=int(sliding_window), causal=bool(causal),
        scale=float(np.float32(1.0 / math.sqrt(head_dim)) if scale is None else
                    np.float32(scale)),
        max_seq_len=int(max_seq_len), num_blocks=int(nb), poison_block=poison, lens=L,
        q_lens=nq, total_q=total_q, num_seqs=num_seqs, num_heads=num_heads,
        head_dim=head_dim, dtype=dtype)


# ----------------------------------------------------------------------------
# the five named workloads
# ----------------------------------------------------------------------------
MODERNBERT_LAYERS = 12
MODERNBERT_WINDOW = 64


def modernbert_window(layer: int) -> int:
    """Layer schedule of the ModernBERT-based reranker discussed in the Flex
    Attention sliding-window review: every third layer (0, 3, 6, ...) is full
    attention, the others use a sliding window of 64."""
    return -1 if layer % 3 == 0 else MODERNBERT_WINDOW


def tiny_decode_f32(device="cpu", bias="normal"):
    """B=4, H=4, D=64, fp32, L ~ U[1,100], 64-block pool, bias [4,4,128]
    N(0,1) padded to max_seq_len=128, scale 1/8, no window."""
    return decode_case(1, num_seqs=4, num_heads=4, head_dim=64, lens=(1, 100),
                       max_seq_len=128, dtype=torch.float32, bias=bias, num_blocks=64,
                       device=device, scale=0.125)


def t5_small_self_decode_bf16(device="cpu"):
    """T5-small-shaped decoder self-attention decode: B=64, H=8, D=64, bf16,
    L ~ U[32,512], bias materialised from a 32-bucket T5 table (max distance
    128, bucket values N(0, sd 0.5)) into [64,8,512]."""
    return decode_case(2, num_seqs=64, num_heads=8, head_dim=64, lens=(32, 512),
                       max_seq_len=512, dtype=torch.bfloat16, bias="t5", device=device)


def t5_large_cross_decode_bf16(device="cpu", bias=None):
    """T5-large-shaped cross-attention decode: B=256, H=16, D=64, bf16, encoder
    lengths U[128,512] in a cross-attention block table; the pool also holds
    NaN-filled self-attention blocks (lengths U[1,64]) owned by a separate
    table that is never passed. bias None or "zero"."""
    return decode_case(3, num_seqs=256, num_heads=16, head_dim=64, lens=(128, 512),
                       max_seq_len=512, dtype=torch.bfloat16, bias=bias,
                       decoy_lens=(1, 64), device=device)


def modernbert_prefill_f32(layer, device="cpu", num_seqs=32, lens=(64, 1024)):
    """ModernBERT-base-shaped encoder-only bidirectional prefill, one layer:
    H=12, D=64, fp32, B=32, L ~ U[64,1024] (the same lengths and block layout
    for every layer), per-layer q/k/v, no bias, window per modernbert_window."""
    return prefill_case(4, num_seqs=num_seqs, num_heads=12, head_dim=64, lens=lens,
                        max_seq_len=1024, dtype=torch.float32, bias=None,
                        sliding_window=modernbert_window(layer), device=device,
                        layer_seed=[4, int(layer)])


def large_biased_decode_bf16(device="cpu", sliding_window=-1, bias="normal",
                             num_seqs=256, evict=False):
    """B=256, H=32, D=128, bf16 q/K/V, fp32 bias [256,32,4096] N(0,1),
    L ~ U[1024,4096], random block permutation; optional window (1024)."""
    return decode_case(5, num_seqs=num_seqs, num_heads=32, head_dim=128, lens=(1024, 4096),
                       max_seq_len=4096, dtype=torch.bfloat16, bias=bias,
                       sliding_window=sliding_window, device=device,
                       evict_before=(sliding_window if evict and sliding_window > 0 else None))
