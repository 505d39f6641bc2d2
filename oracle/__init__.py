"""Float64 CPU oracle for biased, windowed paged attention (ctypes binding).

TEST INFRASTRUCTURE ONLY. Only the tests, ``__graft_entry__.smoke()`` and the
benchmark's ``cpu_baseline`` leg may import this package. The product path
(``sliding_window_mask_amd``) never imports it, and the two share no code.

The arithmetic lives in ``oracle.c`` (plain loops in float64, OpenMP over
(sequence, head)); see ``oracle.h`` for the semantics, the layouts and the
readings taken where the pages are silent. This module only builds the C file
with gcc and passes numpy arrays to it.

Every function here is pinned by ``tests/test_oracle_pins.py`` against things
that do not come from the oracle itself: PyTorch's float64
``scaled_dot_product_attention`` on the un-paged tensors, hand-worked examples
under ``tests/golden/``, and closed-form special cases.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
# PA_ORACLE_LIB points the tests at another build of oracle.c (the mutation
# test loads copies with planted mistakes this way)
_LIB = os.environ.get("PA_ORACLE_LIB") or os.path.join(_HERE, "liboracle.so")
_lib = None

DTYPE_F32 = 0
DTYPE_BF16 = 1


def build(force: bool = True) -> str:
    """Compile oracle.c into liboracle.so with gcc (no fast-math)."""
    if force or not os.path.exists(_LIB):
        tmp = _LIB + ".tmp%d" % os.getpid()
        cmd = ["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-std=c11", "-Wall",
               "-Wextra", "-o", tmp, _SRC, "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(tmp, _LIB)
    return _LIB


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB):
            build()
        lib = ctypes.CDLL(_LIB)
        P, I32, F64 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_double
        lib.oracle_decode_f64.restype = ctypes.c_int
        lib.oracle_decode_f64.argtypes = [P, P, P, P, P, P, P, I32, F64,
                                          I32, I32, I32, I32, I32, I32, I32]
        lib.oracle_prefill_f64.restype = ctypes.c_int
        lib.oracle_prefill_f64.argtypes = [P, P, P, P, P, P, P, P, I32, I32, F64,
                                           I32, I32, I32, I32, I32, I32, I32]
        lib.oracle_decode_chunked_f64.restype = ctypes.c_int
        lib.oracle_decode_chunked_f64.argtypes = lib.oracle_decode_f64.argtypes
        lib.oracle_prefill_chunked_f64.restype = ctypes.c_int
        lib.oracle_prefill_chunked_f64.argtypes = lib.oracle_prefill_f64.argtypes
        lib.oracle_t5_bucket_array.restype = None
        lib.oracle_t5_bucket_array.argtypes = [P, ctypes.c_int64, I32, I32, I32, P]
        lib.oracle_decode_relpos_f64.restype = ctypes.c_int
        lib.oracle_decode_relpos_f64.argtypes = [P, P, P, P, P, P, P, I32, I32, I32, I32, F64,
                                                 I32, I32, I32, I32, I32, I32, I32]
        lib.oracle_prefill_relpos_f64.restype = ctypes.c_int
        lib.oracle_prefill_relpos_f64.argtypes = [P, P, P, P, P, P, P, P, I32, I32, I32, I32,
                                                  I32, F64, I32, I32, I32, I32, I32, I32, I32]
        lib.oracle_decode_ragged_f64.restype = ctypes.c_int
        lib.oracle_decode_ragged_f64.argtypes = [P, P, P, P, P, P, P, P, I32, F64, I32, I32,
                                                 I32, I32, I32, I32, I32]
        lib.oracle_prefill_ragged_f64.restype = ctypes.c_int
        lib.oracle_prefill_ragged_f64.argtypes = [P, P, P, P, P, P, P, P, P, I32, I32, F64, I32,
                                                  I32, I32, I32, I32, I32, I32]
        lib.oracle_kv_write.restype = ctypes.c_int
        lib.oracle_kv_write.argtypes = [P, P, P, P, P, ctypes.c_int64, I32, I32, I32,
                                        ctypes.c_int64, I32]
        lib.oracle_num_threads.restype = ctypes.c_int
        lib.oracle_set_num_threads.restype = None
        lib.oracle_set_num_threads.argtypes = [ctypes.c_int]
        _lib = lib
    return _lib


def num_threads() -> int:
    return int(_load().oracle_num_threads())


def set_num_threads(n: int) -> None:
    """Threads for the following oracle calls (timing only; every row is
    computed the same way whatever the count)."""
    _load().oracle_set_num_threads(int(n))


def _host(a, dtype=None):
    """A C-contiguous host numpy view of a numpy array or CPU torch tensor.

    bf16 torch tensors are passed as their raw 16-bit patterns (the C code
    widens them exactly)."""
    if a is None:
        return None
    if not isinstance(a, np.ndarray):
        import torch  # local: the oracle itself does not need torch
        t = a.detach()
        if t.device.type != "cpu":
            raise ValueError("oracle inputs must be host (CPU) arrays")
        if t.dtype == torch.bfloat16:
            t = t.contiguous().view(torch.int16)
        a = t.contiguous().numpy()
    a = np.ascontiguousarray(a)
    if dtype is not None and a.dtype != dtype:
        raise TypeError("expected %s, got %s" % (dtype, a.dtype))
    return a


def _kv_dtype(a) -> int:
    if isinstance(a, np.ndarray):
        if a.dtype == np.float32:
            return DTYPE_F32
        if a.dtype in (np.uint16, np.int16):
            return DTYPE_BF16
    else:
        import torch
        if a.dtype == torch.float32:
            return DTYPE_F32
        if a.dtype == torch.bfloat16:
            return DTYPE_BF16
    raise TypeError("oracle supports fp32 and bf16 inputs, got %s" % (a.dtype,))


def _ptr(a):
    return None if a is None else a.ctypes.data


def decode(q, k_cache, v_cache, block_tables, context_lens, attn_bias, sliding_window,
           scale, max_seq_len):
    """Float64 decode attention: one query per (sequence, head) at position L-1.

    q [B,H,D]; k_cache, v_cache [num_blocks,H,block_size,D] (fp32 or bf16);
    block_tables int32 [B,max_blocks]; context_lens int32 [B];
    attn_bias fp32 [B,H,max_seq_len] or None. Returns float64 [B,H,D]."""
    dt = _kv_dtype(q)
    qh, kh, vh = _host(q), _host(k_cache), _host(v_cache)
    bt = _host(block_tables, np.int32)
    cl = _host(context_lens, np.int32)
    ab = _host(attn_bias, np.float32)
    B, H, D = qh.shape
    bs = kh.shape[2]
    out = np.zeros((B, H, D), dtype=np.float64)
    rc = _load().oracle_decode_f64(
        _ptr(out), _ptr(qh), _ptr(kh), _ptr(vh), _ptr(bt), _ptr(cl), _ptr(ab),
        int(sliding_window), float(scale), B, H, D, bs, bt.shape[1] if bt.ndim == 2 else 0,
        int(max_seq_len), dt)
    if rc != 0:
        raise ValueError("oracle_decode_f64 rejected its arguments")
    return out


def prefill(q, k_cache, v_cache, block_tables, context_lens, query_start_loc, attn_bias,
            sliding_window, causal, scale, max_seq_len):
    """Float64 prefill attention over packed queries q [total_q,H,D].

    Query t of sequence b (rows query_start_loc[b] ..) sits at position
    L_b - n_q + t. attn_bias fp32 [B,H,max_seq_len,max_seq_len] or None.
    Returns float64 [total_q,H,D]."""
    dt = _kv_dtype(q)
    qh, kh, vh = _host(q), _host(k_cache), _host(v_cache)
    bt = _host(block_tables, np.int32)
    cl = _host(context_lens, np.int32)
    qsl = _host(query_start_loc, np.int32)
    ab = _host(attn_bias, np.float32)
    TQ, H, D = qh.shape
    B = cl.shape[0]
    bs = kh.shape[2]
    out = np.zeros((TQ, H, D), dtype=np.float64)
    rc = _load().oracle_prefill_f64(
        _ptr(out), _ptr(qh), _ptr(kh), _ptr(vh), _ptr(bt), _ptr(cl), _ptr(qsl), _ptr(ab),
        int(sliding_window), int(causal), float(scale), B, H, D, bs,
        bt.shape[1] if bt.ndim == 2 else 0, int(max_seq_len), dt)
    if rc != 0:
        raise ValueError("oracle_prefill_f64 rejected its arguments")
    return out


def decode_chunked(q, k_cache, v_cache, block_tables, context_lens, attn_bias, chunk_size,
                   scale, max_seq_len):
    """Float64 decode with chunked local attention (no window): the query at
    position L-1 sees keys chunk_size * floor((L-1) / chunk_size) .. L-1.
    Arguments and result as in decode()."""
    dt = _kv_dtype(q)
    qh, kh, vh = _host(q), _host(k_cache), _host(v_cache)
    bt = _host(block_tables, np.int32)
    cl = _host(context_lens, np.int32)
    ab = _host(attn_bias, np.float32)
    B, H, D = qh.shape
    out = np.zeros((B, H, D), dtype=np.float64)
    rc = _load().oracle_decode_chunked_f64(
        _ptr(out), _ptr(qh), _ptr(kh), _ptr(vh), _ptr(bt), _ptr(cl), _ptr(ab),
        int(chunk_size), float(scale), B, H, D, kh.shape[2],
        bt.shape[1] if bt.ndim == 2 else 0, int(max_seq_len), dt)
    if rc != 0:
        raise ValueError("oracle_decode_chunked_f64 rejected its arguments")
    return out


def prefill_chunked(q, k_cache, v_cache, block_tables, context_lens, query_start_loc,
                    attn_bias, chunk_size, causal, scale, max_seq_len):
    """Float64 prefill with chunked local attention (no window): a query at
    position p sees the keys j with floor(j / chunk_size) = floor(p /
    chunk_size), and j <= p when causal. Arguments and result as in
    prefill()."""
    dt = _kv_dtype(q)
    qh, kh, vh = _host(q), _host(k_cache), _host(v_cache)
    bt = _host(block_tables, np.int32)
    cl = _host(context_lens, np.int32)
    qsl = _host(query_start_loc, np.int32)
    ab = _host(attn_bias, np.float32)
    TQ, H, D = qh.shape
    B = cl.shape[0]
    out = np.zeros((TQ, H, D), dtype=np.float64)
    rc = _load().oracle_prefill_chunked_f64(
        _ptr(out), _ptr(qh), _ptr(kh), _ptr(vh), _ptr(bt), _ptr(cl), _ptr(qsl), _ptr(ab),
        int(chunk_size), int(causal), float(scale), B, H, D, kh.shape[2],
        bt.shape[1] if bt.ndim == 2 else 0, int(max_seq_len), dt)
    if rc != 0:
        raise ValueError("oracle_prefill_chunked_f64 rejected its arguments")
    return out


def t5_bucket(relative_position, bidirectional, num_buckets, max_distance):
    """T5 relative-position buckets (float64 evaluation) of key - query positions."""
    rp = np.ascontiguousarray(np.asarray(relative_position, dtype=np.int64))
    out = np.empty(rp.shape, dtype=np.int32)
    _load().oracle_t5_bucket_array(_ptr(rp), int(rp.size), int(bidirectional),
                                   int(num_buckets), int(max_distance), _ptr(out))
    return out


def decode_relpos(q, k_cache, v_cache, block_tables, context_lens, rel_table, num_buckets,
                  max_distance, bidirectional, sliding_window, scale, max_seq_len):
    """Float64 decode with the bias a_j = rel_table[h][bucket(j - (L-1))]."""
    dt = _kv_dtype(q)
    qh, kh, vh = _host(q), _host(k_cache), _host(v_cache)
    bt = _host(block_tables, np.int32)
    cl = _host(context_lens, np.int32)
    tab = _host(rel_table, np.float32)
    B, H, D = qh.shape
    out = np.zeros((B, H, D), dtype=np.float64)
    rc = _load().oracle_decode_relpos_f64(
        _ptr(out), _ptr(qh), _ptr(kh), _ptr(vh), _ptr(bt), _ptr(cl), _ptr(tab),
        int(num_buckets), int(max_distance), int(bidirectional), int(sliding_window),
        float(scale), B, H, D, kh.shape[2], bt.shape[1], int(max_seq_len), dt)
    if rc != 0:
        raise ValueError("oracle_decode_relpos_f64 rejected its arguments")
    return out


def prefill_relpos(q, k_cache, v_cache, block_tables, context_lens, query_start_loc, rel_table,
                   num_buckets, max_distance, bidirectional, sliding_window, causal, scale,
                   max_seq_len):
    """Float64 prefill with the bias a(p, j) = rel_table[h][bucket(j - p)]."""
    dt = _kv_dtype(q)
    qh, kh, vh = _host(q), _host(k_cache), _host(v_cache)
    bt = _host(block_tables, np.int32)
    cl = _host(context_lens, np.int32)
    qsl = _host(query_start_loc, np.int32)
    tab = _host(rel_table, np.float32)
    TQ, H, D = qh.shape
    B = cl.shape[0]
    out = np.zeros((TQ, H, D), dtype=np.float64)
    rc = _load().oracle_prefill_relpos_f64(
        _ptr(out), _ptr(qh), _ptr(kh), _ptr(vh), _ptr(bt), _ptr(cl), _ptr(qsl), _ptr(tab),
        int(num_buckets), int(max_distance), int(bidirectional), int(sliding_window),
        int(causal), float(scale), B, H, D, kh.shape[2], bt.shape[1], int(max_seq_len), dt)
    if rc != 0:
        raise ValueError("oracle_prefill_relpos_f64 rejected its arguments")
    return out


def kv_write(k_cache, v_cache, k_new, v_new, slot_mapping):
    """Return copies of the host caches with the new rows scattered in.

    k_cache, v_cache [num_blocks, H, block_size, D]; k_new, v_new [T, H, D];
    slot_mapping int64 [T] (block * block_size + offset, negative = skip)."""
    dt = _kv_dtype(k_cache)
    kc, vc = _host(k_cache).copy(), _host(v_cache).copy()
    kn, vn = _host(k_new), _host(v_new)
    sm = _host(slot_mapping, np.int64)
    nb, H, bs, D = kc.shape
    rc = _load().oracle_kv_write(_ptr(kc), _ptr(vc), _ptr(kn), _ptr(vn), _ptr(sm),
                                 int(sm.shape[0]), H, D, bs, nb, dt)
    if rc != 0:
        raise ValueError("oracle_kv_write rejected its arguments")
    return kc, vc


def decode_ragged(q, k_cache, v_cache, block_tables, context_lens, bias, bias_start,
                  sliding_window, scale, max_seq_len):
    """Float64 decode with a ragged bias: sequence b's rows [H][L_b] start at
    bias[bias_start[b]]."""
    dt = _kv_dtype(q)
    qh, kh, vh = _host(q), _host(k_cache), _host(v_cache)
    bt = _host(block_tables, np.int32)
    cl = _host(context_lens, np.int32)
    bb, bs0 = _host(bias, np.float32), _host(bias_start, np.int64)
    B, H, D = qh.shape
    out = np.zeros((B, H, D), dtype=np.float64)
    rc = _load().oracle_decode_ragged_f64(
        _ptr(out), _ptr(qh), _ptr(kh), _ptr(vh), _ptr(bt), _ptr(cl), _ptr(bb), _ptr(bs0),
        int(sliding_window), float(scale), B, H, D, kh.shape[2], bt.shape[1],
        int(max_seq_len), dt)
    if rc != 0:
        raise ValueError("oracle_decode_ragged_f64 rejected its arguments")
    return out


def prefill_ragged(q, k_cache, v_cache, block_tables, context_lens, query_start_loc, bias,
                   bias_start, sliding_window, causal, scale, max_seq_len):
    """Float64 prefill with a ragged bias: sequence b's rows [H][n_q][L_b]
    start at bias[bias_start[b]]."""
    dt = _kv_dtype(q)
    qh, kh, vh = _host(q), _host(k_cache), _host(v_cache)
    bt = _host(block_tables, np.int32)
    cl = _host(context_lens, np.int32)
    qsl = _host(query_start_loc, np.int32)
    bb, bs0 = _host(bias, np.float32), _host(bias_start, np.int64)
    TQ, H, D = qh.shape
    out = np.zeros((TQ, H, D), dtype=np.float64)
    rc = _load().oracle_prefill_ragged_f64(
        _ptr(out), _ptr(qh), _ptr(kh), _ptr(vh), _ptr(bt), _ptr(cl), _ptr(qsl), _ptr(bb),
        _ptr(bs0), int(sliding_window), int(causal), float(scale), cl.shape[0], H, D,
        kh.shape[2], bt.shape[1], int(max_seq_len), dt)
    if rc != 0:
        raise ValueError("oracle_prefill_ragged_f64 rejected its arguments")
    return out
