"""Python binding of libpaged_attn.so (biased, windowed paged attention on MI355X).

Argument marshalling only: every step of the computation runs in the HIP
kernels behind the C ABI declared in ``include/paged_attn.h``. PyTorch is used
for device memory and streams; tensors are passed as raw pointers together
with the current HIP stream. There is no CPU or PyTorch fallback: if the
library is not built, or a call fails, an exception is raised.

Functions mirror the C entry points:
  paged_attn_decode(...)         decoder self-attention / cross-attention decode
  paged_attn_decode_noalloc(...) the same without a workspace or any device allocation
  paged_attn_prefill(...)        encoder-only (bidirectional) or causal prefill
  paged_attn_decode_relpos(...)  decode with the T5 relative-position bias in-kernel
  paged_attn_prefill_relpos(...) prefill with the T5 relative-position bias in-kernel
  paged_attn_decode_ragged_bias(...), paged_attn_prefill_ragged_bias(...)
                                 the same with an unpadded (packed) bias
  paged_kv_write(...)            scatter new tokens' K/V into the paged caches
  pa_window_first_live_block(...) first block a windowed decode still reads
  pa_decode_workspace_bytes(...)
  pa_decode_default_partition(...)
  pa_check_metadata(...)         host-side range check of lengths / tables
  pa_abi_version()
"""
from __future__ import annotations

import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
# PA_LIB points the binding at another build of the same sources (the CPU
# sanitizer test loads a host-only AddressSanitizer build this way)
LIB_PATH = os.environ.get("PA_LIB") or os.path.join(_HERE, "libpaged_attn.so")
LIB_NOBIAS_PATH = os.path.join(_HERE, "libpaged_attn_nobias.so")

PA_DTYPE_F32 = 0
PA_DTYPE_BF16 = 1
STATUS = {0: "PA_OK", 1: "PA_ERR_NULL_POINTER", 2: "PA_ERR_INVALID_ARG",
          3: "PA_ERR_UNSUPPORTED", 4: "PA_ERR_MISALIGNED", 5: "PA_ERR_WORKSPACE",
          6: "PA_ERR_HIP"}


class PagedAttnError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__("%s: %s" % (STATUS.get(status, status), message))
        self.status = status


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.float32:
        return PA_DTYPE_F32
    if t.dtype == torch.bfloat16:
        return PA_DTYPE_BF16
    raise TypeError("paged attention supports float32 and bfloat16, got %s" % t.dtype)


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _tensor(t, name, device, dtypes=None, shape=None, ndim=None):
    """Check one tensor argument before its pointer crosses the ABI: a device
    (HIP) tensor on `device`, contiguous, of one of `dtypes`, with `shape`
    (None entries unchecked) or `ndim` dimensions. The kernels read raw
    pointers with the documented row-major layout, so a host tensor or a
    strided view would be read as garbage (or fault); it is rejected here."""
    if not isinstance(t, torch.Tensor):
        raise TypeError("%s must be a torch.Tensor, got %s" % (name, type(t).__name__))
    if t.device.type != "cuda" or (device is not None and t.device != device):
        raise ValueError("%s must be a tensor on %s, got %s" % (name, device or "the GPU",
                                                               t.device))
    if dtypes is not None and t.dtype not in dtypes:
        raise TypeError("%s must be %s, got %s" % (name, " or ".join(map(str, dtypes)),
                                                   t.dtype))
    if shape is not None:
        ok = t.dim() == len(shape) and all(w is None or t.shape[i] == w
                                           for i, w in enumerate(shape))
        if not ok:
            raise ValueError("%s must have shape %s, got %s"
                             % (name, tuple("*" if w is None else w for w in shape),
                                tuple(t.shape)))
    elif ndim is not None and t.dim() != ndim:
        raise ValueError("%s must have %d dimensions, got %d" % (name, ndim, t.dim()))
    if not t.is_contiguous():
        raise ValueError("%s must be contiguous" % name)


_FLOAT_DTYPES = (torch.float32, torch.bfloat16)


def _check_attention_args(q, k_cache, v_cache, block_tables, context_lens, out,
                          query_start_loc=None, num_seqs=None):
    """Common checks of decode/prefill tensors; returns q's device."""
    _tensor(q, "q", None, _FLOAT_DTYPES, ndim=3)
    dev = q.device
    _, H, D = q.shape
    _tensor(k_cache, "k_cache", dev, (q.dtype,), shape=(None, None, None, D))
    _tensor(v_cache, "v_cache", dev, (q.dtype,), shape=tuple(k_cache.shape))
    B = num_seqs if num_seqs is not None else q.shape[0]
    _tensor(block_tables, "block_tables", dev, (torch.int32,), shape=(B, None))
    _tensor(context_lens, "context_lens", dev, (torch.int32,), shape=(B,))
    if query_start_loc is not None:
        _tensor(query_start_loc, "query_start_loc", dev, (torch.int32,), shape=(B + 1,))
    _tensor(out, "out", dev, (q.dtype,), shape=tuple(q.shape))
    return dev


def _stream(stream):
    if stream is None:
        return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    if isinstance(stream, torch.cuda.Stream):
        return ctypes.c_void_p(stream.cuda_stream)
    return ctypes.c_void_p(int(stream))


class PagedAttnLib:
    """One loaded copy of the library (the product build or the no-bias build)."""

    def __init__(self, path: str = LIB_PATH):
        if not os.path.exists(path):
            raise RuntimeError(
                "%s is not built; run `python -c 'import __graft_entry__ as g; g.build()'`"
                % path)
        self.path = path
        lib = ctypes.CDLL(path)
        P, I32, I64, F32, SZ = (ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64,
                                ctypes.c_float, ctypes.c_size_t)
        lib.pa_abi_version.restype = ctypes.c_int
        lib.pa_abi_version.argtypes = []
        lib.pa_last_error.restype = ctypes.c_char_p
        lib.pa_last_error.argtypes = []
        lib.pa_decode_default_partition.restype = I32
        lib.pa_decode_default_partition.argtypes = [I32, I32, I32, I32, I32, ctypes.c_int]
        lib.pa_decode_workspace_bytes.restype = SZ
        lib.pa_decode_workspace_bytes.argtypes = [I32, I32, I32, I32, I32, I32, ctypes.c_int]
        lib.paged_attn_decode.restype = ctypes.c_int
        lib.paged_attn_decode.argtypes = [P, P, P, P, P, P, P, I32, F32, I32, I32, I32, I32,
                                          I32, I32, I32, I64, ctypes.c_int, I32, P, SZ, P]
        lib.paged_attn_prefill.restype = ctypes.c_int
        lib.paged_attn_prefill.argtypes = [P, P, P, P, P, P, P, P, I32, I32, F32, I32, I32,
                                           I32, I32, I32, I32, I32, I64, I64, ctypes.c_int, P]
        lib.paged_attn_decode_noalloc.restype = ctypes.c_int
        lib.paged_attn_decode_noalloc.argtypes = [P, P, P, P, P, P, P, I32, F32, I32, I32, I32,
                                                  I32, I32, I32, I32, I64, ctypes.c_int, I32, P]
        lib.paged_attn_decode_chunked.restype = ctypes.c_int
        lib.paged_attn_decode_chunked.argtypes = lib.paged_attn_decode.argtypes
        lib.paged_attn_prefill_chunked.restype = ctypes.c_int
        lib.paged_attn_prefill_chunked.argtypes = lib.paged_attn_prefill.argtypes
        lib.paged_attn_decode_relpos.restype = ctypes.c_int
        lib.paged_attn_decode_relpos.argtypes = [P, P, P, P, P, P, P, I32, I32, I32, I32, F32,
                                                 I32, I32, I32, I32, I32, I32, I32, I64,
                                                 ctypes.c_int, I32, P, SZ, P]
        lib.paged_attn_prefill_relpos.restype = ctypes.c_int
        lib.paged_attn_prefill_relpos.argtypes = [P, P, P, P, P, P, P, P, I32, I32, I32, I32,
                                                  I32, F32, I32, I32, I32, I32, I32, I32, I32,
                                                  I64, I64, ctypes.c_int, P]
        lib.paged_attn_decode_ragged_bias.restype = ctypes.c_int
        lib.paged_attn_decode_ragged_bias.argtypes = [P, P, P, P, P, P, P, P, I32, F32, I32,
                                                      I32, I32, I32, I32, I32, I32, I64,
                                                      ctypes.c_int, I32, P, SZ, P]
        lib.paged_attn_prefill_ragged_bias.restype = ctypes.c_int
        lib.paged_attn_prefill_ragged_bias.argtypes = [P, P, P, P, P, P, P, P, P, I32, I32, F32,
                                                       I32, I32, I32, I32, I32, I32, I32, I64,
                                                       I64, ctypes.c_int, P]
        lib.paged_kv_write.restype = ctypes.c_int
        lib.paged_kv_write.argtypes = [P, P, P, P, P, I64, I32, I32, I32, I32, I64,
                                       ctypes.c_int, P]
        lib.pa_window_first_live_block.restype = I32
        lib.pa_window_first_live_block.argtypes = [I32, I32]
        lib.pa_check_metadata.restype = ctypes.c_int
        lib.pa_check_metadata.argtypes = [P, P, P, I32, I32, I32, I32, I32, I64, I64]
        self._lib = lib

    # -- small queries ------------------------------------------------------
    def pa_abi_version(self) -> int:
        return int(self._lib.pa_abi_version())

    def pa_last_error(self) -> str:
        return self._lib.pa_last_error().decode()

    def _check(self, st: int) -> None:
        if st != 0:
            raise PagedAttnError(st, self.pa_last_error())

    def pa_decode_default_partition(self, num_seqs, num_heads, head_dim, max_seq_len,
                                    sliding_window, dtype=PA_DTYPE_BF16) -> int:
        return int(self._lib.pa_decode_default_partition(num_seqs, num_heads, head_dim,
                                                         max_seq_len, sliding_window, dtype))

    def pa_decode_workspace_bytes(self, num_seqs, num_heads, head_dim, max_seq_len,
                                  sliding_window, partition_tokens=0,
                                  dtype=PA_DTYPE_BF16) -> int:
        return int(self._lib.pa_decode_workspace_bytes(num_seqs, num_heads, head_dim,
                                                       max_seq_len, sliding_window,
                                                       partition_tokens, dtype))

    def pa_check_metadata(self, block_tables, context_lens, query_start_loc, sliding_window,
                          causal, max_seq_len, num_blocks, total_q=0) -> None:
        """Range-check host (CPU) int32 tensors; raises PagedAttnError.

        block_tables [B, max_blocks], context_lens [B], query_start_loc [B+1]
        or None: the shapes are checked here, since the C check reads exactly
        that many entries of each array."""
        for t in (block_tables, context_lens, query_start_loc):
            if t is not None and (not isinstance(t, torch.Tensor) or t.device.type != "cpu"
                                  or t.dtype != torch.int32 or not t.is_contiguous()):
                raise TypeError("pa_check_metadata takes contiguous CPU int32 tensors")
        if context_lens is None or context_lens.dim() != 1:
            raise ValueError("context_lens must be a 1-D tensor [num_seqs]")
        B = context_lens.shape[0]
        if block_tables is None or block_tables.dim() != 2 or block_tables.shape[0] != B:
            raise ValueError("block_tables must have shape (%d, max_blocks_per_seq), got %s"
                             % (B, None if block_tables is None else tuple(block_tables.shape)))
        if query_start_loc is not None and tuple(query_start_loc.shape) != (B + 1,):
            raise ValueError("query_start_loc must have shape (%d,), got %s"
                             % (B + 1, tuple(query_start_loc.shape)))
        self._check(self._lib.pa_check_metadata(
            _ptr(block_tables), _ptr(context_lens), _ptr(query_start_loc),
            int(sliding_window), int(causal), context_lens.shape[0], block_tables.shape[1],
            int(max_seq_len), int(num_blocks), int(total_q)))

    # -- entry points -------------------------------------------------------
    def workspace_for(self, q, max_seq_len, sliding_window, partition_tokens=0):
        """Allocate (torch) the decode workspace a call with these shapes needs."""
        B, H, D = q.shape
        n = self.pa_decode_workspace_bytes(B, H, D, max_seq_len, sliding_window,
                                           partition_tokens, _dtype_code(q))
        if n == 0:
            return None
        return torch.empty(n, dtype=torch.uint8, device=q.device)

    def paged_attn_decode(self, q, k_cache, v_cache, block_tables, context_lens, attn_bias,
                          sliding_window, scale, *, max_seq_len, out=None, workspace=None,
                          partition_tokens=0, stream=None):
        """Decode attention for q [B,H,D]; returns out [B,H,D] (q's dtype).

        k_cache, v_cache [num_blocks,H,16,D]; block_tables int32 [B,max_blocks];
        context_lens int32 [B]; attn_bias fp32 [B,H,max_seq_len] or None.
        Cross-attention: pass the encoder table and lengths, sliding_window -1."""
        return self._decode(self._lib.paged_attn_decode, q, k_cache, v_cache, block_tables,
                            context_lens, attn_bias, sliding_window, scale, max_seq_len, out,
                            workspace, partition_tokens, stream)

    def paged_attn_decode_noalloc(self, q, k_cache, v_cache, block_tables, context_lens,
                                  attn_bias, sliding_window, scale, *, max_seq_len, out,
                                  partition_tokens=0, stream=None):
        """paged_attn_decode without a workspace and without any device
        allocation: split-K partials go to the library's fixed per-GPU scratch
        (PA_NOALLOC_SCRATCH_BYTES; larger needs are rejected). `out` must be
        given. Calls that overlap on one GPU race."""
        _tensor(q, "q", None, _FLOAT_DTYPES, ndim=3)
        B, H, D = q.shape
        dev = _check_attention_args(q, k_cache, v_cache, block_tables, context_lens, out)
        if attn_bias is not None:
            _tensor(attn_bias, "attn_bias", dev, (torch.float32,), shape=(B, H, max_seq_len))
        self._check(self._lib.paged_attn_decode_noalloc(
            _ptr(out), _ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(block_tables),
            _ptr(context_lens), _ptr(attn_bias), int(sliding_window), float(scale), B, H,
            k_cache.shape[1], D, k_cache.shape[2], block_tables.shape[1], int(max_seq_len),
            k_cache.shape[0], _dtype_code(q), int(partition_tokens), _stream(stream)))
        return out

    def paged_attn_decode_chunked(self, q, k_cache, v_cache, block_tables, context_lens,
                                  attn_bias, chunk_size, scale, *, max_seq_len, out=None,
                                  workspace=None, partition_tokens=0, stream=None):
        """Decode with chunked local attention: the query (position L-1) sees
        the keys of its chunk of chunk_size positions. Otherwise as
        paged_attn_decode (no window)."""
        return self._decode(self._lib.paged_attn_decode_chunked, q, k_cache, v_cache,
                            block_tables, context_lens, attn_bias, chunk_size, scale,
                            max_seq_len, out, workspace, partition_tokens, stream)

    def _decode(self, fn, q, k_cache, v_cache, block_tables, context_lens, attn_bias, band,
                scale, max_seq_len, out, workspace, partition_tokens, stream):
        # band: the sliding window, or the chunk size of the chunked entry point
        # (which bounds the workspace like a window of that size)
        _tensor(q, "q", None, _FLOAT_DTYPES, ndim=3)
        B, H, D = q.shape
        if out is None:
            out = torch.empty_like(q)
        dev = _check_attention_args(q, k_cache, v_cache, block_tables, context_lens, out)
        if attn_bias is not None:
            _tensor(attn_bias, "attn_bias", dev, (torch.float32,), shape=(B, H, max_seq_len))
        if workspace is None:
            workspace = self.workspace_for(q, max_seq_len, band, partition_tokens)
        else:
            _tensor(workspace, "workspace", dev, ndim=1)
        ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
        self._check(fn(
            _ptr(out), _ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(block_tables),
            _ptr(context_lens), _ptr(attn_bias), int(band), float(scale), B, H,
            k_cache.shape[1], D, k_cache.shape[2], block_tables.shape[1], int(max_seq_len),
            k_cache.shape[0], _dtype_code(q), int(partition_tokens), _ptr(workspace), ws_bytes,
            _stream(stream)))
        return out

    def paged_attn_prefill(self, q, k_cache, v_cache, block_tables, context_lens,
                           query_start_loc, attn_bias, sliding_window, causal, scale, *,
                           max_seq_len, out=None, stream=None):
        """Prefill attention for packed q [total_q,H,D]; returns out like q.

        query_start_loc int32 [B+1]; attn_bias fp32 [B,H,max_seq_len,max_seq_len]
        or None; causal False for encoder-only bidirectional attention."""
        return self._prefill(self._lib.paged_attn_prefill, q, k_cache, v_cache, block_tables,
                             context_lens, query_start_loc, attn_bias, sliding_window, causal,
                             scale, max_seq_len, out, stream)

    def paged_attn_prefill_chunked(self, q, k_cache, v_cache, block_tables, context_lens,
                                   query_start_loc, attn_bias, chunk_size, causal, scale, *,
                                   max_seq_len, out=None, stream=None):
        """Prefill with chunked local attention: a query at position p sees the
        keys of its chunk (floor(j / chunk_size) == floor(p / chunk_size)), and
        with causal only those up to p. Otherwise as paged_attn_prefill."""
        return self._prefill(self._lib.paged_attn_prefill_chunked, q, k_cache, v_cache,
                             block_tables, context_lens, query_start_loc, attn_bias,
                             chunk_size, causal, scale, max_seq_len, out, stream)

    def _prefill(self, fn, q, k_cache, v_cache, block_tables, context_lens, query_start_loc,
                 attn_bias, band, causal, scale, max_seq_len, out, stream):
        _tensor(q, "q", None, _FLOAT_DTYPES, ndim=3)
        TQ, H, D = q.shape
        if out is None:
            out = torch.empty_like(q)
        B = context_lens.shape[0] if isinstance(context_lens, torch.Tensor) else 0
        dev = _check_attention_args(q, k_cache, v_cache, block_tables, context_lens, out,
                                    query_start_loc, B)
        if attn_bias is not None:
            _tensor(attn_bias, "attn_bias", dev, (torch.float32,),
                    shape=(B, H, max_seq_len, max_seq_len))
        self._check(fn(
            _ptr(out), _ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(block_tables),
            _ptr(context_lens), _ptr(query_start_loc), _ptr(attn_bias), int(band),
            int(bool(causal)), float(scale), context_lens.shape[0], H, k_cache.shape[1], D,
            k_cache.shape[2], block_tables.shape[1], int(max_seq_len), k_cache.shape[0], TQ,
            _dtype_code(q), _stream(stream)))
        return out

    def paged_attn_decode_relpos(self, q, k_cache, v_cache, block_tables, context_lens,
                                 rel_table, num_buckets, max_distance, bidirectional,
                                 sliding_window, scale, *, max_seq_len, out=None,
                                 workspace=None, partition_tokens=0, stream=None):
        """Decode with the T5 relative-position bias computed in the kernel from
        rel_table [H, num_buckets] (fp32); see include/paged_attn.h."""
        _tensor(q, "q", None, _FLOAT_DTYPES, ndim=3)
        B, H, D = q.shape
        if out is None:
            out = torch.empty_like(q)
        dev = _check_attention_args(q, k_cache, v_cache, block_tables, context_lens, out)
        _tensor(rel_table, "rel_table", dev, (torch.float32,), shape=(H, num_buckets))
        if workspace is None:
            workspace = self.workspace_for(q, max_seq_len, sliding_window, partition_tokens)
        else:
            _tensor(workspace, "workspace", dev, ndim=1)
        ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
        self._check(self._lib.paged_attn_decode_relpos(
            _ptr(out), _ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(block_tables),
            _ptr(context_lens), _ptr(rel_table), int(num_buckets), int(max_distance),
            int(bidirectional), int(sliding_window), float(scale), B, H, k_cache.shape[1], D,
            k_cache.shape[2], block_tables.shape[1], int(max_seq_len), k_cache.shape[0],
            _dtype_code(q), int(partition_tokens), _ptr(workspace), ws_bytes, _stream(stream)))
        return out

    def paged_attn_prefill_relpos(self, q, k_cache, v_cache, block_tables, context_lens,
                                  query_start_loc, rel_table, num_buckets, max_distance,
                                  bidirectional, sliding_window, causal, scale, *, max_seq_len,
                                  out=None, stream=None):
        """Prefill with the T5 relative-position bias computed in the kernel."""
        _tensor(q, "q", None, _FLOAT_DTYPES, ndim=3)
        TQ, H, D = q.shape
        if out is None:
            out = torch.empty_like(q)
        B = context_lens.shape[0] if isinstance(context_lens, torch.Tensor) else 0
        dev = _check_attention_args(q, k_cache, v_cache, block_tables, context_lens, out,
                                    query_start_loc, B)
        _tensor(rel_table, "rel_table", dev, (torch.float32,), shape=(H, num_buckets))
        self._check(self._lib.paged_attn_prefill_relpos(
            _ptr(out), _ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(block_tables),
            _ptr(context_lens), _ptr(query_start_loc), _ptr(rel_table), int(num_buckets),
            int(max_distance), int(bidirectional), int(sliding_window), int(bool(causal)),
            float(scale), context_lens.shape[0], H, k_cache.shape[1], D, k_cache.shape[2],
            block_tables.shape[1], int(max_seq_len), k_cache.shape[0], TQ, _dtype_code(q),
            _stream(stream)))
        return out

    def paged_attn_decode_ragged_bias(self, q, k_cache, v_cache, block_tables, context_lens,
                                      attn_bias, bias_start, sliding_window, scale, *,
                                      max_seq_len, out=None, workspace=None,
                                      partition_tokens=0, stream=None):
        """Decode with a packed bias: sequence b's rows [H][L_b] start at
        attn_bias[bias_start[b]] (bias_start int64 [B])."""
        _tensor(q, "q", None, _FLOAT_DTYPES, ndim=3)
        B, H, D = q.shape
        if out is None:
            out = torch.empty_like(q)
        dev = _check_attention_args(q, k_cache, v_cache, block_tables, context_lens, out)
        _tensor(attn_bias, "attn_bias", dev, (torch.float32,), ndim=1)
        _tensor(bias_start, "bias_start", dev, (torch.int64,), shape=(B,))
        if workspace is None:
            workspace = self.workspace_for(q, max_seq_len, sliding_window, partition_tokens)
        else:
            _tensor(workspace, "workspace", dev, ndim=1)
        ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
        self._check(self._lib.paged_attn_decode_ragged_bias(
            _ptr(out), _ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(block_tables),
            _ptr(context_lens), _ptr(attn_bias), _ptr(bias_start), int(sliding_window),
            float(scale), B, H, k_cache.shape[1], D, k_cache.shape[2], block_tables.shape[1],
            int(max_seq_len), k_cache.shape[0], _dtype_code(q), int(partition_tokens),
            _ptr(workspace), ws_bytes, _stream(stream)))
        return out

    def paged_attn_prefill_ragged_bias(self, q, k_cache, v_cache, block_tables, context_lens,
                                       query_start_loc, attn_bias, bias_start, sliding_window,
                                       causal, scale, *, max_seq_len, out=None, stream=None):
        """Prefill with a packed bias: sequence b's rows [H][n_q][L_b] start at
        attn_bias[bias_start[b]]."""
        _tensor(q, "q", None, _FLOAT_DTYPES, ndim=3)
        TQ, H, D = q.shape
        if out is None:
            out = torch.empty_like(q)
        B = context_lens.shape[0] if isinstance(context_lens, torch.Tensor) else 0
        dev = _check_attention_args(q, k_cache, v_cache, block_tables, context_lens, out,
                                    query_start_loc, B)
        _tensor(attn_bias, "attn_bias", dev, (torch.float32,), ndim=1)
        _tensor(bias_start, "bias_start", dev, (torch.int64,), shape=(B,))
        self._check(self._lib.paged_attn_prefill_ragged_bias(
            _ptr(out), _ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(block_tables),
            _ptr(context_lens), _ptr(query_start_loc), _ptr(attn_bias), _ptr(bias_start),
            int(sliding_window), int(bool(causal)), float(scale), context_lens.shape[0], H,
            k_cache.shape[1], D, k_cache.shape[2], block_tables.shape[1], int(max_seq_len),
            k_cache.shape[0], TQ, _dtype_code(q), _stream(stream)))
        return out

    def paged_kv_write(self, k_cache, v_cache, k_new, v_new, slot_mapping, *, stream=None):
        """Scatter k_new, v_new [T,H,D] into the paged caches at slot_mapping
        (int64 [T], block * 16 + offset; negative = skip)."""
        _tensor(k_cache, "k_cache", None, _FLOAT_DTYPES, ndim=4)
        dev = k_cache.device
        _tensor(v_cache, "v_cache", dev, (k_cache.dtype,), shape=tuple(k_cache.shape))
        _tensor(k_new, "k_new", dev, (k_cache.dtype,), shape=(None, None, k_cache.shape[3]))
        T, H, D = k_new.shape
        _tensor(v_new, "v_new", dev, (k_cache.dtype,), shape=(T, H, D))
        _tensor(slot_mapping, "slot_mapping", dev, (torch.int64,), shape=(T,))
        self._check(self._lib.paged_kv_write(
            _ptr(k_cache), _ptr(v_cache), _ptr(k_new), _ptr(v_new), _ptr(slot_mapping), T, H,
            k_cache.shape[1], D, k_cache.shape[2], k_cache.shape[0], _dtype_code(k_cache),
            _stream(stream)))

    def pa_window_first_live_block(self, context_len, sliding_window) -> int:
        return int(self._lib.pa_window_first_live_block(int(context_len), int(sliding_window)))


_default = None


def lib() -> PagedAttnLib:
    """The product library (loaded once)."""
    global _default
    if _default is None:
        _default = PagedAttnLib(LIB_PATH)
    return _default


def paged_attn_decode(*args, **kwargs):
    return lib().paged_attn_decode(*args, **kwargs)


def paged_attn_prefill(*args, **kwargs):
    return lib().paged_attn_prefill(*args, **kwargs)


def paged_attn_decode_noalloc(*args, **kwargs):
    return lib().paged_attn_decode_noalloc(*args, **kwargs)


def paged_attn_decode_chunked(*args, **kwargs):
    return lib().paged_attn_decode_chunked(*args, **kwargs)


def paged_attn_prefill_chunked(*args, **kwargs):
    return lib().paged_attn_prefill_chunked(*args, **kwargs)


def paged_attn_decode_relpos(*args, **kwargs):
    return lib().paged_attn_decode_relpos(*args, **kwargs)


def paged_attn_prefill_relpos(*args, **kwargs):
    return lib().paged_attn_prefill_relpos(*args, **kwargs)


def paged_attn_decode_ragged_bias(*args, **kwargs):
    return lib().paged_attn_decode_ragged_bias(*args, **kwargs)


def paged_attn_prefill_ragged_bias(*args, **kwargs):
    return lib().paged_attn_prefill_ragged_bias(*args, **kwargs)


def paged_kv_write(*args, **kwargs):
    return lib().paged_kv_write(*args, **kwargs)


def pa_window_first_live_block(*args, **kwargs):
    return lib().pa_window_first_live_block(*args, **kwargs)


def pa_decode_workspace_bytes(*args, **kwargs):
    return lib().pa_decode_workspace_bytes(*args, **kwargs)


def pa_decode_default_partition(*args, **kwargs):
    return lib().pa_decode_default_partition(*args, **kwargs)


def pa_check_metadata(*args, **kwargs):
    return lib().pa_check_metadata(*args, **kwargs)


def pa_abi_version():
    return lib().pa_abi_version()
