"""C-ABI checks that need no GPU: the library loads, exports every function
include/paged_attn.h declares, and rejects bad arguments on the host before
any HIP call (every call below returns an error status before launching)."""
import ctypes
import os
import re

import pytest
import torch

import sliding_window_mask_amd as pa

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "paged_attn.h")


def declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    names = re.findall(r"^\s*(?:const\s+)?[A-Za-z_][\w]*\s*\**\s*([A-Za-z_]\w*)\s*\(", src,
                       flags=re.M)
    return sorted(set(n for n in names if n not in ("defined",)))


def test_header_declares_entry_points():
    names = declared_functions()
    for n in ("paged_attn_decode", "paged_attn_prefill", "pa_decode_workspace_bytes",
              "pa_last_error", "pa_abi_version", "pa_check_metadata",
              "pa_decode_default_partition", "paged_attn_decode_chunked",
              "paged_attn_prefill_chunked"):
        assert n in names


@pytest.mark.parametrize("path", [pa.LIB_PATH, pa.LIB_NOBIAS_PATH])
def test_library_exports_every_declared_symbol(path):
    lib = ctypes.CDLL(path)
    for name in declared_functions():
        assert hasattr(lib, name), name


def test_abi_version():
    assert pa.pa_abi_version() == 1


# a valid-looking argument list with fake (never dereferenced) device pointers
FAKE = 1 << 20        # 16-byte aligned non-null address


def decode_args(**kw):
    a = dict(out=FAKE, q=FAKE, k=FAKE, v=FAKE, bt=FAKE, cl=FAKE, bias=None, window=-1,
             scale=0.125, B=4, H=4, Hkv=4, D=64, bs=16, maxb=8, msl=128, nb=64, dtype=0,
             part=0, ws=None, wsb=0, stream=None)
    a.update(kw)
    return a


def call_decode(lib, a):
    return lib._lib.paged_attn_decode(a["out"], a["q"], a["k"], a["v"], a["bt"], a["cl"],
                                      a["bias"], a["window"], a["scale"], a["B"], a["H"],
                                      a["Hkv"], a["D"], a["bs"], a["maxb"], a["msl"], a["nb"],
                                      a["dtype"], a["part"], a["ws"], a["wsb"], a["stream"])


@pytest.mark.parametrize("kw,status", [
    (dict(out=None), 1), (dict(q=None), 1), (dict(k=None), 1), (dict(v=None), 1),
    (dict(bt=None), 1), (dict(cl=None), 1),
    (dict(window=0), 2), (dict(window=-2), 2),
    (dict(D=96), 3), (dict(D=32), 3), (dict(bs=32), 3), (dict(Hkv=2), 3), (dict(dtype=2), 3),
    (dict(maxb=7), 2), (dict(B=-1), 2), (dict(H=0), 2), (dict(scale=float("inf")), 2),
    (dict(scale=float("nan")), 2), (dict(B=65536), 2), (dict(H=65536, Hkv=65536), 2),
    (dict(q=FAKE + 4), 4), (dict(out=FAKE + 8), 4), (dict(bias=FAKE + 2), 4),
    (dict(part=24), 2), (dict(part=-16), 2), (dict(part=8192), 2),
])
def test_decode_rejects_on_host(kw, status):
    lib = pa.lib()
    st = call_decode(lib, decode_args(**kw))
    assert st == status, (st, lib.pa_last_error())
    assert lib.pa_last_error()


@pytest.mark.parametrize("chunk", [0, -1, -16])
def test_chunked_entry_points_reject_non_positive_chunks(chunk):
    lib = pa.lib()
    a = decode_args(window=chunk)          # the chunk size takes the window's place
    st = lib._lib.paged_attn_decode_chunked(
        a["out"], a["q"], a["k"], a["v"], a["bt"], a["cl"], a["bias"], a["window"], a["scale"],
        a["B"], a["H"], a["Hkv"], a["D"], a["bs"], a["maxb"], a["msl"], a["nb"], a["dtype"],
        a["part"], a["ws"], a["wsb"], a["stream"])
    assert st == 2 and "chunk_size" in lib.pa_last_error()
    st = lib._lib.paged_attn_prefill_chunked(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None,
                                             chunk, 0, 0.125, 2, 4, 4, 64, 16, 8, 128, 64, 10,
                                             0, None)
    assert st == 2 and "chunk_size" in lib.pa_last_error()


def test_chunked_entry_points_check_like_the_base_ones():
    lib = pa.lib()
    a = decode_args(window=32, q=None)
    st = lib._lib.paged_attn_decode_chunked(
        a["out"], a["q"], a["k"], a["v"], a["bt"], a["cl"], a["bias"], a["window"], a["scale"],
        a["B"], a["H"], a["Hkv"], a["D"], a["bs"], a["maxb"], a["msl"], a["nb"], a["dtype"],
        a["part"], a["ws"], a["wsb"], a["stream"])
    assert st == 1                                       # NULL q
    st = lib._lib.paged_attn_prefill_chunked(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None,
                                             32, 2, 0.125, 2, 4, 4, 64, 16, 8, 128, 64, 10,
                                             0, None)
    assert st == 2                                       # causal must be 0 or 1
    # an empty batch launches nothing and needs no pointers
    assert lib._lib.paged_attn_decode_chunked(None, None, None, None, None, None, None, 32,
                                              0.125, 0, 4, 4, 64, 16, 8, 128, 64, 0, 0, None,
                                              0, None) == 0


def test_decode_workspace_required():
    lib = pa.lib()
    # a long max_seq_len with a short partition needs a workspace
    n = lib.pa_decode_workspace_bytes(4, 4, 64, 4096, -1, 256, 0)
    assert n > 0
    st = call_decode(lib, decode_args(msl=4096, maxb=256, part=256))
    assert st == 5, lib.pa_last_error()
    st = call_decode(lib, decode_args(msl=4096, maxb=256, part=256, ws=FAKE, wsb=n - 1))
    assert st == 5
    st = call_decode(lib, decode_args(msl=4096, maxb=256, part=256, ws=FAKE + 16, wsb=n))
    assert st == 4     # workspace must be 256-byte aligned


def test_workspace_sizes():
    lib = pa.lib()
    # one partition covers everything: no workspace
    assert lib.pa_decode_workspace_bytes(4, 4, 64, 128, -1, 0, 0) == 0
    assert lib.pa_decode_workspace_bytes(256, 16, 64, 512, -1, 0, 1) == 0
    # a window bounds the partitions a sequence can need
    full = lib.pa_decode_workspace_bytes(256, 32, 128, 4096, -1, 512, 1)
    win = lib.pa_decode_workspace_bytes(256, 32, 128, 4096, 1024, 512, 1)
    assert 0 < win < full
    rows = 256 * 32 * 8
    assert full >= rows * (128 + 2) * 4
    assert lib.pa_decode_workspace_bytes(4, 4, 64, 128, -1, 24, 0) == 0   # invalid partition


def test_default_partition_is_block_multiple():
    lib = pa.lib()
    for shape in [(4, 4, 64, 128, -1), (64, 8, 64, 512, -1), (256, 16, 64, 512, -1),
                  (256, 32, 128, 4096, -1), (256, 32, 128, 4096, 1024), (1, 1, 64, 1, -1)]:
        p = lib.pa_decode_default_partition(*shape)
        assert p % 16 == 0 and 16 <= p <= 4096, (shape, p)


def test_empty_batch_is_ok_without_launch():
    lib = pa.lib()
    assert call_decode(lib, decode_args(B=0, out=None, q=None)) == 0


def prefill_call(lib, **kw):
    a = dict(out=FAKE, q=FAKE, k=FAKE, v=FAKE, bt=FAKE, cl=FAKE, qsl=FAKE, bias=None,
             window=-1, causal=0, scale=0.125, B=2, H=4, Hkv=4, D=64, bs=16, maxb=8, msl=128,
             nb=64, tq=10, dtype=0, stream=None)
    a.update(kw)
    return lib._lib.paged_attn_prefill(a["out"], a["q"], a["k"], a["v"], a["bt"], a["cl"],
                                       a["qsl"], a["bias"], a["window"], a["causal"],
                                       a["scale"], a["B"], a["H"], a["Hkv"], a["D"], a["bs"],
                                       a["maxb"], a["msl"], a["nb"], a["tq"], a["dtype"],
                                       a["stream"])


@pytest.mark.parametrize("kw,status", [
    (dict(qsl=None), 1), (dict(causal=2), 2), (dict(tq=-1), 2), (dict(window=0), 2),
    (dict(D=80), 3), (dict(dtype=2), 3), (dict(qsl=FAKE + 2), 4), (dict(k=None), 1),
    (dict(B=65536), 2), (dict(H=65536, Hkv=65536), 2), (dict(maxb=7), 2),
    (dict(scale=float("nan")), 2),
])
def test_prefill_rejects_on_host(kw, status):
    lib = pa.lib()
    st = prefill_call(lib, **kw)
    assert st == status, (st, lib.pa_last_error())


def test_prefill_without_queries_needs_no_pointers():
    # an empty packed query tensor may have a NULL data pointer; nothing is
    # computed, but the scalar arguments are still checked
    lib = pa.lib()
    none = dict(out=None, q=None, k=None, v=None, bt=None, cl=None, qsl=None)
    assert prefill_call(lib, tq=0, **none) == 0, lib.pa_last_error()
    assert prefill_call(lib, tq=0, D=80, **none) == 3
    assert prefill_call(lib, tq=0, causal=2, **none) == 2
    assert prefill_call(lib, tq=0, window=0, **none) == 2
    assert prefill_call(lib, tq=1, **dict(none, k=FAKE, v=FAKE, bt=FAKE, cl=FAKE)) == 1
    st = lib._lib.paged_attn_prefill_ragged_bias(None, None, None, None, None, None, None, None,
                                                 None, -1, 0, 0.125, 2, 4, 4, 64, 16, 8, 128,
                                                 64, 0, 0, None)
    assert st == 0, lib.pa_last_error()


def test_check_metadata_host():
    lib = pa.lib()
    bt = torch.tensor([[3, 1, 0], [2, 3, 9]], dtype=torch.int32)
    cl = torch.tensor([40, 17], dtype=torch.int32)
    lib.pa_check_metadata(bt, cl, None, -1, 0, 48, 4)   # entry 9 backs no token
    with pytest.raises(pa.PagedAttnError):        # 9 is outside a 4-block pool
        lib.pa_check_metadata(bt, torch.tensor([40, 33], dtype=torch.int32), None, -1, 0, 48, 4)
    with pytest.raises(pa.PagedAttnError):        # length beyond max_seq_len
        lib.pa_check_metadata(bt, torch.tensor([49, 1], dtype=torch.int32), None, -1, 0, 48, 4)
    # with a window, entries before it are never read, so they may be anything
    bt2 = torch.tensor([[-5, 1, 0], [2, 3, 9]], dtype=torch.int32)
    lib.pa_check_metadata(bt2, torch.tensor([40, 20], dtype=torch.int32), None, 16, 0, 48, 4)
    with pytest.raises(pa.PagedAttnError):
        lib.pa_check_metadata(bt2, torch.tensor([40, 20], dtype=torch.int32), None, 30, 0, 48, 4)
    # prefill: query counts and start offsets
    qsl = torch.tensor([0, 40, 57], dtype=torch.int32)
    lib.pa_check_metadata(bt, cl, qsl, -1, 0, 48, 4, total_q=57)
    with pytest.raises(pa.PagedAttnError):
        lib.pa_check_metadata(bt, cl, qsl, -1, 0, 48, 4, total_q=58)
    with pytest.raises(pa.PagedAttnError):        # more queries than keys
        lib.pa_check_metadata(bt, cl, torch.tensor([0, 41, 58], dtype=torch.int32), -1, 0,
                              48, 4, total_q=58)


def test_check_metadata_rejects_mismatched_shapes():
    """The C check reads num_seqs rows of the table and num_seqs + 1 query
    offsets: the binding refuses arrays of other shapes before the call, and
    the C check refuses a table too narrow for max_seq_len."""
    lib = pa.lib()
    bt = torch.tensor([[3, 1, 0], [2, 3, 9]], dtype=torch.int32)
    cl = torch.tensor([40, 17], dtype=torch.int32)
    with pytest.raises(ValueError):               # table has fewer rows than sequences
        lib.pa_check_metadata(bt[:1].contiguous(), cl, None, -1, 0, 48, 4)
    with pytest.raises(ValueError):               # 1-D table
        lib.pa_check_metadata(bt.reshape(-1), cl, None, -1, 0, 48, 4)
    with pytest.raises(ValueError):               # B offsets instead of B + 1
        lib.pa_check_metadata(bt, cl, torch.tensor([0, 40], dtype=torch.int32), -1, 0, 48, 4,
                              total_q=40)
    with pytest.raises(ValueError):
        lib.pa_check_metadata(bt, cl.reshape(2, 1), None, -1, 0, 48, 4)
    with pytest.raises(TypeError):
        lib.pa_check_metadata(bt, cl.to(torch.int64), None, -1, 0, 48, 4)
    with pytest.raises(pa.PagedAttnError):        # 3 blocks cover 48 tokens, not 64
        lib.pa_check_metadata(bt, torch.tensor([40, 17], dtype=torch.int32), None, -1, 0, 64,
                              16)


def test_binding_fails_loudly_without_library(tmp_path):
    with pytest.raises(RuntimeError):
        pa.PagedAttnLib(str(tmp_path / "missing.so"))


def relpos_decode_call(lib, **kw):
    a = dict(out=FAKE, q=FAKE, k=FAKE, v=FAKE, bt=FAKE, cl=FAKE, tab=FAKE, nb=32, md=128,
             bidir=0, window=-1, scale=0.125, B=4, H=4, Hkv=4, D=64, bs=16, maxb=8, msl=128,
             nblk=64, dtype=0, part=0, ws=None, wsb=0, stream=None)
    a.update(kw)
    return lib._lib.paged_attn_decode_relpos(
        a["out"], a["q"], a["k"], a["v"], a["bt"], a["cl"], a["tab"], a["nb"], a["md"],
        a["bidir"], a["window"], a["scale"], a["B"], a["H"], a["Hkv"], a["D"], a["bs"],
        a["maxb"], a["msl"], a["nblk"], a["dtype"], a["part"], a["ws"], a["wsb"], a["stream"])


@pytest.mark.parametrize("kw,status", [
    (dict(tab=None), 1), (dict(tab=FAKE + 2), 4), (dict(bidir=2), 2), (dict(nb=1), 2),
    (dict(nb=31, bidir=1), 2), (dict(nb=66), 2), (dict(md=16), 2), (dict(md=1025), 2),
    (dict(nb=2, bidir=1), 2), (dict(D=96), 3), (dict(window=0), 2),
])
def test_decode_relpos_rejects_on_host(kw, status):
    lib = pa.lib()
    st = relpos_decode_call(lib, **kw)
    assert st == status, (st, lib.pa_last_error())


def test_prefill_relpos_rejects_on_host():
    lib = pa.lib()
    st = lib._lib.paged_attn_prefill_relpos(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None, 32,
                                            128, 1, -1, 0, 0.125, 2, 4, 4, 64, 16, 8, 128, 64,
                                            10, 0, None)
    assert st == 1
    st = lib._lib.paged_attn_prefill_relpos(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 32,
                                            4, 1, -1, 0, 0.125, 2, 4, 4, 64, 16, 8, 128, 64, 10,
                                            0, None)
    assert st == 2     # max_distance must exceed the exact range (8 for 16 buckets a side)


@pytest.mark.parametrize("kw,status", [
    (dict(k=None), 1), (dict(slots=None), 1), (dict(slots=FAKE + 4), 4), (dict(kn=FAKE + 8), 4),
    (dict(D=96), 3), (dict(Hkv=1), 3), (dict(bs=8), 3), (dict(T=-1), 2), (dict(dtype=2), 3),
])
def test_kv_write_rejects_on_host(kw, status):
    lib = pa.lib()
    a = dict(k=FAKE, v=FAKE, kn=FAKE, vn=FAKE, slots=FAKE, T=4, H=2, Hkv=2, D=64, bs=16, nb=8,
             dtype=1, stream=None)
    a.update(kw)
    st = lib._lib.paged_kv_write(a["k"], a["v"], a["kn"], a["vn"], a["slots"], a["T"], a["H"],
                                 a["Hkv"], a["D"], a["bs"], a["nb"], a["dtype"], a["stream"])
    assert st == status, (st, lib.pa_last_error())


def test_kv_write_empty_is_ok():
    lib = pa.lib()
    assert lib._lib.paged_kv_write(None, None, None, None, None, 0, 2, 2, 64, 16, 8, 1,
                                   None) == 0


def test_window_first_live_block():
    lib = pa.lib()
    f = lib.pa_window_first_live_block
    assert f(100, -1) == 0 and f(0, 24) == 0 and f(24, 24) == 0
    assert f(25, 24) == 0                      # first visible token 1 -> block 0
    assert f(40, 24) == 1                      # first visible token 16 -> block 1
    assert f(1000, 64) == (1000 - 64) // 16
    # monotone in the context length: once a block is dead it stays dead
    prev = 0
    for L in range(0, 500):
        cur = f(L, 37)
        assert cur >= prev
        prev = cur


def test_ragged_bias_requires_pointers():
    lib = pa.lib()
    st = lib._lib.paged_attn_decode_ragged_bias(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None,
                                                -1, 0.125, 4, 4, 4, 64, 16, 8, 128, 64, 0, 0,
                                                None, 0, None)
    assert st == 1
    st = lib._lib.paged_attn_decode_ragged_bias(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE,
                                                FAKE + 4, -1, 0.125, 4, 4, 4, 64, 16, 8, 128,
                                                64, 0, 0, None, 0, None)
    assert st == 4
    st = lib._lib.paged_attn_prefill_ragged_bias(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None,
                                                 FAKE, -1, 0, 0.125, 2, 4, 4, 64, 16, 8, 128,
                                                 64, 10, 0, None)
    assert st == 1


def test_no_bias_build_rejects_a_bias():
    nob = pa.PagedAttnLib(pa.LIB_NOBIAS_PATH)
    st = call_decode(nob, decode_args(bias=FAKE))
    assert st == 3, nob.pa_last_error()


def test_binding_rejects_host_tensors_before_any_call():
    # CPU tensors would reach the kernels as host pointers: the binding
    # refuses them (and non-tensors) before the library is called
    lib = pa.lib()
    q = torch.zeros(2, 4, 64)
    cache = torch.zeros(8, 4, 16, 64)
    bt = torch.zeros(2, 4, dtype=torch.int32)
    cl = torch.ones(2, dtype=torch.int32)
    with pytest.raises(ValueError, match="q must be a tensor on"):
        lib.paged_attn_decode(q, cache, cache, bt, cl, None, -1, 0.125, max_seq_len=64)
    with pytest.raises(ValueError, match="q must be a tensor on"):
        lib.paged_attn_prefill(q, cache, cache, bt, cl, torch.tensor([0, 1, 2], dtype=torch.int32),
                               None, -1, False, 0.125, max_seq_len=64)
    with pytest.raises(TypeError, match="q must be a torch.Tensor"):
        lib.paged_attn_decode([0.0], cache, cache, bt, cl, None, -1, 0.125, max_seq_len=64)
    with pytest.raises(ValueError, match="k_cache must be a tensor on"):
        lib.paged_kv_write(cache, cache, q, q, torch.zeros(2, dtype=torch.int64))
