"""Seeded randomised parity sweep: each case draws a shape (batch, heads,
head_dim, lengths, pool size), a dtype, a window, a mask (causal or not), a
bias kind and a decode partition from its seed, runs the HIP entry point and
compares with the float64 oracle. Also a cross-kernel identity: a causal
prefill with one query per sequence (the last position) is the same
computation as decode, so the two kernels must agree to the dtype tolerance."""
import numpy as np
import pytest
import torch

import oracle
import workloads
from gpu_helpers import (BS, TOL, assert_close, gpu_decode, gpu_prefill, log, oracle_decode,
                         oracle_prefill, to_device, to_host)

import sliding_window_mask_amd as pa

pytestmark = pytest.mark.gpu
DTYPES = [torch.float32, torch.bfloat16]


def draw(seed):
    r = np.random.default_rng(seed)
    return dict(B=int(r.integers(1, 7)), H=int(r.integers(1, 5)), D=int(r.choice([64, 128])),
                maxlen=int(r.choice([17, 64, 100, 300, 700])),
                dtype=DTYPES[int(r.integers(0, 2))],
                window=int(r.choice([-1, -1, 1, 5, 16, 63, 200])),
                causal=bool(r.integers(0, 2)),
                bias=[None, "normal", "zero"][int(r.integers(0, 3))],
                partition=int(r.choice([0, 0, 16, 64, 256])),
                rng=r)


@pytest.mark.parametrize("seed", range(24))
def test_random_decode(seed):
    d = draw(1000 + seed)
    msl = -(-d["maxlen"] // BS) * BS
    lens = d["rng"].integers(0, d["maxlen"] + 1, size=d["B"]).tolist()
    log("random decode %d: %s" % (seed, {k: v for k, v in d.items() if k != "rng"}))
    case = to_device(workloads.decode_case(2000 + seed, num_seqs=d["B"], num_heads=d["H"],
                                           head_dim=d["D"], lens=lens, max_seq_len=msl,
                                           dtype=d["dtype"], bias=d["bias"],
                                           sliding_window=d["window"]))
    assert_close(gpu_decode(case, partition=d["partition"]), oracle_decode(case), d["dtype"],
                 "random decode %d" % seed)


@pytest.mark.parametrize("seed", range(24))
def test_random_prefill(seed):
    d = draw(3000 + seed)
    msl = -(-d["maxlen"] // BS) * BS
    lens = d["rng"].integers(0, d["maxlen"] + 1, size=d["B"])
    q_lens = [int(d["rng"].integers(0, L + 1)) if d["rng"].integers(0, 2) else int(L)
              for L in lens]
    log("random prefill %d: %s q_lens %s" % (seed, {k: v for k, v in d.items() if k != "rng"},
                                             q_lens))
    case = to_device(workloads.prefill_case(4000 + seed, num_seqs=d["B"], num_heads=d["H"],
                                            head_dim=d["D"], lens=lens.tolist(),
                                            max_seq_len=msl, dtype=d["dtype"],
                                            bias=None if d["bias"] == "zero" else d["bias"],
                                            sliding_window=d["window"], causal=d["causal"],
                                            q_lens=q_lens))
    assert_close(gpu_prefill(case), oracle_prefill(case), d["dtype"],
                 "random prefill %d" % seed)


@pytest.mark.parametrize("dtype", DTYPES)
@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("window", [-1, 24])
def test_prefill_last_query_equals_decode(dtype, D, window):
    # decode's query sits at position L-1 and sees keys j <= L-1 (and, with a
    # window, L-1-j < W): exactly a causal prefill row with n_q = 1
    lens = [1, 16, 17, 95, 300]
    msl = 304
    dc = to_device(workloads.decode_case(5000 + D, num_seqs=len(lens), num_heads=3, head_dim=D,
                                         lens=lens, max_seq_len=msl, dtype=dtype, bias=None,
                                         sliding_window=window))
    qsl = torch.arange(len(lens) + 1, dtype=torch.int32, device="cuda")
    pre = pa.paged_attn_prefill(dc.q, dc.k_cache, dc.v_cache, dc.block_tables,
                                dc.context_lens, qsl, None, window, True, dc.scale,
                                max_seq_len=msl)
    dec = gpu_decode(dc, bias=None)
    torch.cuda.synchronize()
    err = float((pre.double() - dec.double()).abs().max())
    log("prefill(n_q=1) vs decode D=%d W=%d dtype=%s: %.3e" % (D, window, dtype, err))
    assert err <= TOL[dtype]
    assert_close(dec, oracle_decode(dc, bias=None), dtype, "decode")


def pack(dense, lens, q_lens=None):
    """Packed (ragged) copy of a padded bias: decode rows [H][L_b], prefill
    rows [H][n_q][L_b] (the last n_q positions), back to back, with offsets."""
    parts, starts, off = [], [], 0
    for b, L in enumerate(lens):
        L = int(L)
        if q_lens is None:
            part = dense[b, :, :L]
        else:
            nq = int(q_lens[b])
            part = dense[b, :, L - nq:L, :L]
        parts.append(part.reshape(-1))
        starts.append(off)
        off += part.numel()
    packed = torch.cat(parts) if parts else torch.zeros(0)
    return packed.contiguous(), torch.tensor(starts, dtype=torch.int64)


@pytest.mark.parametrize("seed", range(16))
def test_random_relpos(seed):
    # in-kernel T5 bias over random bucket tables, both kernels' dtypes and head dims
    d = draw(6000 + seed)
    r = d["rng"]
    nb = int(r.choice([4, 8, 16, 32]))
    md = int(r.choice([nb, 2 * nb, 128, 1000]))
    bidir = int(r.integers(0, 2))
    msl = -(-d["maxlen"] // BS) * BS
    lens = r.integers(0, d["maxlen"] + 1, size=d["B"])
    table = torch.from_numpy(r.standard_normal((d["H"], nb)).astype(np.float32) * 2.0)
    log("random relpos %d: %s nb=%d md=%d bidir=%d" % (
        seed, {k: v for k, v in d.items() if k != "rng"}, nb, md, bidir))
    dc = to_device(workloads.decode_case(6100 + seed, num_seqs=d["B"], num_heads=d["H"],
                                         head_dim=d["D"], lens=lens.tolist(), max_seq_len=msl,
                                         dtype=d["dtype"], bias=None,
                                         sliding_window=d["window"]))
    out = pa.paged_attn_decode_relpos(dc.q, dc.k_cache, dc.v_cache, dc.block_tables,
                                      dc.context_lens, table.to("cuda"), nb, md, bidir,
                                      d["window"], dc.scale, max_seq_len=msl,
                                      partition_tokens=d["partition"])
    h = to_host(dc)
    ref = oracle.decode_relpos(h.q, h.k_cache, h.v_cache, h.block_tables, h.context_lens,
                               table, nb, md, bidir, d["window"], h.scale, msl)
    assert_close(out, ref, d["dtype"], "random relpos decode %d" % seed)
    q_lens = [int(r.integers(0, L + 1)) for L in lens]
    pc = to_device(workloads.prefill_case(6200 + seed, num_seqs=d["B"], num_heads=d["H"],
                                          head_dim=d["D"], lens=lens.tolist(), max_seq_len=msl,
                                          dtype=d["dtype"], bias=None,
                                          sliding_window=d["window"], causal=d["causal"],
                                          q_lens=q_lens))
    out = pa.paged_attn_prefill_relpos(pc.q, pc.k_cache, pc.v_cache, pc.block_tables,
                                       pc.context_lens, pc.query_start_loc, table.to("cuda"),
                                       nb, md, bidir, d["window"], d["causal"], pc.scale,
                                       max_seq_len=msl)
    h = to_host(pc)
    ref = oracle.prefill_relpos(h.q, h.k_cache, h.v_cache, h.block_tables, h.context_lens,
                                h.query_start_loc, table, nb, md, bidir, d["window"],
                                int(d["causal"]), h.scale, msl)
    assert_close(out, ref, d["dtype"], "random relpos prefill %d" % seed)


@pytest.mark.parametrize("seed", range(16))
def test_random_ragged_bias(seed):
    # packed bias offsets over random lengths (zero lengths included), both
    # entry points, both dtypes and head dims
    d = draw(7000 + seed)
    r = d["rng"]
    msl = -(-d["maxlen"] // BS) * BS
    lens = r.integers(0, d["maxlen"] + 1, size=d["B"])
    log("random ragged %d: %s" % (seed, {k: v for k, v in d.items() if k != "rng"}))
    dc = to_device(workloads.decode_case(7100 + seed, num_seqs=d["B"], num_heads=d["H"],
                                         head_dim=d["D"], lens=lens.tolist(), max_seq_len=msl,
                                         dtype=d["dtype"], bias="normal",
                                         sliding_window=d["window"]))
    packed, starts = pack(dc.attn_bias.cpu(), lens)
    out = pa.paged_attn_decode_ragged_bias(dc.q, dc.k_cache, dc.v_cache, dc.block_tables,
                                           dc.context_lens, packed.to("cuda"),
                                           starts.to("cuda"), d["window"], dc.scale,
                                           max_seq_len=msl, partition_tokens=d["partition"])
    h = to_host(dc)
    ref = oracle.decode_ragged(h.q, h.k_cache, h.v_cache, h.block_tables, h.context_lens,
                               packed, starts, d["window"], h.scale, msl)
    assert_close(out, ref, d["dtype"], "random ragged decode %d" % seed)
    q_lens = [int(r.integers(0, L + 1)) for L in lens]
    pc = to_device(workloads.prefill_case(7200 + seed, num_seqs=d["B"], num_heads=d["H"],
                                          head_dim=d["D"], lens=lens.tolist(), max_seq_len=msl,
                                          dtype=d["dtype"], bias="normal",
                                          sliding_window=d["window"], causal=d["causal"],
                                          q_lens=q_lens))
    packed, starts = pack(pc.attn_bias.cpu(), lens, q_lens)
    out = pa.paged_attn_prefill_ragged_bias(pc.q, pc.k_cache, pc.v_cache, pc.block_tables,
                                            pc.context_lens, pc.query_start_loc,
                                            packed.to("cuda"), starts.to("cuda"), d["window"],
                                            d["causal"], pc.scale, max_seq_len=msl)
    h = to_host(pc)
    ref = oracle.prefill_ragged(h.q, h.k_cache, h.v_cache, h.block_tables, h.context_lens,
                                h.query_start_loc, packed, starts, d["window"],
                                int(d["causal"]), h.scale, msl)
    assert_close(out, ref, d["dtype"], "random ragged prefill %d" % seed)


@pytest.mark.parametrize("seed", range(16))
def test_random_chunked(seed):
    """Chunked local attention, decode and prefill, on drawn shapes: chunk
    sizes from 1 to beyond the longest sequence, zero-length sequences and
    partial query sets included."""
    d = draw(6000 + seed)
    chunk = int(d["rng"].choice([1, 3, 16, 31, 64, 129, 1000]))
    msl = -(-d["maxlen"] // BS) * BS
    lens = d["rng"].integers(0, d["maxlen"] + 1, size=d["B"])
    log("random chunked %d: C=%d %s" % (seed, chunk, {k: v for k, v in d.items() if k != "rng"}))
    dc = to_device(workloads.decode_case(6100 + seed, num_seqs=d["B"], num_heads=d["H"],
                                         head_dim=d["D"], lens=lens.tolist(), max_seq_len=msl,
                                         dtype=d["dtype"], bias=d["bias"]))
    out = pa.lib().paged_attn_decode_chunked(dc.q, dc.k_cache, dc.v_cache, dc.block_tables,
                                             dc.context_lens, dc.attn_bias, chunk, dc.scale,
                                             max_seq_len=dc.max_seq_len,
                                             partition_tokens=d["partition"])
    torch.cuda.synchronize()
    h = to_host(dc)
    ref = oracle.decode_chunked(h.q, h.k_cache, h.v_cache, h.block_tables, h.context_lens,
                                h.attn_bias, chunk, h.scale, h.max_seq_len)
    assert_close(out, ref, d["dtype"], "random chunked decode %d" % seed)
    q_lens = [int(d["rng"].integers(0, L + 1)) if d["rng"].integers(0, 2) else int(L)
              for L in lens]
    pc = to_device(workloads.prefill_case(6200 + seed, num_seqs=d["B"], num_heads=d["H"],
                                          head_dim=d["D"], lens=lens.tolist(), max_seq_len=msl,
                                          dtype=d["dtype"],
                                          bias=None if d["bias"] == "zero" else d["bias"],
                                          causal=d["causal"], q_lens=q_lens))
    outp = pa.lib().paged_attn_prefill_chunked(pc.q, pc.k_cache, pc.v_cache, pc.block_tables,
                                               pc.context_lens, pc.query_start_loc,
                                               pc.attn_bias, chunk, pc.causal, pc.scale,
                                               max_seq_len=pc.max_seq_len)
    torch.cuda.synchronize()
    hp = to_host(pc)
    refp = oracle.prefill_chunked(hp.q, hp.k_cache, hp.v_cache, hp.block_tables,
                                  hp.context_lens, hp.query_start_loc, hp.attn_bias, chunk,
                                  int(hp.causal), hp.scale, hp.max_seq_len)
    assert_close(outp, refp, d["dtype"], "random chunked prefill %d" % seed)
