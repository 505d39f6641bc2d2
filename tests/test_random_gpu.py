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
