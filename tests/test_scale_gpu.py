"""GPU parity for the sign of the scale: a negative scale (low scores weigh
most) and a zero scale (every visible key weighs the same), with a
materialised bias and with the in-kernel T5 bias, on every kernel family:
decode (split and single partition), fp32 prefill and bf16 prefill. The
bf16 prefill keeps scores unscaled until the exponent and folds the sign
into q and the bias, so these cases exercise that fold."""
import pytest
import torch

import oracle
import workloads
from gpu_helpers import assert_close, gpu_decode, gpu_prefill, log, oracle_decode, \
    oracle_prefill, to_device, to_host

import sliding_window_mask_amd as pa

pytestmark = pytest.mark.gpu
DEV = "cuda"
DTYPES = [torch.float32, torch.bfloat16]
SCALES = [-0.3, 0.0]


@pytest.mark.parametrize("dtype", DTYPES)
@pytest.mark.parametrize("scale", SCALES)
@pytest.mark.parametrize("window", [-1, 20])
def test_decode_scale_sign(dtype, scale, window):
    log("decode scale=%g dtype=%s W=%d" % (scale, dtype, window))
    case = to_device(workloads.decode_case(1300 + window, num_seqs=5, num_heads=3, head_dim=64,
                                           lens=(1, 300), max_seq_len=304, dtype=dtype,
                                           bias="normal", sliding_window=window, scale=scale))
    ref = oracle_decode(case)
    for p in (0, 64):
        assert_close(gpu_decode(case, partition=p), ref, dtype,
                     "decode scale=%g W=%d P=%d" % (scale, window, p))


@pytest.mark.parametrize("dtype", DTYPES)
@pytest.mark.parametrize("scale", SCALES)
@pytest.mark.parametrize("causal,window", [(False, -1), (True, -1), (False, 9)])
def test_prefill_scale_sign(dtype, scale, causal, window):
    log("prefill scale=%g dtype=%s causal=%s W=%d" % (scale, dtype, causal, window))
    case = to_device(workloads.prefill_case(1310 + window, num_seqs=4, num_heads=3, head_dim=64,
                                            lens=[1, 33, 70, 140], max_seq_len=144,
                                            dtype=dtype, bias="normal", sliding_window=window,
                                            causal=causal, scale=scale))
    assert_close(gpu_prefill(case), oracle_prefill(case), dtype,
                 "prefill scale=%g causal=%s W=%d" % (scale, causal, window))
    assert_close(gpu_prefill(case, bias=None), oracle_prefill(case, bias=None), dtype,
                 "prefill no bias scale=%g" % scale)


@pytest.mark.parametrize("dtype", DTYPES)
@pytest.mark.parametrize("scale", SCALES)
def test_relpos_scale_sign(dtype, scale):
    log("relpos scale=%g dtype=%s" % (scale, dtype))
    table = (torch.randn(3, 32, generator=torch.Generator().manual_seed(13)) * 2.0).to(DEV)
    pc = to_device(workloads.prefill_case(1320, num_seqs=3, num_heads=3, head_dim=64,
                                          lens=[50, 129, 200], max_seq_len=208, dtype=dtype,
                                          bias=None, causal=True, scale=scale))
    out = pa.paged_attn_prefill_relpos(pc.q, pc.k_cache, pc.v_cache, pc.block_tables,
                                       pc.context_lens, pc.query_start_loc, table, 32, 128, 0,
                                       -1, True, pc.scale, max_seq_len=pc.max_seq_len)
    torch.cuda.synchronize()
    h = to_host(pc)
    ref = oracle.prefill_relpos(h.q, h.k_cache, h.v_cache, h.block_tables, h.context_lens,
                                h.query_start_loc, table.cpu(), 32, 128, 0, -1, 1, h.scale,
                                h.max_seq_len)
    assert_close(out, ref, dtype, "prefill relpos scale=%g" % scale)
    dc = to_device(workloads.decode_case(1321, num_seqs=4, num_heads=3, head_dim=64,
                                         lens=(1, 250), max_seq_len=256, dtype=dtype, bias=None,
                                         scale=scale))
    out = pa.paged_attn_decode_relpos(dc.q, dc.k_cache, dc.v_cache, dc.block_tables,
                                      dc.context_lens, table, 32, 128, 0, -1, dc.scale,
                                      max_seq_len=dc.max_seq_len)
    torch.cuda.synchronize()
    h = to_host(dc)
    ref = oracle.decode_relpos(h.q, h.k_cache, h.v_cache, h.block_tables, h.context_lens,
                               table.cpu(), 32, 128, 0, -1, h.scale, h.max_seq_len)
    assert_close(out, ref, dtype, "decode relpos scale=%g" % scale)
