"""GPU parity of the chunked-local-attention entry points (paged_attn_decode_chunked,
paged_attn_prefill_chunked, through the C ABI) against the float64 oracle.

A query at position p sees the keys j of its own chunk, floor(j / C) ==
floor(p / C) (causal prefill: also j <= p); the decode query sits at L-1.
Cases cover chunk sizes from 1 to beyond every length, chunks that start
inside a 16-token block and chunks that are not a multiple of the key tiles,
bias or none, both dtypes and head dims, several decode partitions, partial
query sets, and blocks before a decode query's chunk pointed at a NaN block
(never read)."""
import numpy as np
import pytest
import torch

import oracle
import sliding_window_mask_amd as pa
import workloads
from gpu_helpers import assert_close, log, to_device, to_host

pytestmark = pytest.mark.gpu


def gpu_decode_chunked(case, chunk, partition=0):
    out = pa.lib().paged_attn_decode_chunked(case.q, case.k_cache, case.v_cache,
                                             case.block_tables, case.context_lens,
                                             case.attn_bias, chunk, case.scale,
                                             max_seq_len=case.max_seq_len,
                                             partition_tokens=partition)
    torch.cuda.synchronize()
    return out


def oracle_decode_chunked(case, chunk):
    h = to_host(case)
    return oracle.decode_chunked(h.q, h.k_cache, h.v_cache, h.block_tables, h.context_lens,
                                 h.attn_bias, chunk, h.scale, h.max_seq_len)


def gpu_prefill_chunked(case, chunk):
    out = pa.lib().paged_attn_prefill_chunked(case.q, case.k_cache, case.v_cache,
                                              case.block_tables, case.context_lens,
                                              case.query_start_loc, case.attn_bias, chunk,
                                              case.causal, case.scale,
                                              max_seq_len=case.max_seq_len)
    torch.cuda.synchronize()
    return out


def oracle_prefill_chunked(case, chunk):
    h = to_host(case)
    return oracle.prefill_chunked(h.q, h.k_cache, h.v_cache, h.block_tables, h.context_lens,
                                  h.query_start_loc, h.attn_bias, chunk, int(h.causal),
                                  h.scale, h.max_seq_len)


@pytest.mark.parametrize("dtype,D", [(torch.float32, 64), (torch.bfloat16, 128)])
@pytest.mark.parametrize("chunk", [1, 7, 16, 33, 256, 5000])
@pytest.mark.parametrize("bias", ["normal", None])
def test_decode_chunked(dtype, D, chunk, bias):
    log("decode chunked %s D=%d C=%d bias=%s" % (dtype, D, chunk, bias))
    case = to_device(workloads.decode_case(3000 + chunk, num_seqs=9, num_heads=3, head_dim=D,
                                           lens=(1, 700), max_seq_len=720, dtype=dtype,
                                           bias=bias))
    ref = oracle_decode_chunked(case, chunk)
    for partition in (0, 64):
        assert_close(gpu_decode_chunked(case, chunk, partition), ref, dtype,
                     "decode chunked C=%d P=%d" % (chunk, partition))


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
def test_decode_chunked_never_reads_before_the_chunk(dtype):
    """Blocks wholly before each query's chunk point at the NaN-filled poison
    block, and the bias there is NaN: the result must still be the oracle's."""
    C = 100
    case = workloads.decode_case(3100, num_seqs=8, num_heads=2, head_dim=64, lens=(150, 600),
                                 max_seq_len=640, dtype=dtype, bias="normal")
    for b in range(case.num_seqs):
        start = (int(case.lens[b]) - 1) // C * C
        case.block_tables[b, :start // 16] = case.poison_block
        case.attn_bias[b, :, :start] = float("nan")
    case = to_device(case)
    out = gpu_decode_chunked(case, C)
    assert torch.isfinite(out).all()
    assert_close(out, oracle_decode_chunked(case, C), dtype, "decode chunked, evicted")


@pytest.mark.parametrize("dtype,D", [(torch.float32, 64), (torch.float32, 128),
                                     (torch.bfloat16, 64), (torch.bfloat16, 128)])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("chunk", [1, 5, 16, 40, 64, 100, 1000])
def test_prefill_chunked(dtype, D, causal, chunk):
    log("prefill chunked %s D=%d causal=%s C=%d" % (dtype, D, causal, chunk))
    lens = [1, 17, 63, 64, 65, 130, 257]
    case = to_device(workloads.prefill_case(3200 + chunk, num_seqs=len(lens), num_heads=2,
                                            head_dim=D, lens=lens, max_seq_len=272,
                                            dtype=dtype, causal=causal))
    assert_close(gpu_prefill_chunked(case, chunk), oracle_prefill_chunked(case, chunk), dtype,
                 "prefill chunked C=%d causal=%s" % (chunk, causal))


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("chunk", [9, 48])
def test_prefill_chunked_with_bias_and_partial_queries(dtype, causal, chunk):
    lens = [5, 40, 100, 200]
    case = to_device(workloads.prefill_case(3300 + chunk, num_seqs=4, num_heads=2, head_dim=64,
                                            lens=lens, q_lens=[5, 1, 70, 133],
                                            max_seq_len=208, dtype=dtype, causal=causal,
                                            bias="normal"))
    assert_close(gpu_prefill_chunked(case, chunk), oracle_prefill_chunked(case, chunk), dtype,
                 "prefill chunked, bias, partial q, C=%d causal=%s" % (chunk, causal))


def test_prefill_chunked_one_is_own_value():
    """Chunks of one position: every row returns its own value row exactly."""
    case = to_device(workloads.prefill_case(3400, num_seqs=3, num_heads=2, head_dim=64,
                                            lens=[1, 30, 77], max_seq_len=80,
                                            dtype=torch.float32, bias="normal"))
    out = gpu_prefill_chunked(case, 1).cpu()
    h = to_host(case)
    for b in range(3):
        L = int(h.lens[b])
        q0 = int(h.query_start_loc[b])
        for t in range(L):
            blk = int(h.block_tables[b, t // 16])
            assert torch.equal(out[q0 + t], h.v_cache[blk, :, t % 16, :])


def test_modernbert_shaped_chunked_layer_sampled():
    """A ModernBERT-shaped layer (32 sequences of U[64,1024], 12 heads) with
    128-token chunks, in the launch configuration of the windowed layers; the
    oracle checks a sample of whole sequences."""
    from gpu_helpers import sample_prefill
    case = workloads.prefill_case(4, num_seqs=32, num_heads=12, head_dim=64, lens=(64, 1024),
                                  max_seq_len=1024, dtype=torch.float32, device="cuda",
                                  layer_seed=[4, 1])
    out = gpu_prefill_chunked(case, 128).cpu().double().numpy()
    sub = sample_prefill(case, [0, 7, 19, 31])
    ref = oracle_prefill_chunked(sub, 128)
    err = float(np.max(np.abs(out[sub.rows.numpy()] - ref)))
    log("modernbert chunked sample max err %.3g" % err)
    assert err <= 1e-5
