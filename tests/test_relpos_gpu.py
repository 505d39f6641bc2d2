"""GPU parity of the in-kernel T5 relative-position bias (decode and prefill)
against the float64 oracle, and bit-identity with the materialised-bias path
when the materialised bias holds the same bucket values."""
import numpy as np
import pytest
import torch

import oracle
import workloads
from gpu_helpers import assert_close, gpu_decode, gpu_prefill, log, to_device, to_host

import sliding_window_mask_amd as pa

pytestmark = pytest.mark.gpu
DEV = "cuda"


def decode_relpos(case, table, nb, md, bidir, window=None, partition=0):
    out = pa.paged_attn_decode_relpos(case.q, case.k_cache, case.v_cache, case.block_tables,
                                      case.context_lens, table, nb, md, bidir,
                                      case.sliding_window if window is None else window,
                                      case.scale, max_seq_len=case.max_seq_len,
                                      partition_tokens=partition)
    torch.cuda.synchronize()
    return out


def oracle_decode_relpos(case, table, nb, md, bidir, window=None):
    h = to_host(case)
    return oracle.decode_relpos(h.q, h.k_cache, h.v_cache, h.block_tables, h.context_lens,
                                table.cpu(), nb, md, bidir,
                                h.sliding_window if window is None else window, h.scale,
                                h.max_seq_len)


def test_t5_small_decode_inline_equals_materialised_bit_exact():
    log("t5 small decode: inline vs materialised")
    case = to_device(workloads.t5_small_self_decode_bf16())
    dense = gpu_decode(case)
    inline = decode_relpos(case, case.t5_table, 32, 128, 0)
    assert torch.equal(inline.view(torch.int16), dense.view(torch.int16))
    assert_close(inline, oracle_decode_relpos(case, case.t5_table, 32, 128, 0), torch.bfloat16,
                 "t5 inline")


@pytest.mark.parametrize("nb,md,bidir", [(32, 128, 0), (32, 128, 1), (16, 40, 0), (64, 1024, 0),
                                         (2, 5, 0), (8, 9, 1)])
@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
def test_decode_relpos_shapes(nb, md, bidir, dtype):
    case = to_device(workloads.decode_case(700 + nb + md, num_seqs=6, num_heads=3, head_dim=64,
                                           lens=(1, 600), max_seq_len=608, dtype=dtype,
                                           bias=None))
    g = torch.Generator().manual_seed(nb * md)
    table = (torch.randn(3, nb, generator=g) * 2.0).to(DEV)
    ref = oracle_decode_relpos(case, table, nb, md, bidir)
    for p in (0, 64):
        assert_close(decode_relpos(case, table, nb, md, bidir, partition=p), ref, dtype,
                     "relpos nb=%d md=%d bidir=%d P=%d" % (nb, md, bidir, p))


def test_decode_relpos_with_window():
    case = to_device(workloads.decode_case(720, num_seqs=5, num_heads=2, head_dim=128,
                                           lens=(50, 400), max_seq_len=400,
                                           dtype=torch.bfloat16, bias=None, sliding_window=37,
                                           evict_before=37))
    table = (torch.randn(2, 32, generator=torch.Generator().manual_seed(1))).to(DEV)
    assert_close(decode_relpos(case, table, 32, 128, 0), oracle_decode_relpos(
        case, table, 32, 128, 0), torch.bfloat16, "relpos window")


@pytest.mark.parametrize("bidir,causal", [(1, False), (0, True), (1, True), (0, False)])
@pytest.mark.parametrize("window", [-1, 64])
def test_prefill_relpos(bidir, causal, window):
    case = to_device(workloads.prefill_case(730 + bidir, num_seqs=4, num_heads=3, head_dim=64,
                                            lens=[1, 70, 200, 333], max_seq_len=336,
                                            dtype=torch.float32, sliding_window=window,
                                            causal=causal))
    table = (torch.randn(3, 32, generator=torch.Generator().manual_seed(2)) * 0.5).to(DEV)
    out = pa.paged_attn_prefill_relpos(case.q, case.k_cache, case.v_cache, case.block_tables,
                                       case.context_lens, case.query_start_loc, table, 32, 128,
                                       bidir, window, causal, case.scale,
                                       max_seq_len=case.max_seq_len)
    torch.cuda.synchronize()
    h = to_host(case)
    ref = oracle.prefill_relpos(h.q, h.k_cache, h.v_cache, h.block_tables, h.context_lens,
                                h.query_start_loc, table.cpu(), 32, 128, bidir, window,
                                int(causal), h.scale, h.max_seq_len)
    assert_close(out, ref, torch.float32, "prefill relpos bidir=%d causal=%s W=%d"
                 % (bidir, causal, window))
    # the same values as a materialised bias give the identical result
    pos = np.arange(case.max_seq_len)
    buckets = oracle.t5_bucket(pos[None, :] - pos[:, None], bidir, 32, 128)
    dense = table.cpu()[:, torch.from_numpy(buckets.astype(np.int64))]
    dense = dense[None].expand(case.num_seqs, -1, -1, -1).contiguous().to(DEV)
    assert torch.equal(gpu_prefill(case, bias=dense), out)


@pytest.mark.parametrize("nb,bidir,causal", [(8, 0, True), (16, 1, False), (16, 1, True)])
@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
def test_prefill_relpos_end_bucket_edge(nb, bidir, causal, dtype):
    # max distance one past the exact buckets (4 per direction here): distance
    # 4 keeps bucket 4, distance 5 and beyond fall in the end bucket 7, so a
    # tile the kernels treat as wholly beyond the maximum distance one key too
    # early changes the result. Query sets starting at positions 3 and 29 put
    # a wave's first row exactly 4 keys past the end of a 32-key tile (and of
    # a 16-key chunk), and 4 keys before the start of one; lengths span many
    # tiles on both sides of each row
    md = 5
    case = to_device(workloads.prefill_case(760 + nb + causal, num_seqs=4, num_heads=2,
                                            head_dim=64, lens=[1, 40, 130, 300],
                                            q_lens=[1, 37, 101, 263], max_seq_len=304,
                                            dtype=dtype, causal=causal))
    table = (torch.randn(2, nb, generator=torch.Generator().manual_seed(nb)) * 2.0).to(DEV)
    half = nb // 2 if bidir else nb
    b_in = oracle.t5_bucket(np.array([-(md - 1), -md]), bidir, nb, md)
    assert b_in[0] != b_in[1] and b_in[1] == half - 1       # the edge is visible
    out = pa.paged_attn_prefill_relpos(case.q, case.k_cache, case.v_cache, case.block_tables,
                                       case.context_lens, case.query_start_loc, table, nb, md,
                                       bidir, -1, causal, case.scale,
                                       max_seq_len=case.max_seq_len)
    h = to_host(case)
    ref = oracle.prefill_relpos(h.q, h.k_cache, h.v_cache, h.block_tables, h.context_lens,
                                h.query_start_loc, table.cpu(), nb, md, bidir, -1, int(causal),
                                h.scale, h.max_seq_len)
    assert_close(out, ref, dtype, "prefill relpos end bucket nb=%d bidir=%d causal=%s %s"
                 % (nb, bidir, causal, dtype))


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
@pytest.mark.parametrize("bidir,causal,window", [(1, False, -1), (0, True, -1), (1, False, 64)])
def test_prefill_relpos_full_size_every_sequence(dtype, bidir, causal, window):
    # the ModernBERT-shaped layer (32 sequences of U[64, 1024] tokens, 12
    # heads, head_dim 64) with a T5 bias of 32 buckets and maximum distance
    # 128 as the benchmark times it: encoder buckets (bidirectional, with and
    # without a 64-token window) and decoder buckets (causal); every sequence
    # against the oracle
    what = "full-size relpos %s bidir=%d causal=%s W=%d" % (dtype, bidir, causal, window)
    log(what)
    case = workloads.prefill_case(4, num_seqs=32, num_heads=12, head_dim=64, lens=(64, 1024),
                                  max_seq_len=1024, dtype=dtype, sliding_window=window,
                                  causal=causal, device=DEV, layer_seed=[4, 0])
    table = (torch.randn(12, 32, generator=torch.Generator().manual_seed(5)) * 0.5).to(DEV)
    out = pa.paged_attn_prefill_relpos(case.q, case.k_cache, case.v_cache, case.block_tables,
                                       case.context_lens, case.query_start_loc, table, 32, 128,
                                       bidir, window, causal, case.scale,
                                       max_seq_len=case.max_seq_len)
    h = to_host(case)
    ref = oracle.prefill_relpos(h.q, h.k_cache, h.v_cache, h.block_tables, h.context_lens,
                                h.query_start_loc, table.cpu(), 32, 128, bidir, window,
                                int(causal), h.scale, h.max_seq_len)
    assert_close(out, ref, dtype, what)
