"""GPU parity of the bf16 MFMA prefill (v_mfma_f32_16x16x32_bf16) against the
float64 oracle on the same bf16-rounded inputs: lengths, windows, causal
masks, partial query sets, materialised / ragged / T5 biases, and a
ModernBERT-shaped layer in bf16 checked on sampled sequences."""
import numpy as np
import pytest
import torch

import oracle
import workloads
from gpu_helpers import (BS, assert_close, gpu_prefill, log, oracle_prefill, sample_prefill,
                         to_device, to_host)

import sliding_window_mask_amd as pa

pytestmark = pytest.mark.gpu
DEV = "cuda"
BF = torch.bfloat16


def small(seed, lens, D=64, H=3, window=-1, causal=False, bias=None, q_lens=None, msl=None):
    msl = msl or max(16, -(-max(lens) // 16) * 16)
    return workloads.prefill_case(seed, num_seqs=len(lens), num_heads=H, head_dim=D, lens=lens,
                                  max_seq_len=msl, dtype=BF, bias=bias, sliding_window=window,
                                  causal=causal, q_lens=q_lens)


@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("window", [-1, 1, 3, 16, 64])
@pytest.mark.parametrize("causal", [False, True])
def test_small_prefill_bf16(D, window, causal):
    lens = [1, 15, 16, 17, 31, 32, 33, 63, 64, 65, 130]
    case = to_device(small(900 + D + window, lens, D=D, window=window, causal=causal))
    out = gpu_prefill(case)
    assert out.dtype == BF
    assert_close(out, oracle_prefill(case), BF, "bf16 D=%d W=%d causal=%s" % (D, window, causal))


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("window", [-1, 9])
def test_prefill_bf16_with_bias(causal, window):
    case = to_device(small(910, [5, 33, 70, 129], window=window, causal=causal, bias="normal",
                           msl=144))
    assert_close(gpu_prefill(case), oracle_prefill(case), BF, "bf16 bias")


def test_prefill_bf16_partial_queries():
    case = to_device(small(920, [40, 17, 100, 130], q_lens=[4, 17, 1, 70], window=21,
                           causal=True, msl=144))
    assert_close(gpu_prefill(case), oracle_prefill(case), BF, "bf16 partial q")


def test_prefill_bf16_window_one_returns_own_value():
    case = to_device(small(930, [1, 20, 77], window=1))
    out = gpu_prefill(case).cpu()
    qsl = case.query_start_loc.cpu()
    for b in range(3):
        for t in range(int(case.lens[b])):
            v = case.v_cache[case.block_tables[b, t // BS].long(), :, t % BS, :].cpu()
            assert torch.equal(out[int(qsl[b]) + t].view(torch.int16), v.view(torch.int16))


@pytest.mark.parametrize("bidir,causal", [(1, False), (0, True)])
def test_prefill_bf16_relpos(bidir, causal):
    case = to_device(small(940, [70, 200, 333], causal=causal, msl=336))
    table = (torch.randn(3, 32, generator=torch.Generator().manual_seed(4)) * 0.5).to(DEV)
    out = pa.paged_attn_prefill_relpos(case.q, case.k_cache, case.v_cache, case.block_tables,
                                       case.context_lens, case.query_start_loc, table, 32, 128,
                                       bidir, -1, causal, case.scale,
                                       max_seq_len=case.max_seq_len)
    torch.cuda.synchronize()
    h = to_host(case)
    ref = oracle.prefill_relpos(h.q, h.k_cache, h.v_cache, h.block_tables, h.context_lens,
                                h.query_start_loc, table.cpu(), 32, 128, bidir, -1, int(causal),
                                h.scale, h.max_seq_len)
    assert_close(out, ref, BF, "bf16 relpos")


def test_prefill_bf16_deterministic():
    case = to_device(small(950, [300, 511, 64], window=64, msl=512))
    a = gpu_prefill(case)
    assert torch.equal(gpu_prefill(case).view(torch.int16), a.view(torch.int16))


@pytest.mark.parametrize("layer,causal,bias", [(0, False, None), (1, False, None),
                                               (0, True, None), (0, False, "normal"),
                                               (0, True, "normal"), (1, False, "normal")])
def test_modernbert_shaped_bf16_layer_every_sequence(layer, causal, bias):
    """A full-attention (0) and a window-64 (1) layer of the bf16 ModernBERT-
    shaped prefill, the full-attention one under a causal mask, and each with
    a materialised fp32 bias [32, 12, 1024, 1024], as the benchmark launches
    them, with every one of the 32 sequences (all heads and queries) against
    the oracle."""
    what = "bf16 layer %d causal=%s bias=%s all sequences" % (layer, causal, bias)
    log(what)
    case = workloads.prefill_case(4, num_seqs=32, num_heads=12, head_dim=64, lens=(64, 1024),
                                  max_seq_len=1024, dtype=BF, bias=bias,
                                  sliding_window=workloads.modernbert_window(layer),
                                  causal=causal, device=DEV, layer_seed=[4, layer])
    out = gpu_prefill(case)
    assert_close(out, oracle_prefill(case), BF, what)


@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("bias", [None, "normal", "relpos"])
@pytest.mark.parametrize("partial", [False, True])
def test_prefill_bf16_bidirectional_128_query_tiles(D, bias, partial):
    # bidirectional launches without a window run in workgroups of 128 queries
    # (four waves of 32, 32x32x16 MFMAs): lengths on both sides of 32 and 128
    # and their multiples, a last wave with one query, and query sets that
    # start part-way into the sequence (the last n_q positions)
    lens = [1, 31, 32, 33, 97, 127, 128, 129, 160, 255, 257, 300]
    q_lens = [L for L in lens] if not partial else [1, 30, 1, 32, 96, 1, 127, 128, 33, 200,
                                                    129, 171]
    msl = 304
    scale = -0.09 if partial else None   # a negative scale on the partial sets
    log("bf16 128-query tiles D=%d bias=%s partial=%s" % (D, bias, partial))
    case = to_device(workloads.prefill_case(1500 + D + 3 * partial, num_seqs=len(lens),
                                            num_heads=2, head_dim=D, lens=lens, max_seq_len=msl,
                                            dtype=BF, bias="normal" if bias == "normal" else None,
                                            q_lens=q_lens, scale=scale))
    if bias != "relpos":
        assert_close(gpu_prefill(case), oracle_prefill(case), BF,
                     "bf16 128-query tiles D=%d bias=%s partial=%s" % (D, bias, partial))
        return
    nb, md = 16, 64
    table = torch.from_numpy(np.random.default_rng(D).standard_normal((2, nb)).astype(np.float32))
    out = pa.paged_attn_prefill_relpos(case.q, case.k_cache, case.v_cache, case.block_tables,
                                       case.context_lens, case.query_start_loc, table.to(DEV),
                                       nb, md, 1, -1, False, case.scale, max_seq_len=msl)
    h = to_host(case)
    ref = oracle.prefill_relpos(h.q, h.k_cache, h.v_cache, h.block_tables, h.context_lens,
                                h.query_start_loc, table, nb, md, 1, -1, 0, h.scale, msl)
    assert_close(out, ref, BF, "bf16 128-query tiles relpos D=%d partial=%s" % (D, partial))


@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("bias", [None, "relpos"])
@pytest.mark.parametrize("partial", [False, True])
def test_prefill_bf16_causal_128_query_tiles(D, bias, partial):
    # causal launches without a window or a materialised bias at head_dim 64
    # also run in workgroups of 128 queries: the workgroup stages keys up to
    # its last row, each wave stops after the tile holding its own last row and
    # masks only the tiles crossing its diagonal; query sets that start
    # part-way into the sequence move the diagonal off the tile grid
    lens = [1, 31, 32, 33, 97, 127, 128, 129, 160, 255, 257, 300]
    q_lens = [L for L in lens] if not partial else [1, 30, 1, 32, 96, 1, 127, 128, 33, 200,
                                                    129, 171]
    msl = 304
    log("bf16 causal 128-query tiles D=%d bias=%s partial=%s" % (D, bias, partial))
    case = to_device(workloads.prefill_case(1600 + D + 3 * partial, num_seqs=len(lens),
                                            num_heads=2, head_dim=D, lens=lens, max_seq_len=msl,
                                            dtype=BF, causal=True, q_lens=q_lens,
                                            scale=-0.09 if partial else None))
    what = "bf16 causal 128-query tiles D=%d bias=%s partial=%s" % (D, bias, partial)
    if bias is None:
        assert_close(gpu_prefill(case), oracle_prefill(case), BF, what)
        return
    # decoder self-attention buckets (one direction), as a T5 decoder's prompt
    nb, md = 32, 128
    table = torch.from_numpy(
        np.random.default_rng(D + 7).standard_normal((2, nb)).astype(np.float32))
    out = pa.paged_attn_prefill_relpos(case.q, case.k_cache, case.v_cache, case.block_tables,
                                       case.context_lens, case.query_start_loc, table.to(DEV),
                                       nb, md, 0, -1, True, case.scale, max_seq_len=msl)
    h = to_host(case)
    ref = oracle.prefill_relpos(h.q, h.k_cache, h.v_cache, h.block_tables, h.context_lens,
                                h.query_start_loc, table, nb, md, 0, -1, 1, h.scale, msl)
    assert_close(out, ref, BF, what)


def _pack_rows(dense, lens, q_lens):
    """The ragged layout of a padded prefill bias: per sequence, the rows of
    its n_q queries over its L keys, heads outermost."""
    parts, starts, off = [], [], 0
    for b, (L, nq) in enumerate(zip(lens, q_lens)):
        L, nq = int(L), int(nq)
        parts.append(dense[b, :, L - nq:L, :L].reshape(-1))
        starts.append(off)
        off += dense.shape[1] * nq * L
    return torch.cat(parts).contiguous(), torch.tensor(starts, dtype=torch.int64)


@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("partial", [False, True])
@pytest.mark.parametrize("causal", [False, True])
def test_prefill_bf16_bias_read_paths_agree(D, partial, causal):
    # launches without a window read the bias of whole 32-key tiles (causal:
    # tiles every row of the wave sees whole) as 128-byte row segments passed
    # between lanes through LDS when every row is 16-byte aligned, and entry
    # by entry otherwise: a padded bias with row pitch 320 (aligned), the same
    # values with pitch 306 (not aligned) and the ragged layout (rows of L
    # entries, aligned or not) must give bit-identical outputs, and match the
    # oracle
    lens = [31, 32, 64, 100, 129, 256, 257, 300]
    q_lens = lens if not partial else [1, 32, 33, 99, 2, 200, 129, 300]
    what = "bf16 bias read paths D=%d partial=%s causal=%s" % (D, partial, causal)
    log(what)
    case = to_device(workloads.prefill_case(1600 + D + partial, num_seqs=len(lens), num_heads=2,
                                            head_dim=D, lens=lens, max_seq_len=320, dtype=BF,
                                            bias="normal", q_lens=q_lens, causal=causal))
    out_a = gpu_prefill(case)
    bias_b = case.attn_bias[:, :, :306, :306].contiguous()
    out_b = pa.paged_attn_prefill(case.q, case.k_cache, case.v_cache, case.block_tables,
                                  case.context_lens, case.query_start_loc, bias_b, -1, causal,
                                  case.scale, max_seq_len=306)
    packed, starts = _pack_rows(case.attn_bias.cpu(), case.lens, case.q_lens)
    out_c = pa.paged_attn_prefill_ragged_bias(case.q, case.k_cache, case.v_cache,
                                              case.block_tables, case.context_lens,
                                              case.query_start_loc, packed.to(DEV),
                                              starts.to(DEV), -1, causal, case.scale,
                                              max_seq_len=320)
    torch.cuda.synchronize()
    assert_close(out_a, oracle_prefill(case), BF, what)
    assert torch.equal(out_a.view(torch.int16), out_b.view(torch.int16))
    assert torch.equal(out_a.view(torch.int16), out_c.view(torch.int16))
