"""Checks of the seeded input generators (CPU only)."""
import os

import numpy as np
import torch

import workloads

BS = workloads.BLOCK_SIZE
GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def test_generators_are_deterministic():
    a = workloads.tiny_decode_f32()
    b = workloads.tiny_decode_f32()
    for name in ("q", "k_cache", "v_cache", "block_tables", "context_lens", "attn_bias"):
        x, y = getattr(a, name), getattr(b, name)
        assert torch.equal(torch.nan_to_num(x, nan=7.0), torch.nan_to_num(y, nan=7.0)), name
    c = workloads.decode_case(2, num_seqs=4, num_heads=4, head_dim=64, lens=(1, 100),
                              max_seq_len=128, dtype=torch.float32, num_blocks=64)
    assert not torch.equal(a.context_lens, c.context_lens) or not torch.equal(
        torch.nan_to_num(a.q), torch.nan_to_num(c.q))


def test_tiny_decode_shapes():
    c = workloads.tiny_decode_f32()
    assert c.q.shape == (4, 4, 64) and c.q.dtype == torch.float32
    assert c.k_cache.shape == (64, 4, 16, 64)
    assert c.block_tables.shape == (4, 8)
    assert c.attn_bias.shape == (4, 4, 128)
    assert c.scale == 0.125
    assert np.all((c.lens >= 1) & (c.lens <= 100))


def test_block_assignment_and_poison():
    c = workloads.t5_large_cross_decode_bf16()
    L = c.lens
    seen = set()
    for b in range(c.num_seqs):
        n = -(-int(L[b]) // BS)
        ids = c.block_tables[b, :n].tolist()
        assert len(set(ids)) == n and not (set(ids) & seen) and c.poison_block not in ids
        seen |= set(ids)
        assert all(x == c.poison_block for x in c.block_tables[b, n:].tolist())
        # valid slots are finite, the tail of the last block is NaN
        last = c.block_tables[b, n - 1].long()
        tail = int(L[b]) - (n - 1) * BS
        assert torch.isfinite(c.k_cache[last, :, :tail].float()).all()
        assert torch.isnan(c.k_cache[last, :, tail:].float()).all()
    # decoy (self-attention) blocks are disjoint from the cross table and NaN
    for b in range(c.num_seqs):
        n = -(-int(c.decoy_lens[b]) // BS)
        ids = c.decoy_table[b, :n].tolist()
        assert not (set(ids) & seen)
        assert torch.isnan(c.k_cache[torch.tensor(ids)].float()).all()
    assert torch.isnan(c.v_cache[c.poison_block].float()).all()


def test_bias_padding_is_nan():
    c = workloads.tiny_decode_f32()
    for b in range(4):
        L = int(c.lens[b])
        assert torch.isfinite(c.attn_bias[b, :, :L]).all()
        assert torch.isnan(c.attn_bias[b, :, L:]).all()


def test_eviction_unmaps_blocks_before_window():
    c = workloads.decode_case(3, num_seqs=6, num_heads=2, head_dim=64, lens=(40, 120),
                              max_seq_len=128, dtype=torch.bfloat16, bias="normal",
                              sliding_window=20, evict_before=20)
    for b in range(6):
        L = int(c.lens[b])
        first = max(L - 20, 0) // BS
        assert all(x == c.poison_block for x in c.block_tables[b, :first].tolist())
        assert torch.isnan(c.attn_bias[b, :, :first * BS]).all()
        assert torch.isfinite(c.attn_bias[b, :, first * BS:L]).all()


def test_t5_bucket_exact_range():
    n = np.arange(16)
    assert np.array_equal(workloads.t5_bucket(n), n)


def test_t5_bucket_monotone_and_clamped():
    n = np.arange(0, 5000)
    b = workloads.t5_bucket(n)
    assert np.all(np.diff(b) >= 0)
    assert b.max() == 31 and b.min() == 0
    # beyond the maximum distance 128 every distance uses the last bucket
    assert np.all(b[128:] == 31)
    # negative distances (keys after the query) map to bucket 0
    assert np.all(workloads.t5_bucket(-np.arange(1, 50)) == 0)


def test_t5_materialised_bias_reuses_last_bucket_beyond_128():
    c = workloads.t5_small_self_decode_bf16()
    tab = c.t5_table
    for b in range(c.num_seqs):
        L = int(c.lens[b])
        far = [j for j in range(L) if L - 1 - j >= 128]
        if far:
            got = c.attn_bias[b, :, far]
            assert torch.equal(got, tab[:, 31:32].expand_as(got))
        # distance 0 (the query's own position) uses bucket 0
        assert torch.equal(c.attn_bias[b, :, L - 1], tab[:, 0])


def test_modernbert_schedule_matches_printed_layers():
    rows = [ln.split() for ln in open(os.path.join(GOLDEN, "modernbert_layer_windows.txt"))
            if ln.strip() and not ln.startswith("#")]
    assert len(rows) == 6
    for layer1, kind, window in rows:
        assert workloads.modernbert_window(int(layer1) - 1) == int(window)
        assert (kind == "full_attention") == (int(window) == -1)


def test_prefill_case_layout():
    c = workloads.prefill_case(9, num_seqs=3, num_heads=2, head_dim=64, lens=[5, 16, 17],
                               max_seq_len=32, dtype=torch.float32)
    assert c.query_start_loc.tolist() == [0, 5, 21, 38]
    assert c.q.shape == (38, 2, 64)
