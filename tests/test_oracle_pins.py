"""Pins for the float64 oracle (CPU only).

The oracle is trusted only because these checks tie it to things it does not
compute itself:

* PyTorch's float64 ``scaled_dot_product_attention`` applied to K/V that the
  test un-pages with plain tensor indexing, with the additive mask
  ``scale * A + M`` (M = 0 or -inf from the window / causal definition). This
  pins the whole formula of "PagedAttention: Support custom attention bias for
  T5 model" (attention equation in the PR description), the gather through
  the block table, bias indexing, windows and query positions.
* Hand-worked closed forms whose expected value is derived in the comments.
* Special cases: L = 1, W = 1, W >= L, empty and fully masked rows, a null
  bias equal to a zero bias, a constant bias equal to none, relabelled
  physical blocks, and a bias "probe" that isolates one key.

Each check is chosen so that a plausible slip in the oracle (dropping the bias,
adding it after the scale, a wrong block/slot/head index, a transposed bias
index, an off-by-one window edge, a reversed causal mask, a wrong prefill
query position) fails at least one of them.
"""
import math

import numpy as np
import pytest
import torch
import torch.nn.functional as F

import oracle
import workloads

BS = workloads.BLOCK_SIZE


# ----------------------------------------------------------------------------
# helpers (test side, independent of the oracle)
# ----------------------------------------------------------------------------
def unpage(cache, table, L):
    """Dense [H, L, D] float64 tensor of one sequence's cache rows."""
    j = torch.arange(L)
    phys = table[j // BS].long()
    slot = j % BS
    return cache[phys, :, slot, :].permute(1, 0, 2).double()


def window_mask(pos, L, window, causal):
    """Additive mask [len(pos), L]: 0 where key j is visible to position p."""
    p = torch.as_tensor(pos, dtype=torch.long)[:, None]
    j = torch.arange(L)[None, :]
    ok = torch.ones(p.shape[0], L, dtype=torch.bool)
    if causal:
        ok &= j <= p
    if window > 0:
        ok &= (p - j).abs() < window
    m = torch.zeros(ok.shape, dtype=torch.float64)
    m[~ok] = float("-inf")
    return m


def sdpa_decode(case):
    """Library cross-check of decode: SDPA(q, K, V, mask = scale*A + M)."""
    B, H, D = case.q.shape
    out = torch.zeros(B, H, D, dtype=torch.float64)
    for b in range(B):
        L = int(case.lens[b])
        if L == 0:
            continue
        K = unpage(case.k_cache, case.block_tables[b], L)
        V = unpage(case.v_cache, case.block_tables[b], L)
        M = window_mask([L - 1], L, case.sliding_window, False)          # [1, L]
        mask = M.expand(H, 1, L).clone()
        if case.attn_bias is not None:
            mask = mask + case.scale * case.attn_bias[b, :, :L].double()[:, None, :]
        qb = case.q[b].double()[:, None, :]                                  # [H,1,D]
        out[b] = F.scaled_dot_product_attention(qb, K, V, attn_mask=mask,
                                                scale=case.scale)[:, 0, :]
    return out.numpy()


def sdpa_prefill(case):
    TQ, H, D = case.q.shape
    out = torch.zeros(TQ, H, D, dtype=torch.float64)
    qsl = case.query_start_loc
    for b in range(case.num_seqs):
        L = int(case.lens[b])
        q0, q1 = int(qsl[b]), int(qsl[b + 1])
        nq = q1 - q0
        if nq == 0:
            continue
        pos = list(range(L - nq, L))
        K = unpage(case.k_cache, case.block_tables[b], L)
        V = unpage(case.v_cache, case.block_tables[b], L)
        M = window_mask(pos, L, case.sliding_window, case.causal)           # [nq, L]
        mask = M[None].expand(H, nq, L).clone()
        if case.attn_bias is not None:
            mask = mask + case.scale * case.attn_bias[b][:, pos, :L].double()
        qb = case.q[q0:q1].double().permute(1, 0, 2)                        # [H,nq,D]
        out[q0:q1] = F.scaled_dot_product_attention(qb, K, V, attn_mask=mask,
                                                    scale=case.scale).permute(1, 0, 2)
    return out.numpy()


def run_decode(case, bias="case", window=None):
    return oracle.decode(case.q, case.k_cache, case.v_cache, case.block_tables,
                         case.context_lens, case.attn_bias if bias == "case" else bias,
                         case.sliding_window if window is None else window, case.scale,
                         case.max_seq_len)


def run_prefill(case, bias="case", window=None):
    return oracle.prefill(case.q, case.k_cache, case.v_cache, case.block_tables,
                          case.context_lens, case.query_start_loc,
                          case.attn_bias if bias == "case" else bias,
                          case.sliding_window if window is None else window,
                          int(case.causal), case.scale, case.max_seq_len)


def small_decode(seed, dtype=torch.float32, bias="normal", window=-1, lens=(1, 40), H=3,
                 D=8, B=4, max_seq_len=48, scale=None):
    return workloads.decode_case(seed, num_seqs=B, num_heads=H, head_dim=D, lens=lens,
                                 max_seq_len=max_seq_len, dtype=dtype, bias=bias,
                                 sliding_window=window, scale=scale)


def small_prefill(seed, dtype=torch.float32, bias="normal", window=-1, causal=False,
                  lens=(1, 40), q_lens=None, H=2, D=8, B=3, max_seq_len=48, scale=None):
    return workloads.prefill_case(seed, num_seqs=B, num_heads=H, head_dim=D, lens=lens,
                                  max_seq_len=max_seq_len, dtype=dtype, bias=bias,
                                  sliding_window=window, causal=causal, q_lens=q_lens,
                                  scale=scale)


# ----------------------------------------------------------------------------
# library cross-check
# ----------------------------------------------------------------------------
@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
@pytest.mark.parametrize("bias", ["normal", None, "t5"])
@pytest.mark.parametrize("window", [-1, 1, 5, 16, 17, 100])
def test_decode_equals_sdpa(dtype, bias, window):
    case = small_decode(11 + window, dtype=dtype, bias=bias, window=window, lens=(1, 45),
                        scale=0.3)
    np.testing.assert_allclose(run_decode(case), sdpa_decode(case), rtol=0, atol=1e-12)


def test_decode_equals_sdpa_d64_fixed_pool():
    case = workloads.tiny_decode_f32()
    np.testing.assert_allclose(run_decode(case), sdpa_decode(case), rtol=0, atol=1e-12)


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("window", [-1, 1, 3, 16, 33])
@pytest.mark.parametrize("bias", ["normal", None])
def test_prefill_equals_sdpa(dtype, causal, window, bias):
    case = small_prefill(21 + window, dtype=dtype, bias=bias, window=window, causal=causal)
    np.testing.assert_allclose(run_prefill(case), sdpa_prefill(case), rtol=0, atol=1e-12)


@pytest.mark.parametrize("causal", [False, True])
def test_prefill_partial_queries_equals_sdpa(causal):
    # fewer queries than keys: they sit at the last n_q positions
    case = small_prefill(31, bias="normal", window=7, causal=causal, lens=[30, 17, 5],
                         q_lens=[4, 17, 1])
    np.testing.assert_allclose(run_prefill(case), sdpa_prefill(case), rtol=0, atol=1e-12)


def test_prefill_asymmetric_bias_index():
    # bias[b,h,i,j] with i = query position, j = key position: transposing it
    # must change the result (so the SDPA check above really pins the order)
    case = small_prefill(41, bias="normal", lens=[20, 9, 33])
    ref = run_prefill(case)
    tb = case.attn_bias.transpose(2, 3).contiguous()
    assert np.max(np.abs(run_prefill(case, bias=tb) - ref)) > 1e-3


# ----------------------------------------------------------------------------
# hand-worked closed forms
# ----------------------------------------------------------------------------
def hand_case(k_rows, v_rows, q, bias_row, scale, window=-1):
    """One sequence, one head, D=2, keys scattered over a 4-block pool in the
    order table = [2, 0, 3] (so logical block 0 is physical block 2)."""
    L = len(k_rows)
    table = np.array([[2, 0, 3]], np.int32)
    k = np.full((4, 1, BS, 2), np.nan, np.float32)
    v = np.full((4, 1, BS, 2), np.nan, np.float32)
    for j in range(L):
        k[table[0, j // BS], 0, j % BS] = k_rows[j]
        v[table[0, j // BS], 0, j % BS] = v_rows[j]
    bias = None
    if bias_row is not None:
        bias = np.full((1, 1, 48), np.nan, np.float32)
        bias[0, 0, :L] = bias_row
    return oracle.decode(np.array([[q]], np.float32), k, v, table,
                         np.array([L], np.int32), bias, window, scale, 48)[0, 0]


def test_hand_bias_added_before_scale():
    # Two keys with q.k = 0 for both, bias (0, 2), scale 1/2. Adding the bias
    # before the 1/sqrt(d_k) factor gives scores (0, 1): weights 1 : e.
    # (Adding it after would give (0, 2): weights 1 : e^2.)
    v0, v1 = np.array([1.0, -2.0]), np.array([3.0, 5.0])
    got = hand_case([[0, 1], [0, -1]], [v0, v1], [1, 0], [0.0, 2.0], 0.5)
    want = (v0 + math.e * v1) / (1 + math.e)
    np.testing.assert_allclose(got, want, rtol=0, atol=1e-15)


def test_hand_dot_product_and_gather():
    # 20 keys across two physical blocks (2 then 0). q = (1, 2), k_j = (j, -j)
    # so q.k_j = -j; the bias a_j = j cancels it exactly: all scores equal,
    # and the output is the plain mean of the values v_j = (j, j^2).
    L = 20
    k = [[j, -j] for j in range(L)]
    v = [[j, j * j] for j in range(L)]
    got = hand_case(k, v, [1, 2], [float(j) for j in range(L)], 0.7)
    want = np.array([np.mean(np.arange(L)), np.mean(np.arange(L) ** 2)])
    np.testing.assert_allclose(got, want, rtol=0, atol=1e-12)


def test_hand_window_keeps_last_w():
    # Same equal-score set-up with window 5: the decode query at position 19
    # sees keys 15..19 only, so the output is the mean of v_15..v_19.
    L = 20
    k = [[j, -j] for j in range(L)]
    v = [[j, j * j] for j in range(L)]
    got = hand_case(k, v, [1, 2], [float(j) for j in range(L)], 0.7, window=5)
    js = np.arange(15, 20)
    np.testing.assert_allclose(got, [js.mean(), (js ** 2).mean()], rtol=0, atol=1e-12)


def test_hand_sign_of_dot_product():
    # No bias, scale 1, keys k_0 = (0,0), k_1 = (1,0) and q = (ln 3, 0):
    # scores (0, ln 3): weights 1 : 3, out = (v0 + 3 v1) / 4.
    v0, v1 = np.array([4.0, 0.0]), np.array([0.0, 8.0])
    q = [np.float32(math.log(3.0)), 0.0]
    got = hand_case([[0, 0], [1, 0]], [v0, v1], q, None, 1.0)
    w1 = math.exp(float(np.float32(math.log(3.0))))
    np.testing.assert_allclose(got, (v0 + w1 * v1) / (1 + w1), rtol=0, atol=1e-15)


# ----------------------------------------------------------------------------
# special cases
# ----------------------------------------------------------------------------
def test_single_token_returns_its_value():
    case = small_decode(51, lens=[1, 1, 1, 1])
    out = run_decode(case)
    for b in range(4):
        v0 = case.v_cache[case.block_tables[b, 0].long(), :, 0, :].double().numpy()
        np.testing.assert_array_equal(out[b], v0)


def test_window_one_returns_newest_value():
    case = small_decode(52, window=1, lens=(2, 45))
    out = run_decode(case)
    for b in range(4):
        j = int(case.lens[b]) - 1
        vj = case.v_cache[case.block_tables[b, j // BS].long(), :, j % BS, :].double().numpy()
        np.testing.assert_array_equal(out[b], vj)


@pytest.mark.parametrize("causal", [False, True])
def test_prefill_window_one_returns_own_value(causal):
    case = small_prefill(53, window=1, causal=causal)
    out = run_prefill(case)
    for b in range(case.num_seqs):
        q0 = int(case.query_start_loc[b])
        for t in range(int(case.lens[b])):
            vt = case.v_cache[case.block_tables[b, t // BS].long(), :, t % BS, :]
            np.testing.assert_array_equal(out[q0 + t], vt.double().numpy())


def test_window_at_least_length_equals_no_window():
    case = small_decode(54, lens=(1, 40))
    ref = run_decode(case, window=-1)
    for w in (40, 41, 1000):
        np.testing.assert_array_equal(run_decode(case, window=w), ref)
    pc = small_prefill(55, lens=(1, 40), causal=False)
    pref = run_prefill(pc, window=-1)
    np.testing.assert_array_equal(run_prefill(pc, window=40), pref)


def test_null_bias_equals_zero_bias_bit_exact():
    case = small_decode(56, bias="zero")
    np.testing.assert_array_equal(run_decode(case, bias=None), run_decode(case))
    pc = small_prefill(57, bias=None)
    zero = torch.zeros(pc.num_seqs, pc.num_heads, pc.max_seq_len, pc.max_seq_len)
    np.testing.assert_array_equal(run_prefill(pc, bias=zero), run_prefill(pc))


def test_constant_bias_equals_no_bias():
    case = small_decode(58, bias=None)
    c = torch.full((4, 3, 48), 3.75)
    np.testing.assert_allclose(run_decode(case, bias=c), run_decode(case), rtol=0, atol=1e-12)


def test_zero_scale_is_the_mean_of_visible_values():
    # scale 0 makes every visible score 0 whatever q and the bias hold, so each
    # output is the plain average of the V rows the query may see
    case = small_decode(61, window=7, lens=(1, 40), scale=0.0)
    out = run_decode(case)
    for b in range(case.num_seqs):
        L = int(case.lens[b])
        V = unpage(case.v_cache, case.block_tables[b], L)              # [H, L, D]
        np.testing.assert_allclose(out[b], V[:, max(0, L - 7):L].mean(1).numpy(),
                                   rtol=0, atol=1e-12)
    pc = small_prefill(62, causal=True, window=5, scale=0.0)
    pout = run_prefill(pc)
    qsl = pc.query_start_loc
    for b in range(pc.num_seqs):
        L = int(pc.lens[b])
        V = unpage(pc.v_cache, pc.block_tables[b], L)
        for t in range(int(qsl[b + 1] - qsl[b])):
            p = L - int(qsl[b + 1] - qsl[b]) + t
            np.testing.assert_allclose(pout[int(qsl[b]) + t], V[:, max(0, p - 4):p + 1].mean(1),
                                       rtol=0, atol=1e-12)


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
def test_negative_scale(dtype):
    # a negative scale weights low scores most; (q, A, -s) and (-q, -A, s)
    # give every key the same score, so the two agree bit for bit, and both
    # match SDPA called with the negative scale
    case = small_decode(63, dtype=dtype, window=9, lens=(1, 45), scale=-0.3)
    out = run_decode(case)
    np.testing.assert_allclose(out, sdpa_decode(case), rtol=0, atol=1e-12)
    flipped = oracle.decode(-case.q, case.k_cache, case.v_cache, case.block_tables,
                            case.context_lens, -case.attn_bias, 9, -case.scale, case.max_seq_len)
    np.testing.assert_array_equal(out, flipped)
    pc = small_prefill(64, dtype=dtype, causal=True, window=6, scale=-0.3)
    pout = run_prefill(pc)
    np.testing.assert_allclose(pout, sdpa_prefill(pc), rtol=0, atol=1e-12)
    pflip = oracle.prefill(-pc.q, pc.k_cache, pc.v_cache, pc.block_tables, pc.context_lens,
                           pc.query_start_loc, -pc.attn_bias, 6, 1, -pc.scale, pc.max_seq_len)
    np.testing.assert_array_equal(pout, pflip)


def test_empty_and_fully_masked_rows_are_zero():
    case = small_decode(59, lens=[0, 5, 17, 3])
    bias = torch.zeros(4, 3, 48)
    bias[2] = float("-inf")         # every score of sequence 2 is -inf
    out = run_decode(case, bias=bias)
    assert np.all(out[0] == 0) and np.all(out[2] == 0)
    assert np.all(np.isfinite(out))


def test_block_relabelling_is_bit_exact():
    case = small_decode(60, lens=(10, 45))
    ref = run_decode(case)
    nb = case.num_blocks
    perm = torch.from_numpy(np.random.default_rng(7).permutation(nb))
    inv = torch.argsort(perm)
    # physical block p moves to slot inv[p]
    k2 = case.k_cache[perm]
    v2 = case.v_cache[perm]
    t2 = inv[case.block_tables.long()].int()
    out = oracle.decode(case.q, k2, v2, t2, case.context_lens, case.attn_bias, -1,
                        case.scale, case.max_seq_len)
    np.testing.assert_array_equal(out, ref)


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
def test_bias_probe_isolates_one_key(dtype):
    # bias -1e4 everywhere except 0 at one key j*: exp of the gap is exactly 0
    # in float64, so out = v_{j*} exactly.
    case = small_decode(61, dtype=dtype, bias=None, lens=[37, 37, 37, 37])
    for js in (0, 15, 16, 31, 36):
        bias = torch.full((4, 3, 48), -1e4)
        bias[:, :, js] = 0.0
        out = run_decode(case, bias=bias)
        for b in range(4):
            vj = case.v_cache[case.block_tables[b, js // BS].long(), :, js % BS, :]
            np.testing.assert_array_equal(out[b], vj.double().numpy())


def test_poisoned_slots_are_never_read():
    for seed in range(3):
        case = small_decode(70 + seed, lens=(1, 45), window=7)
        assert torch.isnan(case.k_cache).any()
        assert np.all(np.isfinite(run_decode(case)))
        pc = small_prefill(80 + seed, window=5)
        assert np.all(np.isfinite(run_prefill(pc)))


def test_oracle_rejects_bad_scalars():
    case = small_decode(90)
    with pytest.raises(ValueError):
        run_decode(case, window=0)
    with pytest.raises(ValueError):
        oracle.decode(case.q, case.k_cache, case.v_cache, case.block_tables,
                      case.context_lens, None, -1, 1.0, 8)       # L > max_seq_len


# ----------------------------------------------------------------------------
# T5 relative-position bias (in-oracle bucketing)
# ----------------------------------------------------------------------------
def test_t5_bucket_closed_forms_unidirectional():
    # 32 buckets, max distance 128, decoder: exact below 16; beyond, bucket
    # 16 + floor(16 * log(n/16) / log(8)). log(2)/log(8) = 1/3 and
    # log(4)/log(8) = 2/3 exactly, so n = 32 -> 16 + 5 and n = 64 -> 16 + 10.
    rp = -np.array([0, 1, 15, 16, 32, 64, 112, 113, 128, 1000])       # keys before the query
    want = [0, 1, 15, 16, 21, 26, 30, 31, 31, 31]
    assert oracle.t5_bucket(rp, 0, 32, 128).tolist() == want
    # keys after the query (never visible to a causal decoder) share bucket 0
    assert oracle.t5_bucket([1, 5, 500], 0, 32, 128).tolist() == [0, 0, 0]


def test_t5_bucket_closed_forms_bidirectional():
    # 16 buckets per side, exact below 8; log(n/8)/log(16) is 1/4, 1/2, 3/4, 1
    # for n = 16, 32, 64, 128: buckets 8 + 2, 8 + 4, 8 + 6, then the clamp 15.
    n = np.array([0, 7, 8, 16, 32, 64, 128, 5000])
    assert oracle.t5_bucket(-n, 1, 32, 128).tolist() == [0, 7, 8, 10, 12, 14, 15, 15]
    # keys after the query use the upper half, with the same spacing
    pos = n[n > 0]
    assert (oracle.t5_bucket(pos, 1, 32, 128) - oracle.t5_bucket(-pos, 1, 32, 128)
            == 16).all()


def test_t5_bucket_monotone_and_last_value_beyond_max_distance():
    d = np.arange(0, 3000)
    for bidir in (0, 1):
        b = oracle.t5_bucket(-d, bidir, 32, 128)
        assert np.all(np.diff(b) >= 0)
        assert np.all(b[128:] == b[128])
        assert b[128] == (15 if bidir else 31)


def test_t5_bucket_matches_input_generator():
    # the generator's numpy bucketing (used to materialise T5 biases) and the
    # oracle's C bucketing are written independently; they must agree
    d = np.arange(0, 5000)
    assert np.array_equal(oracle.t5_bucket(-d, 0, 32, 128), workloads.t5_bucket(d))


def test_decode_relpos_equals_materialised_bias_bit_exact():
    case = workloads.decode_case(91, num_seqs=5, num_heads=3, head_dim=16, lens=(1, 200),
                                 max_seq_len=208, dtype=torch.bfloat16, bias="t5")
    dense = run_decode(case)
    inline = oracle.decode_relpos(case.q, case.k_cache, case.v_cache, case.block_tables,
                                  case.context_lens, case.t5_table, 32, 128, 0, -1,
                                  case.scale, case.max_seq_len)
    np.testing.assert_array_equal(inline, dense)


@pytest.mark.parametrize("bidir", [0, 1])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("window", [-1, 9])
def test_prefill_relpos_equals_sdpa(bidir, causal, window):
    case = small_prefill(92 + bidir, bias=None, window=window, causal=causal,
                         lens=[40, 150, 7], max_seq_len=160)
    tab = torch.randn(case.num_heads, 32, generator=torch.Generator().manual_seed(5)) * 0.5
    got = oracle.prefill_relpos(case.q, case.k_cache, case.v_cache, case.block_tables,
                                case.context_lens, case.query_start_loc, tab, 32, 128, bidir,
                                window, int(causal), case.scale, case.max_seq_len)
    # dense bias built from the bucket map, checked through SDPA
    pos = np.arange(case.max_seq_len)
    buckets = oracle.t5_bucket(pos[None, :] - pos[:, None], bidir, 32, 128)   # [p, j]
    dense = tab[:, torch.from_numpy(buckets.astype(np.int64))]                 # [H, MS, MS]
    case.attn_bias = dense[None].expand(case.num_seqs, -1, -1, -1).contiguous()
    np.testing.assert_allclose(got, sdpa_prefill(case), rtol=0, atol=1e-12)


# ----------------------------------------------------------------------------
# KV-cache write (scatter through the slot mapping)
# ----------------------------------------------------------------------------
@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
def test_kv_write_reads_back_through_the_table(dtype):
    g = torch.Generator().manual_seed(3)
    nb, H, D, T = 9, 3, 8, 40
    k = torch.randn(nb, H, BS, D, generator=g).to(dtype)
    v = torch.randn(nb, H, BS, D, generator=g).to(dtype)
    kn = torch.randn(T, H, D, generator=g).to(dtype)
    vn = torch.randn(T, H, D, generator=g).to(dtype)
    table = torch.tensor([6, 2, 8], dtype=torch.int32)          # logical blocks of one sequence
    slots = (table[torch.arange(T) // BS].long() * BS + torch.arange(T) % BS)
    slots[[3, 17]] = -1                                         # skipped tokens
    kc, vc = oracle.kv_write(k, v, kn, vn, slots)
    kc, vc = torch.from_numpy(kc), torch.from_numpy(vc)
    if dtype == torch.bfloat16:
        kc, vc = kc.view(torch.bfloat16), vc.view(torch.bfloat16)
    got_k = unpage(kc, table, T).permute(1, 0, 2)              # [T, H, D]
    got_v = unpage(vc, table, T).permute(1, 0, 2)
    keep = slots >= 0
    assert torch.equal(got_k[keep], kn[keep].double())
    assert torch.equal(got_v[keep], vn[keep].double())
    # skipped tokens and untouched blocks keep their old contents
    old_k = unpage(k, table, T).permute(1, 0, 2)
    assert torch.equal(got_k[~keep], old_k[~keep])
    for blk in set(range(nb)) - {6, 2, 8}:
        assert torch.equal(kc[blk], k[blk]) and torch.equal(vc[blk], v[blk])


def test_kv_write_rejects_slots_outside_the_pool():
    k = torch.zeros(2, 1, BS, 4)
    with pytest.raises(ValueError):
        oracle.kv_write(k, k, torch.zeros(1, 1, 4), torch.zeros(1, 1, 4),
                        torch.tensor([2 * BS], dtype=torch.int64))


# ----------------------------------------------------------------------------
# ragged bias layout
# ----------------------------------------------------------------------------
def pack_decode_bias(dense, lens):
    """[B,H,MS] padded -> packed [H][L_b] rows per sequence + start offsets."""
    parts, starts, off = [], [], 0
    for b, L in enumerate(lens):
        parts.append(dense[b, :, :int(L)].reshape(-1))
        starts.append(off)
        off += dense.shape[1] * int(L)
    return torch.cat(parts).contiguous(), torch.tensor(starts, dtype=torch.int64)


def pack_prefill_bias(dense, lens, q_lens):
    parts, starts, off = [], [], 0
    for b, (L, nq) in enumerate(zip(lens, q_lens)):
        L, nq = int(L), int(nq)
        parts.append(dense[b, :, L - nq:L, :L].reshape(-1))
        starts.append(off)
        off += dense.shape[1] * nq * L
    return torch.cat(parts).contiguous(), torch.tensor(starts, dtype=torch.int64)


@pytest.mark.parametrize("window", [-1, 7])
def test_decode_ragged_equals_padded_bit_exact(window):
    case = small_decode(95, bias="normal", window=window, lens=[0, 1, 30, 45], max_seq_len=48)
    packed, starts = pack_decode_bias(case.attn_bias, case.lens)
    assert packed.numel() == case.num_heads * int(case.lens.sum())
    got = oracle.decode_ragged(case.q, case.k_cache, case.v_cache, case.block_tables,
                               case.context_lens, packed, starts, window, case.scale,
                               case.max_seq_len)
    np.testing.assert_array_equal(got, run_decode(case))


@pytest.mark.parametrize("causal", [False, True])
def test_prefill_ragged_equals_padded_bit_exact(causal):
    case = small_prefill(96, bias="normal", window=9, causal=causal, lens=[40, 17, 5],
                         q_lens=[40, 3, 5])
    packed, starts = pack_prefill_bias(case.attn_bias, case.lens, case.q_lens)
    got = oracle.prefill_ragged(case.q, case.k_cache, case.v_cache, case.block_tables,
                                case.context_lens, case.query_start_loc, packed, starts, 9,
                                int(causal), case.scale, case.max_seq_len)
    np.testing.assert_array_equal(got, run_prefill(case))


def test_thread_count_does_not_change_results():
    # the CPU baseline times the oracle at its default thread count and on one
    # thread; every row is computed the same way either way
    case = small_decode(61, lens=(10, 90), B=16, max_seq_len=96)
    ref = run_decode(case)
    n = oracle.num_threads()
    oracle.set_num_threads(1)
    try:
        assert oracle.num_threads() == 1
        one = run_decode(case)
    finally:
        oracle.set_num_threads(n)
    assert oracle.num_threads() == n
    np.testing.assert_array_equal(one, ref)


# ----------------------------------------------------------------------------
# chunked local attention ("[V1] Add sliding window support to Flex Attention
# backend", attention-groups thread: Llama 4's chunked-local layers). Reading:
# a query sees the keys of its own chunk of chunk_size positions (causal: up to
# itself). The pins tie the oracle to that reading, not the reading to a page.
# ----------------------------------------------------------------------------
def chunk_mask(pos, L, chunk, causal):
    """Additive mask [len(pos), L]: a block-diagonal matrix of all-ones chunks
    (torch.block_diag), optionally intersected with the lower triangle."""
    sizes = [min(chunk, L - s) for s in range(0, L, chunk)]
    ok = torch.block_diag(*[torch.ones(n, n) for n in sizes]).bool()
    if causal:
        ok &= torch.tril(torch.ones(L, L, dtype=torch.bool))
    ok = ok[torch.as_tensor(pos, dtype=torch.long)]
    m = torch.zeros(ok.shape, dtype=torch.float64)
    m[~ok] = float("-inf")
    return m


def sdpa_rows(case, b, pos, mask, bias_rows):
    H = case.q.shape[1]
    L = int(case.lens[b])
    K = unpage(case.k_cache, case.block_tables[b], L)
    V = unpage(case.v_cache, case.block_tables[b], L)
    m = mask[None].expand(H, len(pos), L).clone()
    if bias_rows is not None:
        m = m + case.scale * bias_rows
    return K, V, m


def sdpa_decode_chunked(case, chunk):
    B, H, D = case.q.shape
    out = torch.zeros(B, H, D, dtype=torch.float64)
    for b in range(B):
        L = int(case.lens[b])
        if L == 0:
            continue
        bias = None if case.attn_bias is None else case.attn_bias[b, :, :L].double()[:, None, :]
        K, V, m = sdpa_rows(case, b, [L - 1], chunk_mask([L - 1], L, chunk, False), bias)
        out[b] = F.scaled_dot_product_attention(case.q[b].double()[:, None, :], K, V,
                                                attn_mask=m, scale=case.scale)[:, 0, :]
    return out.numpy()


def sdpa_prefill_chunked(case, chunk):
    TQ, H, D = case.q.shape
    out = torch.zeros(TQ, H, D, dtype=torch.float64)
    qsl = case.query_start_loc
    for b in range(case.num_seqs):
        L = int(case.lens[b])
        q0, q1 = int(qsl[b]), int(qsl[b + 1])
        if q1 == q0:
            continue
        pos = list(range(L - (q1 - q0), L))
        bias = None if case.attn_bias is None else case.attn_bias[b][:, pos, :L].double()
        K, V, m = sdpa_rows(case, b, pos, chunk_mask(pos, L, chunk, case.causal), bias)
        qb = case.q[q0:q1].double().permute(1, 0, 2)
        out[q0:q1] = F.scaled_dot_product_attention(qb, K, V, attn_mask=m,
                                                    scale=case.scale).permute(1, 0, 2)
    return out.numpy()


def run_decode_chunked(case, chunk, bias="case"):
    return oracle.decode_chunked(case.q, case.k_cache, case.v_cache, case.block_tables,
                                 case.context_lens, case.attn_bias if bias == "case" else bias,
                                 chunk, case.scale, case.max_seq_len)


def run_prefill_chunked(case, chunk, bias="case"):
    return oracle.prefill_chunked(case.q, case.k_cache, case.v_cache, case.block_tables,
                                  case.context_lens, case.query_start_loc,
                                  case.attn_bias if bias == "case" else bias, chunk,
                                  int(case.causal), case.scale, case.max_seq_len)


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
@pytest.mark.parametrize("bias", ["normal", None])
@pytest.mark.parametrize("chunk", [1, 5, 16, 17, 64])
def test_decode_chunked_equals_sdpa(dtype, bias, chunk):
    case = small_decode(2100 + chunk, dtype=dtype, bias=bias, B=6)
    np.testing.assert_allclose(run_decode_chunked(case, chunk), sdpa_decode_chunked(case, chunk),
                               rtol=0, atol=1e-12)


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("chunk", [1, 3, 8, 16, 33])
@pytest.mark.parametrize("partial", [False, True])
def test_prefill_chunked_equals_sdpa(dtype, causal, chunk, partial):
    case = small_prefill(2200 + chunk, dtype=dtype, causal=causal,
                         lens=[5, 21, 40] if partial else (1, 40),
                         q_lens=[1, 7, 20] if partial else None)
    np.testing.assert_allclose(run_prefill_chunked(case, chunk),
                               sdpa_prefill_chunked(case, chunk), rtol=0, atol=1e-12)


def test_chunk_covering_the_sequence_equals_full_attention_bit_exact():
    d = small_decode(2300)
    assert np.array_equal(run_decode_chunked(d, 1000), run_decode(d, window=-1))
    for causal in (False, True):
        p = small_prefill(2301, causal=causal)
        assert np.array_equal(run_prefill_chunked(p, 1000), run_prefill(p, window=-1))


def test_chunk_one_returns_own_value():
    """A chunk of one position holds only the query's own key: out = v_p
    exactly, whatever the bias and scale."""
    d = small_decode(2310, lens=(1, 40))
    out = run_decode_chunked(d, 1)
    for b in range(d.q.shape[0]):
        L = int(d.lens[b])
        v = unpage(d.v_cache, d.block_tables[b], L)[:, L - 1, :]
        assert np.array_equal(out[b], v.numpy())
    p = small_prefill(2311)
    outp = run_prefill_chunked(p, 1)
    for b in range(p.num_seqs):
        L = int(p.lens[b])
        q0 = int(p.query_start_loc[b])
        v = unpage(p.v_cache, p.block_tables[b], L)
        for t in range(L):
            assert np.array_equal(outp[q0 + t], v[:, t, :].numpy())


@pytest.mark.parametrize("chunk", [3, 16, 21])
def test_decode_chunked_equals_window_over_the_chunks_tail_bit_exact(chunk):
    """The decode query sits at L-1, so its chunk's visible keys are the last
    ((L-1) mod C) + 1 tokens: the same key set, in the same order, as a window
    of that size."""
    case = small_decode(2320 + chunk, B=6)
    out = run_decode_chunked(case, chunk)
    for b in range(6):
        L = int(case.lens[b])
        w = (L - 1) % chunk + 1
        assert np.array_equal(out[b], run_decode(case, window=w)[b])


def test_oracle_rejects_non_positive_chunks():
    d = small_decode(2330)
    p = small_prefill(2331)
    for c in (0, -1):
        with pytest.raises(ValueError):
            run_decode_chunked(d, c)
        with pytest.raises(ValueError):
            run_prefill_chunked(p, c)
