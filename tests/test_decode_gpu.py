"""GPU parity of paged_attn_decode (through the C ABI) against the float64
oracle: the four decode workloads, edge cases, and the exactness properties
(bit-exact gathering, null == zero bias, relabelling, determinism)."""
import numpy as np
import pytest
import torch

import workloads
from gpu_helpers import (BS, TOL, assert_close, gpu_decode, log, max_err, oracle_decode,
                         sample_decode, to_device)

pytestmark = pytest.mark.gpu

DEV = "cuda"


def small(seed, dtype=torch.float32, D=64, H=3, B=5, lens=(1, 80), msl=96, bias="normal",
          window=-1, **kw):
    return workloads.decode_case(seed, num_seqs=B, num_heads=H, head_dim=D, lens=lens,
                                 max_seq_len=msl, dtype=dtype, bias=bias,
                                 sliding_window=window, **kw)


# ---------------------------------------------------------------------------
# the named decode workloads
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("bias", ["normal", None])
def test_tiny_decode_f32(bias):
    log("tiny_decode_f32 bias=%s" % bias)
    case = to_device(workloads.tiny_decode_f32(bias=bias))
    assert_close(gpu_decode(case), oracle_decode(case), torch.float32, "tiny")


def test_tiny_decode_null_bias_matches_oracle_without_bias():
    case = to_device(workloads.tiny_decode_f32())
    assert_close(gpu_decode(case, bias=None), oracle_decode(case, bias=None), torch.float32,
                 "tiny null")


def test_t5_small_self_decode_bf16():
    log("t5_small_self_decode_bf16")
    case = to_device(workloads.t5_small_self_decode_bf16())
    assert_close(gpu_decode(case), oracle_decode(case), torch.bfloat16, "t5-small")


def test_t5_large_cross_decode_null_equals_zero_bias():
    log("t5_large_cross_decode_bf16")
    case = to_device(workloads.t5_large_cross_decode_bf16(bias="zero"))
    out_zero = gpu_decode(case)
    out_null = gpu_decode(case, bias=None)
    assert torch.equal(out_zero.view(torch.int16), out_null.view(torch.int16))
    assert_close(out_null, oracle_decode(case, bias=None), torch.bfloat16, "t5-large cross")


@pytest.mark.parametrize("window,evict", [(-1, False), (1024, True)])
def test_large_biased_decode_sampled(window, evict):
    """Full-size run (256 x 32 heads, L up to 4096, default launch
    configuration) checked on 40 sequences the oracle computes: the longest,
    the shortest, the first and last, and 36 more spread over the batch."""
    log("large_biased_decode_bf16 window=%d evict=%s" % (window, evict))
    case = workloads.large_biased_decode_bf16(device=DEV, sliding_window=window, evict=evict)
    out = gpu_decode(case)
    L = case.lens
    spread = np.linspace(1, 254, 36).astype(int).tolist()
    seqs = sorted(set([int(np.argmax(L)), int(np.argmin(L)), 0, 255] + spread))
    assert len(seqs) >= 32
    sub = sample_decode(case, seqs)
    ref = oracle_decode(sub)
    assert_close(out[torch.tensor(seqs, device=DEV)], ref, torch.bfloat16, "large sample")
    assert torch.isfinite(out.float()).all()
    del case, out
    torch.cuda.empty_cache()


# ---------------------------------------------------------------------------
# shapes, windows and partitions
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("window", [-1, 1, 7, 16, 33, 200])
def test_small_shapes(dtype, D, window):
    case = to_device(small(100 + D + window, dtype=dtype, D=D, window=window, lens=(1, 300),
                           msl=320, B=6))
    ref = oracle_decode(case)
    assert_close(gpu_decode(case), ref, dtype, "D=%d W=%d" % (D, window))


@pytest.mark.parametrize("partition", [16, 32, 48, 64, 128, 256, 4096])
@pytest.mark.parametrize("window", [-1, 40])
def test_partition_sweep(partition, window):
    case = to_device(small(200, dtype=torch.bfloat16, D=128, window=window, lens=(1, 700),
                           msl=720, B=7, H=2))
    ref = oracle_decode(case)
    out = gpu_decode(case, partition=partition)
    assert_close(out, ref, torch.bfloat16, "P=%d W=%d" % (partition, window))


def test_split_equals_single_partition_within_tolerance():
    case = to_device(small(201, dtype=torch.float32, lens=(100, 500), msl=512, B=4))
    one = gpu_decode(case, partition=512)
    for p in (16, 64, 176):
        assert max_err(gpu_decode(case, partition=p), one.double().cpu().numpy()) <= 1e-5


@pytest.mark.parametrize("L", [0, 1, 2, 15, 16, 17, 31, 32, 33, 255, 256, 257])
def test_edge_lengths(L):
    case = to_device(small(300 + L, dtype=torch.float32, lens=[L, 1, L, 17], B=4, msl=272))
    ref = oracle_decode(case)
    out = gpu_decode(case)
    assert_close(out, ref, torch.float32, "L=%d" % L)
    if L == 0:
        assert torch.all(out[0] == 0)
    out2 = gpu_decode(case, partition=16)
    assert_close(out2, ref, torch.float32, "L=%d P=16" % L)


def test_window_edge_cases():
    case = to_device(small(310, dtype=torch.float32, lens=[1, 16, 17, 50, 64, 65], B=6,
                           msl=80))
    for w in (1, 2, 15, 16, 17, 49, 50, 51, 64, 65, 1000):
        assert_close(gpu_decode(case, window=w), oracle_decode(case, window=w), torch.float32,
                     "W=%d" % w)


def test_window_one_returns_newest_value_exactly():
    case = to_device(small(320, dtype=torch.bfloat16, lens=(1, 90)))
    out = gpu_decode(case, window=1).cpu()
    for b in range(case.q.shape[0]):
        j = int(case.lens[b]) - 1
        v = case.v_cache[case.block_tables[b, j // BS].long(), :, j % BS, :].cpu()
        assert torch.equal(out[b].view(torch.int16), v.view(torch.int16))


def test_window_at_least_length_equals_no_window_bit_exact():
    case = to_device(small(321, dtype=torch.bfloat16, lens=(1, 90)))
    ref = gpu_decode(case, window=-1)
    for w in (90, 96, 5000):
        assert torch.equal(gpu_decode(case, window=w).view(torch.int16), ref.view(torch.int16))


def test_evicted_blocks_are_never_touched():
    # blocks wholly before the window are NaN and unmapped: output stays finite
    for dtype in (torch.float32, torch.bfloat16):
        case = to_device(small(330, dtype=dtype, D=128, lens=(100, 600), msl=640, B=5,
                               window=48, evict_before=48))
        assert_close(gpu_decode(case), oracle_decode(case), dtype, "evicted")


def test_scale_one():
    case = to_device(small(340, dtype=torch.float32, scale=1.0, lens=(1, 60), msl=64))
    assert_close(gpu_decode(case), oracle_decode(case), torch.float32, "scale=1")


# ---------------------------------------------------------------------------
# exactness properties
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
def test_null_bias_equals_zero_bias_bit_exact(dtype):
    case = to_device(small(400, dtype=dtype, bias="zero", lens=(1, 300), msl=320))
    for p in (0, 32):
        a = gpu_decode(case, partition=p)
        b = gpu_decode(case, bias=None, partition=p)
        assert torch.equal(a.view(torch.int16), b.view(torch.int16))


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
def test_gather_probe_bit_exact(dtype):
    """bias -1e4 except 0 at one key j*: every other weight is exactly 0 in
    fp32, so the output must be v_{j*} bit for bit (any wrong block or slot
    in the gather shows)."""
    case = to_device(small(410, dtype=dtype, D=64, bias=None, lens=[70, 70, 70, 70], B=4,
                           msl=80))
    for js in (0, 1, 15, 16, 17, 31, 32, 47, 48, 63, 64, 69):
        bias = torch.full((4, 3, 80), -1e4, device=DEV)
        bias[:, :, js] = 0.0
        for p in (0, 16):
            out = gpu_decode(case, bias=bias, partition=p).cpu()
            for b in range(4):
                v = case.v_cache[case.block_tables[b, js // BS].long(), :, js % BS, :].cpu()
                assert torch.equal(out[b].float(), v.float()), (js, b, p)


def test_block_relabelling_bit_identical():
    case = to_device(small(420, dtype=torch.bfloat16, lens=(10, 90)))
    ref = gpu_decode(case)
    perm = torch.from_numpy(np.random.default_rng(3).permutation(case.num_blocks)).to(DEV)
    inv = torch.argsort(perm)
    case.k_cache = case.k_cache[perm].contiguous()
    case.v_cache = case.v_cache[perm].contiguous()
    case.block_tables = inv[case.block_tables.long()].int().contiguous()
    assert torch.equal(gpu_decode(case).view(torch.int16), ref.view(torch.int16))


def test_run_to_run_deterministic():
    case = to_device(small(430, dtype=torch.bfloat16, D=128, lens=(200, 700), msl=720))
    a = gpu_decode(case, partition=64)
    for _ in range(3):
        assert torch.equal(gpu_decode(case, partition=64).view(torch.int16),
                           a.view(torch.int16))


def test_fully_masked_rows_are_zero():
    case = to_device(small(440, dtype=torch.float32, lens=[30, 40, 50], B=3, bias="zero",
                           msl=64))
    bias = case.attn_bias.clone()
    bias[1] = float("-inf")
    for p in (0, 16):
        out = gpu_decode(case, bias=bias, partition=p)
        assert torch.all(out[1] == 0)
        assert_close(out, oracle_decode(case, bias=bias), torch.float32, "masked P=%d" % p)


def test_constant_bias_shift_invariance():
    case = to_device(small(450, dtype=torch.float32, bias="zero", lens=(1, 60), msl=64))
    base = gpu_decode(case, bias=None)
    shifted = gpu_decode(case, bias=torch.full_like(case.attn_bias, 2.5))
    assert max_err(shifted, base.double().cpu().numpy()) <= 1e-5


def test_output_dtype_and_rounding():
    # bf16 output is the round-to-nearest-even of the fp32 result: check the
    # bf16 result is within half an ulp (+ the fp32 tolerance) of the oracle
    case = to_device(small(460, dtype=torch.bfloat16, lens=(1, 60), msl=64))
    out = gpu_decode(case)
    assert out.dtype == torch.bfloat16
    ref = oracle_decode(case)
    g = out.float().cpu().double().numpy()
    ulp = np.exp2(np.floor(np.log2(np.maximum(np.abs(ref), 1e-30))) - 7)
    assert np.all(np.abs(g - ref) <= 0.5 * ulp + 1e-4)
