"""GPU parity at the largest batch and head counts the C ABI accepts.

paged_attn_decode and paged_attn_prefill take up to 65535 sequences and 65535
heads (larger values are rejected on the host, see test_abi.py). Decode puts
the sequence on the grid's z dimension, whose hardware limit is 65535, and
prefill numbers (sequence, head) pairs on a one-dimensional grid; these cases
run both at the limit, with short contexts so the float64 oracle checks every
output row."""
import pytest
import torch

import workloads
from gpu_helpers import (assert_close, gpu_decode, gpu_prefill, log, oracle_decode,
                         oracle_prefill, to_device)

pytestmark = pytest.mark.gpu

MAX = 65535


@pytest.mark.parametrize("dtype,D,H,window", [(torch.float32, 64, 1, -1),
                                              (torch.bfloat16, 128, 2, 7)])
def test_decode_max_batch(dtype, D, H, window):
    log("decode max batch: B=%d H=%d D=%d %s W=%d" % (MAX, H, D, dtype, window))
    case = to_device(workloads.decode_case(960 + D, num_seqs=MAX, num_heads=H, head_dim=D,
                                           lens=(1, 40), max_seq_len=48, dtype=dtype,
                                           bias="normal", sliding_window=window))
    assert_close(gpu_decode(case), oracle_decode(case), dtype,
                 "decode B=%d H=%d D=%d W=%d" % (MAX, H, D, window))


def test_decode_max_heads():
    log("decode max heads: B=2 H=%d D=64 fp32" % MAX)
    case = to_device(workloads.decode_case(970, num_seqs=2, num_heads=MAX, head_dim=64,
                                           lens=[17, 3], max_seq_len=32, dtype=torch.float32,
                                           bias="normal"))
    assert_close(gpu_decode(case), oracle_decode(case), torch.float32, "decode H=%d" % MAX)


@pytest.mark.parametrize("window,causal", [(-1, False), (5, False), (-1, True)])
def test_prefill_max_batch(window, causal):
    log("prefill max batch: B=%d H=1 D=64 fp32 W=%d causal=%s" % (MAX, window, causal))
    case = to_device(workloads.prefill_case(980, num_seqs=MAX, num_heads=1, head_dim=64,
                                            lens=(1, 20), max_seq_len=32, dtype=torch.float32,
                                            sliding_window=window, causal=causal))
    assert_close(gpu_prefill(case), oracle_prefill(case), torch.float32,
                 "prefill B=%d W=%d causal=%s" % (MAX, window, causal))


def test_prefill_max_heads():
    log("prefill max heads: B=1 H=%d D=64 bf16" % MAX)
    case = to_device(workloads.prefill_case(990, num_seqs=1, num_heads=MAX, head_dim=64,
                                            lens=[17], max_seq_len=32, dtype=torch.bfloat16))
    assert_close(gpu_prefill(case), oracle_prefill(case), torch.bfloat16,
                 "prefill H=%d" % MAX)
