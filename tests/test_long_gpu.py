"""GPU parity at the largest sizes the kernels plan for: prefill contexts of
up to 4096 keys (64 query tiles, hundreds of key tiles, the last queries of a
long prompt as well as a whole 2049-token sequence), and decode contexts
longer than the longest partition (4096 tokens), run both with the library's
default plan and with 4096-token partitions, so that the merge kernel
combines full-length partitions. Both dtypes, both head dims."""
import pytest
import torch

import workloads
from gpu_helpers import (assert_close, gpu_decode, gpu_prefill, log, oracle_decode,
                         oracle_prefill, to_device)

pytestmark = pytest.mark.gpu
DTYPES = [torch.float32, torch.bfloat16]


@pytest.mark.parametrize("dtype", DTYPES)
@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("causal,window", [(False, -1), (True, -1), (False, 512), (True, 300)])
def test_prefill_long_contexts(dtype, D, causal, window):
    log("long prefill dtype=%s D=%d causal=%s W=%d" % (dtype, D, causal, window))
    lens = [4096, 2049, 1500]
    q_lens = [64, 2049, 100]
    case = to_device(workloads.prefill_case(1400 + D + window, num_seqs=3, num_heads=2,
                                            head_dim=D, lens=lens, max_seq_len=4096, dtype=dtype,
                                            bias=None, sliding_window=window, causal=causal,
                                            q_lens=q_lens))
    assert_close(gpu_prefill(case), oracle_prefill(case), dtype,
                 "long prefill D=%d causal=%s W=%d" % (D, causal, window))


@pytest.mark.parametrize("dtype", DTYPES)
@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("window", [-1, 5000])
def test_decode_beyond_one_partition(dtype, D, window):
    log("long decode dtype=%s D=%d W=%d" % (dtype, D, window))
    lens = [8192, 4097, 4096, 4095, 1, 6000]
    case = to_device(workloads.decode_case(1410 + D, num_seqs=len(lens), num_heads=2,
                                           head_dim=D, lens=lens, max_seq_len=8192,
                                           dtype=dtype, bias="normal", sliding_window=window))
    ref = oracle_decode(case)
    for p in (0, 4096):
        assert_close(gpu_decode(case, partition=p), ref, dtype,
                     "long decode D=%d W=%d P=%d" % (D, window, p))
