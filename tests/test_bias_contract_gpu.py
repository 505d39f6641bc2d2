"""The bias contract of the prefill entry points: a bias entry whose key the
query cannot see is never read.

Every in-range entry of the materialised bias that no query may read (keys
outside the window, past the causal diagonal or outside the query's chunk,
and whole rows of positions that are not queried) is NaN-filled here; entries
past a sequence's length are NaN already. The outputs must be finite and
match the float64 oracle, which itself reads only visible entries (so a mask
below that poisoned a visible entry would show as a NaN oracle result).
Padded and ragged layouts, fp32 and bf16 (both bf16 kernels: bidirectional
launches without a window, and causal ones without a window at head_dim 64,
take the 32-query-per-wave one)."""
import numpy as np
import pytest
import torch

import oracle
from bias_poison import pack, poisoned_case
from gpu_helpers import assert_close, log, to_device, to_host

import sliding_window_mask_amd as pa

pytestmark = pytest.mark.gpu
DEV = "cuda"

MASKS = [  # (window, chunk, causal, partial query sets)
    (-1, 0, False, False), (-1, 0, False, True), (-1, 0, True, False), (-1, 0, True, True),
    (1, 0, False, False), (5, 0, False, True), (16, 0, False, False), (17, 0, True, True),
    (64, 0, False, False), (-1, 8, False, False), (-1, 16, True, True), (-1, 33, False, True),
]


@pytest.mark.parametrize("dtype,D", [(torch.float32, 64), (torch.float32, 128),
                                     (torch.bfloat16, 64), (torch.bfloat16, 128)])
@pytest.mark.parametrize("window,chunk,causal,partial", MASKS)
@pytest.mark.parametrize("layout", ["padded", "ragged"])
def test_invisible_bias_entries_never_read(dtype, D, window, chunk, causal, partial, layout):
    if layout == "ragged" and chunk > 0:
        pytest.skip("the chunked entry points take the padded layout only")
    host = poisoned_case(900 + D + max(window, 0) + chunk, dtype, D, window, chunk, causal,
                         partial)
    case = to_device(host)
    what = "%s D=%d W=%d C=%d causal=%s partial=%s %s" % (dtype, D, window, chunk, causal,
                                                         partial, layout)
    log("bias contract " + what)
    h = to_host(case)
    if layout == "ragged":
        packed, starts = pack(host.attn_bias, host.lens, host.q_lens)
        out = pa.paged_attn_prefill_ragged_bias(
            case.q, case.k_cache, case.v_cache, case.block_tables, case.context_lens,
            case.query_start_loc, packed.to(DEV), starts.to(DEV), window, causal, case.scale,
            max_seq_len=case.max_seq_len)
        ref = oracle.prefill_ragged(h.q, h.k_cache, h.v_cache, h.block_tables, h.context_lens,
                                    h.query_start_loc, packed, starts, window, int(causal),
                                    h.scale, h.max_seq_len)
    elif chunk > 0:
        out = pa.paged_attn_prefill_chunked(
            case.q, case.k_cache, case.v_cache, case.block_tables, case.context_lens,
            case.query_start_loc, case.attn_bias, chunk, causal, case.scale,
            max_seq_len=case.max_seq_len)
        ref = oracle.prefill_chunked(h.q, h.k_cache, h.v_cache, h.block_tables,
                                     h.context_lens, h.query_start_loc, h.attn_bias, chunk,
                                     int(causal), h.scale, h.max_seq_len)
    else:
        out = pa.paged_attn_prefill(
            case.q, case.k_cache, case.v_cache, case.block_tables, case.context_lens,
            case.query_start_loc, case.attn_bias, window, causal, case.scale,
            max_seq_len=case.max_seq_len)
        ref = oracle.prefill(h.q, h.k_cache, h.v_cache, h.block_tables, h.context_lens,
                             h.query_start_loc, h.attn_bias, window, int(causal), h.scale,
                             h.max_seq_len)
    torch.cuda.synchronize()
    assert np.all(np.isfinite(ref)), "the poison mask hit a visible entry"
    assert_close(out, ref, dtype, what)
