"""CPU check of the poisoned-bias inputs the GPU bias-contract test uses: the
oracle reads only the bias entries of visible keys, so NaN in every other
in-range entry leaves its result unchanged, bit for bit. This also pins the
test's poison mask: a mask that hit a visible entry would give NaN here."""
import numpy as np
import pytest
import torch

import oracle
from bias_poison import pack, poisoned_case


@pytest.mark.parametrize("window,chunk,causal,partial", [
    (-1, 0, False, True), (-1, 0, True, True), (5, 0, False, False), (17, 0, True, True),
    (-1, 16, True, True), (-1, 33, False, False)])
def test_poisoned_bias_is_never_read_by_the_oracle(window, chunk, causal, partial):
    clean = poisoned_case(950, torch.float32, 8, window, chunk, causal, partial, poison=False)
    bad = poisoned_case(950, torch.float32, 8, window, chunk, causal, partial)
    assert torch.isnan(bad.attn_bias).sum() > torch.isnan(clean.attn_bias).sum()

    def run(c):
        if chunk > 0:
            return oracle.prefill_chunked(c.q, c.k_cache, c.v_cache, c.block_tables,
                                          c.context_lens, c.query_start_loc, c.attn_bias, chunk,
                                          int(causal), c.scale, c.max_seq_len)
        return oracle.prefill(c.q, c.k_cache, c.v_cache, c.block_tables, c.context_lens,
                              c.query_start_loc, c.attn_bias, window, int(causal), c.scale,
                              c.max_seq_len)

    ref, got = run(clean), run(bad)
    assert np.all(np.isfinite(got))
    assert np.array_equal(ref, got)
    if chunk == 0:
        packed, starts = pack(bad.attn_bias, bad.lens, bad.q_lens)
        rag = oracle.prefill_ragged(bad.q, bad.k_cache, bad.v_cache, bad.block_tables,
                                    bad.context_lens, bad.query_start_loc, packed, starts,
                                    window, int(causal), bad.scale, bad.max_seq_len)
        assert np.array_equal(ref, rag)
