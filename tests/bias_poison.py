"""Bias inputs for the prefill bias-contract tests: a materialised bias whose
every in-range entry that no query may read is NaN (keys outside the window,
past the causal diagonal or outside the query's chunk, and the rows of
positions that are not queried). Input synthesis only; the visibility rule
here is the test's own statement of the documented one."""
import numpy as np
import torch

import workloads

LENS = [1, 15, 16, 17, 40, 63, 64, 65, 130, 200]
PARTIAL_Q = [1, 15, 3, 17, 1, 20, 64, 2, 100, 131]


def readable(L, nq, msl, window, chunk, causal):
    """[msl, msl] bool: entry (query position p, key j) may be read, i.e. p is
    one of the n_q queried positions and j is visible to it."""
    pos = np.arange(msl)
    p, j = pos[:, None], pos[None, :]
    ok = (p >= L - nq) & (p < L) & (j < L)
    if causal:
        ok &= j <= p
    if window > 0:
        ok &= np.abs(p - j) < window
    if chunk > 0:
        ok &= (j // chunk) == (p // chunk)
    return ok


def poisoned_case(seed, dtype, D, window, chunk, causal, partial, poison=True):
    q_lens = PARTIAL_Q if partial else None
    case = workloads.prefill_case(seed, num_seqs=len(LENS), num_heads=2, head_dim=D,
                                  lens=LENS, q_lens=q_lens, max_seq_len=208, dtype=dtype,
                                  bias="normal", sliding_window=window, causal=causal)
    bias = case.attn_bias
    for b in range(len(LENS) if poison else 0):
        L, nq = case.lens[b], case.q_lens[b]
        bad = ~readable(int(L), int(nq), case.max_seq_len, window, chunk, causal)
        bias[b, :, torch.from_numpy(bad)] = float("nan")
    return case


def pack(dense, lens, q_lens):
    parts, starts, off = [], [], 0
    for b, (L, nq) in enumerate(zip(lens, q_lens)):
        L, nq = int(L), int(nq)
        parts.append(dense[b, :, L - nq:L, :L].reshape(-1))
        starts.append(off)
        off += dense.shape[1] * nq * L
    return torch.cat(parts).contiguous(), torch.tensor(starts, dtype=torch.int64)
