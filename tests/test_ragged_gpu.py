"""GPU parity of the ragged (packed, unpadded) bias layout against the
float64 oracle, and bit-identity with the padded layout holding the same
values."""
import numpy as np
import pytest
import torch

import oracle
import workloads
from gpu_helpers import assert_close, gpu_decode, gpu_prefill, to_device, to_host

import sliding_window_mask_amd as pa

pytestmark = pytest.mark.gpu
DEV = "cuda"


def pack_decode(dense, lens):
    parts, starts, off = [], [], 0
    for b, L in enumerate(lens):
        parts.append(dense[b, :, :int(L)].reshape(-1))
        starts.append(off)
        off += dense.shape[1] * int(L)
    return torch.cat(parts).contiguous(), torch.tensor(starts, dtype=torch.int64)


def pack_prefill(dense, lens, q_lens):
    parts, starts, off = [], [], 0
    for b, (L, nq) in enumerate(zip(lens, q_lens)):
        L, nq = int(L), int(nq)
        parts.append(dense[b, :, L - nq:L, :L].reshape(-1))
        starts.append(off)
        off += dense.shape[1] * nq * L
    return torch.cat(parts).contiguous(), torch.tensor(starts, dtype=torch.int64)


@pytest.mark.parametrize("dtype,D", [(torch.bfloat16, 128), (torch.float32, 64)])
@pytest.mark.parametrize("window,partition", [(-1, 0), (-1, 64), (100, 0)])
def test_decode_ragged(dtype, D, window, partition):
    case = to_device(workloads.decode_case(800 + D, num_seqs=7, num_heads=4, head_dim=D,
                                           lens=(0, 700), max_seq_len=720, dtype=dtype,
                                           bias="normal", sliding_window=window))
    packed, starts = pack_decode(case.attn_bias.cpu(), case.lens)
    packed, starts = packed.to(DEV), starts.to(DEV)
    out = pa.paged_attn_decode_ragged_bias(case.q, case.k_cache, case.v_cache, case.block_tables,
                                           case.context_lens, packed, starts, window, case.scale,
                                           max_seq_len=case.max_seq_len,
                                           partition_tokens=partition)
    torch.cuda.synchronize()
    h = to_host(case)
    ref = oracle.decode_ragged(h.q, h.k_cache, h.v_cache, h.block_tables, h.context_lens,
                               packed.cpu(), starts.cpu(), window, h.scale, h.max_seq_len)
    assert_close(out, ref, dtype, "ragged decode")
    padded = gpu_decode(case, partition=partition)
    assert torch.equal(out.view(torch.int16), padded.view(torch.int16))


@pytest.mark.parametrize("causal,window", [(False, -1), (True, -1), (False, 33)])
def test_prefill_ragged(causal, window):
    case = to_device(workloads.prefill_case(810, num_seqs=4, num_heads=3, head_dim=64,
                                            lens=[9, 130, 64, 200], q_lens=[9, 70, 1, 200],
                                            max_seq_len=208, dtype=torch.float32,
                                            bias="normal", sliding_window=window,
                                            causal=causal))
    packed, starts = pack_prefill(case.attn_bias.cpu(), case.lens, case.q_lens)
    packed, starts = packed.to(DEV), starts.to(DEV)
    out = pa.paged_attn_prefill_ragged_bias(case.q, case.k_cache, case.v_cache,
                                            case.block_tables, case.context_lens,
                                            case.query_start_loc, packed, starts, window, causal,
                                            case.scale, max_seq_len=case.max_seq_len)
    torch.cuda.synchronize()
    h = to_host(case)
    ref = oracle.prefill_ragged(h.q, h.k_cache, h.v_cache, h.block_tables, h.context_lens,
                                h.query_start_loc, packed.cpu(), starts.cpu(), window,
                                int(causal), h.scale, h.max_seq_len)
    assert_close(out, ref, torch.float32, "ragged prefill")
    assert torch.equal(out, gpu_prefill(case))
