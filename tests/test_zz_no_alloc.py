"""paged_attn_decode_noalloc: the decode entry point for callers that cannot
allocate device memory. Its split-K partials live in the library's fixed
per-GPU scratch array; results must equal paged_attn_decode with a
caller-allocated workspace, call after call (the second call smaller than the
first, reusing the array), and match the float64 oracle. Shapes whose
partials would not fit the array are refused on the host."""
import ctypes

import numpy as np
import pytest
import torch

import workloads
from gpu_helpers import assert_close, log, oracle_decode, to_device

import sliding_window_mask_amd as pa

SCRATCH_BYTES = 16 << 20
FAKE = 1 << 20        # 256-byte aligned, never dereferenced (host rejections only)


def test_noalloc_refuses_shapes_beyond_its_scratch():
    """A shape whose split-K partials exceed the scratch array is refused
    before any HIP call (PA_ERR_WORKSPACE), and bad arguments are refused as
    by paged_attn_decode."""
    lib = pa.lib()
    need = lib.pa_decode_workspace_bytes(256, 32, 128, 4096, -1, 16, 1)
    assert need > SCRATCH_BYTES
    st = lib._lib.paged_attn_decode_noalloc(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None, -1, 0.1,
                                            256, 32, 32, 128, 16, 256, 4096, 50000, 1, 16, None)
    assert st == 5, lib.pa_last_error()
    assert "scratch" in lib.pa_last_error()
    st = lib._lib.paged_attn_decode_noalloc(FAKE, None, FAKE, FAKE, FAKE, FAKE, None, -1, 0.1,
                                            4, 4, 4, 64, 16, 8, 128, 64, 0, 0, None)
    assert st == 1                                       # NULL q
    st = lib._lib.paged_attn_decode_noalloc(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None, 0, 0.1,
                                            4, 4, 4, 64, 16, 8, 128, 64, 0, 0, None)
    assert st == 2                                       # window 0
    assert lib._lib.paged_attn_decode_noalloc(None, None, None, None, None, None, None, -1, 0.1,
                                              0, 4, 4, 64, 16, 8, 128, 64, 0, 0, None) == 0


CASES = [
    # (seed, B, H, D, dtype, lens, max_seq_len, window, bias, partition)
    (1500, 48, 8, 128, torch.bfloat16, (1, 3000), 3072, -1, "normal", 256),
    (1501, 5, 4, 64, torch.float32, (0, 300), 320, 100, "normal", 64),
]


@pytest.mark.gpu
def test_noalloc_matches_decode_with_workspace_call_after_call():
    lib = pa.lib()
    for (seed, B, H, D, dtype, lens, msl, window, bias, part) in CASES:
        case = to_device(workloads.decode_case(seed, num_seqs=B, num_heads=H, head_dim=D,
                                               lens=lens, max_seq_len=msl, dtype=dtype,
                                               bias=bias, sliding_window=window))
        need = lib.pa_decode_workspace_bytes(B, H, D, msl, window, part,
                                             pa._dtype_code(case.q))
        log("noalloc B=%d H=%d D=%d %s W=%d partition=%d: %d bytes of partials"
            % (B, H, D, dtype, window, part, need))
        assert 0 < need <= SCRATCH_BYTES
        out = torch.full_like(case.q, float("nan"))
        lib.paged_attn_decode_noalloc(case.q, case.k_cache, case.v_cache, case.block_tables,
                                      case.context_lens, case.attn_bias, window, case.scale,
                                      max_seq_len=msl, out=out, partition_tokens=part)
        torch.cuda.synchronize()
        ws = torch.empty(need, dtype=torch.uint8, device="cuda")
        ref_out = lib.paged_attn_decode(case.q, case.k_cache, case.v_cache, case.block_tables,
                                        case.context_lens, case.attn_bias, window, case.scale,
                                        max_seq_len=msl, workspace=ws, partition_tokens=part)
        torch.cuda.synchronize()
        bits = torch.int16 if dtype == torch.bfloat16 else torch.int32
        assert torch.equal(out.view(bits), ref_out.view(bits))
        assert_close(out, oracle_decode(case), dtype, "noalloc seed %d" % seed)
