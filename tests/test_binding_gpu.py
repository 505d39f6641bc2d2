"""The binding's argument checks on device tensors: wrong dtypes, shapes,
strides, devices and mismatched caches are rejected before the library is
called (so no kernel is launched with them)."""
import pytest
import torch

import sliding_window_mask_amd as pa

pytestmark = pytest.mark.gpu
DEV = "cuda"


def args(dtype=torch.bfloat16, B=2, H=4, D=64, msl=64):
    q = torch.zeros(B, H, D, dtype=dtype, device=DEV)
    k = torch.zeros(8, H, 16, D, dtype=dtype, device=DEV)
    v = torch.zeros_like(k)
    bt = torch.zeros(B, msl // 16, dtype=torch.int32, device=DEV)
    cl = torch.ones(B, dtype=torch.int32, device=DEV)
    bias = torch.zeros(B, H, msl, device=DEV)
    return q, k, v, bt, cl, bias


def decode(q, k, v, bt, cl, bias, **kw):
    return pa.paged_attn_decode(q, k, v, bt, cl, bias, -1, 0.125, max_seq_len=64, **kw)


def test_valid_call_passes_the_checks():
    out = decode(*args())
    torch.cuda.synchronize()
    assert out.shape == (2, 4, 64)


@pytest.mark.parametrize("case,exc,match", [
    ("q_f16", TypeError, "q must be"),
    ("k_dtype", TypeError, "k_cache must be"),
    ("v_shape", ValueError, "v_cache must have shape"),
    ("k_headdim", ValueError, "k_cache must have shape"),
    ("q_strided", ValueError, "q must be contiguous"),
    ("bt_int64", TypeError, "block_tables must be"),
    ("cl_rows", ValueError, "context_lens must have shape"),
    ("bias_f64", TypeError, "attn_bias must be"),
    ("bias_bf16", TypeError, "attn_bias must be"),
    ("bias_shape", ValueError, "attn_bias must have shape"),
    ("bias_host", ValueError, "attn_bias must be a tensor on"),
    ("out_dtype", TypeError, "out must be"),
])
def test_decode_rejects(case, exc, match):
    q, k, v, bt, cl, bias = args()
    kw = {}
    if case == "q_f16":
        q = q.half()
    elif case == "k_dtype":
        k = k.float()
    elif case == "v_shape":
        v = torch.zeros(9, 4, 16, 64, dtype=k.dtype, device=DEV)
    elif case == "k_headdim":
        k = torch.zeros(8, 4, 16, 128, dtype=q.dtype, device=DEV)
        v = torch.zeros_like(k)
    elif case == "q_strided":
        q = torch.zeros(2, 64, 4, dtype=q.dtype, device=DEV).transpose(1, 2)
    elif case == "bt_int64":
        bt = bt.long()
    elif case == "cl_rows":
        cl = torch.ones(3, dtype=torch.int32, device=DEV)
    elif case == "bias_f64":
        bias = bias.double()
    elif case == "bias_bf16":
        bias = bias.bfloat16()
    elif case == "bias_shape":
        bias = torch.zeros(2, 4, 32, device=DEV)
    elif case == "bias_host":
        bias = bias.cpu()
    elif case == "out_dtype":
        kw["out"] = torch.zeros(2, 4, 64, device=DEV)
    with pytest.raises(exc, match=match):
        decode(q, k, v, bt, cl, bias, **kw)


def test_prefill_and_cache_reject():
    q, k, v, bt, cl, _ = args()
    qp = torch.zeros(2, 4, 64, dtype=q.dtype, device=DEV)
    with pytest.raises(ValueError, match="query_start_loc must have shape"):
        pa.paged_attn_prefill(qp, k, v, bt, cl, torch.zeros(2, dtype=torch.int32, device=DEV),
                              None, -1, False, 0.125, max_seq_len=64)
    with pytest.raises(ValueError, match="attn_bias must have shape"):
        pa.paged_attn_prefill(qp, k, v, bt, cl, torch.tensor([0, 1, 2], dtype=torch.int32,
                                                             device=DEV),
                              torch.zeros(2, 4, 64, device=DEV), -1, False, 0.125,
                              max_seq_len=64)
    with pytest.raises(TypeError, match="slot_mapping must be"):
        pa.paged_kv_write(k, v, qp, qp, torch.zeros(2, dtype=torch.int32, device=DEV))
    with pytest.raises(TypeError, match="v_new must be"):
        pa.paged_kv_write(k, v, qp, qp.float(), torch.zeros(2, dtype=torch.int64, device=DEV))
