"""GPU tests of the KV-cache write (paged_kv_write) against the float64
oracle's scatter, and a decode loop that writes every new token through the
kernel, decodes with a sliding window, and frees + reuses the blocks that
fall behind the window (pa_window_first_live_block)."""
import numpy as np
import pytest
import torch

import oracle
from gpu_helpers import BS, TOL, log, max_err

import sliding_window_mask_amd as pa

pytestmark = pytest.mark.gpu
DEV = "cuda"


def as_dtype(a, dtype):
    t = torch.from_numpy(a)
    return t.view(torch.bfloat16) if dtype == torch.bfloat16 else t


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
@pytest.mark.parametrize("D", [64, 128])
def test_kv_write_matches_oracle(dtype, D):
    g = torch.Generator().manual_seed(D)
    nb, H, T = 50, 4, 300
    k = torch.randn(nb, H, BS, D, generator=g).to(dtype)
    v = torch.randn(nb, H, BS, D, generator=g).to(dtype)
    kn = torch.randn(T, H, D, generator=g).to(dtype)
    vn = torch.randn(T, H, D, generator=g).to(dtype)
    slots = torch.randperm(nb * BS, generator=g)[:T].long()
    slots[::7] = -1
    kd, vd = k.to(DEV), v.to(DEV)
    pa.paged_kv_write(kd, vd, kn.to(DEV), vn.to(DEV), slots.to(DEV))
    torch.cuda.synchronize()
    rk, rv = oracle.kv_write(k, v, kn, vn, slots)
    assert torch.equal(kd.cpu(), as_dtype(rk, dtype))
    assert torch.equal(vd.cpu(), as_dtype(rv, dtype))


@pytest.mark.parametrize("dtype,D", [(torch.bfloat16, 128), (torch.float32, 64)])
def test_decode_loop_with_window_eviction_and_reuse(dtype, D):
    """Every step appends one token per sequence through paged_kv_write and
    decodes with window W; blocks before pa_window_first_live_block are
    returned to the pool, NaN-poisoned and handed to other sequences, while
    their stale table entries stay in place."""
    W, H, B, pool, steps = 24, 2, 3, 48, 70
    g = torch.Generator().manual_seed(11)
    kc = torch.full((pool, H, BS, D), float("nan"), dtype=dtype, device=DEV)
    vc = torch.full((pool, H, BS, D), float("nan"), dtype=dtype, device=DEV)
    free = list(range(pool))
    max_blocks = 16
    table = torch.zeros(B, max_blocks, dtype=torch.int32)
    lens = [5, 17, 40]
    live_from = [0] * B
    scale = 1.0 / np.sqrt(D)

    def alloc(b, n):
        table[b, n] = free.pop(0)

    def write(b, positions):
        for pos in positions:
            if pos % BS == 0:
                alloc(b, pos // BS)
        slots = torch.tensor([int(table[b, p // BS]) * BS + p % BS for p in positions],
                             dtype=torch.int64, device=DEV)
        kn = torch.randn(len(positions), H, D, generator=g).to(dtype).to(DEV)
        vn = torch.randn(len(positions), H, D, generator=g).to(dtype).to(DEV)
        pa.paged_kv_write(kc, vc, kn, vn, slots)

    for b in range(B):
        write(b, list(range(lens[b])))
    worst = 0.0
    for step in range(steps):
        for b in range(B):
            write(b, [lens[b]])
            lens[b] += 1
        q = torch.randn(B, H, D, generator=g).to(dtype).to(DEV)
        cl = torch.tensor(lens, dtype=torch.int32, device=DEV)
        bt = table.to(DEV)
        out = pa.paged_attn_decode(q, kc, vc, bt, cl, None, W, scale,
                                   max_seq_len=max_blocks * BS)
        torch.cuda.synchronize()
        ref = oracle.decode(q.cpu(), kc.cpu(), vc.cpu(), table, cl.cpu(), None, W, scale,
                            max_blocks * BS)
        err = max_err(out, ref)
        worst = max(worst, err)
        assert err <= TOL[dtype], (step, err)
        # free the blocks no later step can read; poison them before reuse
        for b in range(B):
            first = pa.pa_window_first_live_block(lens[b], W)
            for n in range(live_from[b], first):
                blk = int(table[b, n])
                kc[blk] = float("nan")
                vc[blk] = float("nan")
                free.append(blk)
            live_from[b] = max(live_from[b], first)
    log("  decode loop worst max|err| = %.3e over %d steps" % (worst, steps))
    assert max(lens) > 100 and len(free) < pool
