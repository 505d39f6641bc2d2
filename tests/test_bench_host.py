"""Host-side arithmetic of bench.py, checked on the CPU.

The roofline fields of the benchmark lines rest on two counts: the algorithmic
bytes of a decode call and the algorithmic flops of a prefill layer. Both are
compared here with brute-force counts over every (sequence, head, key) or
(sequence, head, query, key) of small cases, using the visibility rules of the
decode (the W newest tokens) and of bidirectional prefill (|i - j| < W). The
counter-summary reader must hand out a value only for the kernel source it was
measured on.
"""
import os
import subprocess
import sys

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402


def brute_decode_bytes(lens, H, D, esize, window, with_bias, chunk=0):
    total = 0
    for L in lens:
        for _ in range(H):
            i = L - 1                       # the query sits at the newest token
            total += 2 * D * esize          # q read + out write
            for j in range(L):
                if window > 0 and not (0 <= i - j < window):
                    continue
                if chunk > 0 and j // chunk != i // chunk:
                    continue
                total += 2 * D * esize + (4 if with_bias else 0)
    return total


def brute_prefill_flops(lens, H, D, window, chunk=0):
    pairs = 0
    for L in lens:
        for i in range(L):
            for j in range(L):
                if window > 0 and abs(i - j) >= window:
                    continue
                if chunk > 0 and i // chunk != j // chunk:
                    continue
                pairs += 1
    return 4 * D * H * pairs                # q.k and p.v: 2 flops per MAC each


@pytest.mark.parametrize("window", [-1, 1, 5, 16, 40])
@pytest.mark.parametrize("with_bias", [False, True])
@pytest.mark.parametrize("esize", [2, 4])
def test_decode_bytes_match_brute_force(window, with_bias, esize):
    lens = np.array([1, 2, 15, 16, 17, 33, 40], dtype=np.int32)
    got = bench.decode_bytes(lens, 3, 64, esize, window, with_bias)
    assert got == brute_decode_bytes(lens.tolist(), 3, 64, esize, window, with_bias)


@pytest.mark.parametrize("chunk", [1, 5, 16, 40])
def test_chunked_decode_bytes_match_brute_force(chunk):
    lens = np.array([1, 2, 15, 16, 17, 33, 40, 81], dtype=np.int32)
    got = bench.decode_bytes(lens, 3, 64, 2, -1, True, chunk=chunk)
    assert got == brute_decode_bytes(lens.tolist(), 3, 64, 2, -1, True, chunk=chunk)


@pytest.mark.parametrize("window", [-1, 1, 2, 7, 30, 64])
def test_prefill_flops_match_brute_force(window):
    lens = np.array([1, 3, 16, 29, 64, 70], dtype=np.int32)
    got = bench.prefill_flops(lens, 2, 64, window)
    assert got == brute_prefill_flops(lens.tolist(), 2, 64, window)


@pytest.mark.parametrize("chunk", [1, 7, 16, 64, 128])
def test_chunked_prefill_flops_match_brute_force(chunk):
    lens = np.array([1, 3, 16, 29, 64, 70, 130], dtype=np.int32)
    got = bench.prefill_flops(lens, 2, 64, -1, chunk=chunk)
    assert got == brute_prefill_flops(lens.tolist(), 2, 64, -1, chunk=chunk)


def test_read_traffic_requires_the_measured_source(tmp_path, monkeypatch):
    sha = bench.source_sha("pa_prefill.hip")
    (tmp_path / "w_traffic.txt").write_text(
        "# comment = ignored\nkernel_source_sha = %s\nhbm_bytes_per_step = 123\n"
        "hbm_bytes_per_launch = 45\n" % sha)
    (tmp_path / "stale_traffic.txt").write_text(
        "kernel_source_sha = 0000000000000000\nhbm_bytes_per_launch = 45\n")
    monkeypatch.setattr(bench, "PROFILES", str(tmp_path))
    assert bench.read_traffic("w", "pa_prefill.hip") == 45.0
    assert bench.read_traffic("w", "pa_prefill.hip", "hbm_bytes_per_step") == 123.0
    assert bench.read_traffic("w", "pa_decode.hip") is None          # other source
    assert bench.read_traffic("stale", "pa_prefill.hip") is None     # stale hash
    assert bench.read_traffic("missing", "pa_prefill.hip") is None


def test_committed_traffic_summaries_parse():
    """The committed counter summaries hold the keys the bench lines read."""
    for wl, key in (("decode_large_biased_bf16", "hbm_bytes_per_launch"),
                    ("modernbert_prefill_f32", "hbm_bytes_per_step"),
                    ("modernbert_prefill_bf16", "hbm_bytes_per_step"),
                    ("t5_small_self_decode_bf16", "hbm_bytes_per_launch"),
                    ("t5_large_cross_decode_bf16", "hbm_bytes_per_launch"),
                    ("kv_write_modernbert_f32", "hbm_bytes_per_launch")):
        kv = {}
        for ln in open(os.path.join(ROOT, "profiles", "%s_traffic.txt" % wl)):
            if "=" in ln and not ln.startswith("#"):
                k, v = ln.split("=", 1)
                kv[k.strip()] = v.strip()
        assert float(kv[key]) > 0
        assert float(kv["ratio_hbm_to_algorithmic"]) >= 1.0
        assert len(kv["kernel_source_sha"]) == 16


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=300)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
