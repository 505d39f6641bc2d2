"""Host-side arithmetic of bench.py, checked on the CPU.

The roofline fields of the benchmark lines rest on two counts: the algorithmic
bytes of a decode call and the algorithmic flops of a prefill layer. Both are
compared here with brute-force counts over every (sequence, head, key) or
(sequence, head, query, key) of small cases, using the visibility rules of the
decode (the W newest tokens), of bidirectional prefill (|i - j| < W) and of
causal prefill (j <= i). The counter-summary reader must hand out a value only
for the kernel source it was measured on.
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


def brute_prefill_flops(lens, H, D, window, chunk=0, causal=False):
    pairs = 0
    for L in lens:
        for i in range(L):
            for j in range(L):
                if causal and j > i:
                    continue
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


def test_causal_prefill_flops_match_brute_force():
    lens = np.array([1, 2, 3, 16, 29, 64, 70, 130], dtype=np.int32)
    got = bench.prefill_flops(lens, 2, 64, -1, causal=True)
    assert got == brute_prefill_flops(lens.tolist(), 2, 64, -1, causal=True)
    # about half the bidirectional pairs, plus the diagonal
    assert 2 * got - bench.prefill_flops(lens, 2, 64, -1) == 4 * 64 * 2 * int(lens.sum())


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
    for wl, key in (("large_biased_decode_bf16", "hbm_bytes_per_launch"),
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


def test_prefill_bytes_count_each_token_once():
    lens = np.array([1, 16, 17, 300], dtype=np.int32)
    # q, K, V read and out written once per token, head and dim
    assert bench.prefill_bytes(lens, 12, 64, 4) == 4 * 334 * 12 * 64 * 4
    assert bench.prefill_bytes(lens, 12, 64, 2) == 4 * 334 * 12 * 64 * 2


TRACE_HDR = ["Kind", "Dispatch_Id", "Kernel_Name", "Start_Timestamp", "End_Timestamp"]
CTR_HDR = ["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value"]
K_FULL = "void pa::(anonymous namespace)::pa_prefill_f32<64, 1, 0, false, 0>(pa::PrefillArgs)"
K_WIN = "void pa::(anonymous namespace)::pa_prefill_f32<64, 1, 0, false, 1>(pa::PrefillArgs)"
K_TORCH = "void at::native::vectorized_elementwise_kernel<4, at::native::FillFunctor<float> >"


def _write_csv(path, hdr, rows):
    import csv
    with open(path, "w", newline="") as f:
        w = csv.writer(f)
        w.writerow(hdr)
        w.writerows(rows)


def _fake_run(tmp_path):
    """A fake profile of 5 steps of (full, window) launches after 3 warm-up
    steps, torch kernels in between; the timed full launches take 10 us, the
    window ones 4 us, warm-up launches 99 us."""
    rows, d, t = [], 1, 0
    for step in range(8):
        timed = step >= 3
        for k, us in ((K_FULL, 10), (K_WIN, 4)):
            dur = (us if timed else 99) * 1000
            rows.append(["KERNEL_DISPATCH", d, k, t, t + dur])
            d, t = d + 1, t + dur + 500
        rows.append(["KERNEL_DISPATCH", d, K_TORCH, t, t + 7000])
        d, t = d + 1, t + 8000
    _write_csv(tmp_path / "run_kernel_trace.csv", TRACE_HDR, rows)
    return rows


def test_trace_table_keeps_only_the_timed_dispatches(tmp_path):
    _fake_run(tmp_path)
    per = bench.trace_table(str(tmp_path / "run_kernel_trace.csv"), 10)
    assert sorted(per) == sorted([K_FULL, K_WIN])
    assert per[K_FULL] == [10.0] * 5 and per[K_WIN] == [4.0] * 5


def test_write_profiles_round_trip(tmp_path, monkeypatch):
    """Trace and counter summaries written from fake rocprofv3 output are read
    back by read_traffic, and their numbers are the timed launches' ones."""
    import json
    monkeypatch.setattr(bench, "PROFILES", str(tmp_path))
    _fake_run(tmp_path)
    line = {"steps": 5, "launches_per_step": 2, "ms_per_step": 0.015,
            "roofline": {"frac": 0.5}, "algorithmic_bytes_per_step": 1000 * 1024}
    (tmp_path / "line.json").write_text(json.dumps(line) + "\n")
    for ctr, full, win in (("FETCH_SIZE", 600.0, 300.0), ("WRITE_SIZE", 200.0, 100.0)):
        rows = []
        for d in range(1, 9):           # 3 warm-up + 5 timed dispatches of each kernel
            rows.append([2 * d - 1, K_FULL, ctr, full if d > 3 else 1e9])
            rows.append([2 * d, K_WIN, ctr, win if d > 3 else 1e9])
        os.makedirs(tmp_path / ctr, exist_ok=True)
        _write_csv(tmp_path / ctr / "run_counter_collection.csv", CTR_HDR, rows)
        os.makedirs(tmp_path / ("copy_" + ctr), exist_ok=True)
        _write_csv(tmp_path / ("copy_" + ctr) / "run_counter_collection.csv", CTR_HDR,
                   [[1, "void at::native::direct_copy_kernel", ctr,
                     131072.0 if ctr == "FETCH_SIZE" else 262144.0]])
    args = bench.argparse.Namespace(
        write_profiles="modernbert_prefill_f32", bench_line=str(tmp_path / "line.json"),
        trace=str(tmp_path), fetch=str(tmp_path / "FETCH_SIZE"),
        write=str(tmp_path / "WRITE_SIZE"), copy_fetch=str(tmp_path / "copy_FETCH_SIZE"),
        copy_write=str(tmp_path / "copy_WRITE_SIZE"), counter_line=str(tmp_path / "line.json"),
        command="python bench.py ...", counter_commands=["a", "b"])
    bench.write_profiles(args)
    md = (tmp_path / "modernbert_prefill_f32_kernel_trace.md").read_text()
    assert "| 5 | 10.0 | 10.0 | 10.0 |" in md and "| 5 | 4.0 | 4.0 | 4.0 |" in md
    # per step: fetch (600 + 300) KiB x 2 (calibration) + write (200 + 100) KiB
    want = (900 * 2 + 300) * 1024
    src = bench.KERNEL_SOURCE["modernbert_prefill_f32"]
    assert bench.read_traffic("modernbert_prefill_f32", src, "hbm_bytes_per_step") == want
    assert bench.read_traffic("modernbert_prefill_f32", src) == want / 2
    # the summary is tied to every source the workload's kernels come from
    assert bench.read_traffic("modernbert_prefill_f32", "pa_prefill.hip") is None


def test_kernel_tag():
    assert bench.kernel_tag(K_WIN) == "pa_prefill_f32_64_1_0_false_1"
    assert bench.kernel_tag("void pa::(anonymous namespace)::pa_kv_write<256>(pa::KvWriteArgs)") \
        == "pa_kv_write_256"


def test_probe_library_exports_its_entry_points():
    # bench_probes.so (built by __graft_entry__.build()) backs the probe_*
    # workloads; every entry point bench.py binds must be exported
    import ctypes
    path = os.path.join(ROOT, "bench_probes.so")
    if not os.path.exists(path):
        pytest.skip("bench_probes.so not built")
    lib = ctypes.CDLL(path)
    for name in ("pb_mfma", "pb_lds", "pb_stream", "pb_gather", "pb_bias", "pb_mix",
                 "pb_valu", "pb_clock"):
        assert hasattr(lib, name), name


def test_kernel_source_of_window_tags():
    # counter summaries of single layers are named <workload>_w<W>
    assert bench.kernel_source_of("prefill_layer_f32_w64") == bench.KERNEL_SOURCE[
        "prefill_layer_f32"]
    assert bench.kernel_source_of("prefill_layer_bf16_wfull") == "pa_prefill_bf16.hip"
    assert bench.kernel_source_of("modernbert_prefill_bf16") == "pa_prefill_bf16.hip"
    assert bench.kernel_source_of("prefill_layer_bf16_causal") == "pa_prefill_bf16.hip"
