"""Host code under AddressSanitizer and UndefinedBehaviorSanitizer, on the CPU.

1. The oracle (oracle.c) is built with gcc -fsanitize=address,undefined and
   its pins run against that build (PA_ORACLE_LIB) in a subprocess with the
   sanitizer runtime preloaded; any sanitizer report fails the test.
2. The host side of the C ABI (pa_api.cpp: argument validation, workspace
   planning, metadata checks, the no-allocation scratch lookup) is built with
   the sanitizers on its host code only, next to stub kernel launchers (no GPU
   is used: every launch would report an error), and the ABI tests run against
   it (PA_LIB) the same way.
"""
import glob
import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
SAN_ENV = {"ASAN_OPTIONS": "detect_leaks=0:halt_on_error=1",
           "UBSAN_OPTIONS": "halt_on_error=1:print_stacktrace=1"}


def gcc_runtime(name):
    return subprocess.run(["gcc", "-print-file-name=%s" % name], capture_output=True,
                          text=True).stdout.strip()


def run_tests(tests, env_extra):
    env = dict(os.environ, **SAN_ENV, **env_extra)
    r = subprocess.run([sys.executable, "-m", "pytest"] + tests +
                       ["-x", "-q", "-s", "-m", "not gpu", "-p", "no:cacheprovider"],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=900)
    out = r.stdout + r.stderr
    assert "runtime error" not in out and "AddressSanitizer" not in out, out[-4000:]
    assert r.returncode == 0, out[-4000:]
    return out


def test_oracle_pins_under_asan_and_ubsan(tmp_path):
    so = tmp_path / "liboracle_san.so"
    subprocess.run(["gcc", "-O1", "-g", "-fno-omit-frame-pointer", "-fopenmp", "-fPIC",
                    "-shared", "-std=c11", "-fsanitize=address,undefined",
                    "-fno-sanitize-recover=all", "-o", str(so),
                    os.path.join(ROOT, "oracle", "oracle.c"), "-lm"], check=True)
    # libstdc++ is preloaded too: torch throws C++ exceptions, and the
    # sanitizer's interceptor needs the real __cxa_throw at start-up
    pre = "%s:%s" % (gcc_runtime("libasan.so"), gcc_runtime("libstdc++.so"))
    out = run_tests(["tests/test_oracle_pins.py", "tests/test_oracle_bias_reads.py"],
                    {"PA_ORACLE_LIB": str(so), "LD_PRELOAD": pre})
    assert " passed" in out


def test_abi_host_code_under_asan_and_ubsan(tmp_path):
    rt = sorted(glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"))
    if not os.path.exists(HIPCC) or not rt:
        pytest.skip("hipcc or the clang sanitizer runtime is not installed")
    so = tmp_path / "libpaged_attn_host_san.so"
    csrc = os.path.join(ROOT, "sliding_window_mask_amd", "csrc")
    # the sanitizers instrument the host code only (-Xarch_host before each)
    cmd = [HIPCC, "--offload-arch=gfx950", "-O1", "-g", "-fno-omit-frame-pointer",
           "-std=c++17", "-fPIC", "-shared",
           "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
           "-Xarch_host", "-fno-sanitize-recover=all",
           "-I", os.path.join(ROOT, "include"), "-I", csrc, "-o", str(so),
           os.path.join(csrc, "pa_api.cpp"),
           os.path.join(ROOT, "tests", "sanitize", "launch_stubs.cpp")]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stdout + r.stderr
    out = run_tests(["tests/test_abi.py", "tests/test_zz_no_alloc.py"],
                    {"PA_LIB": str(so), "LD_PRELOAD": rt[-1]})
    assert " passed" in out
