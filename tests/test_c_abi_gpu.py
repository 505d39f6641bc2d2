"""The C ABI used from plain C: tests/c_abi/decode_check.c (built by the
package build with gcc, no C++ and no Python) allocates with hipMalloc, runs
paged_attn_decode with and without a window and compares with the float64
oracle, and checks a host-side rejection."""
import os
import subprocess

import pytest

pytestmark = pytest.mark.gpu
BIN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "c_abi", "decode_check")


def test_plain_c_consumer_matches_oracle():
    assert os.path.exists(BIN), "tests/c_abi/decode_check is not built: run the package build"
    r = subprocess.run([BIN], capture_output=True, text=True, timeout=120)
    print(r.stdout, r.stderr)
    assert r.returncode == 0, r.stdout + r.stderr
    lines = [l for l in r.stdout.splitlines() if l.startswith(("decode", "head_dim"))]
    assert len(lines) == 3 and all(l.endswith("ok") for l in lines), r.stdout
