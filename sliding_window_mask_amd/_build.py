"""Build libpaged_attn.so (and the no-bias comparison build) with hipcc for gfx950.

The libraries are built in-tree, next to this file:
  libpaged_attn.so         the product library
  libpaged_attn_nobias.so  the same sources with -DPA_NO_BIAS: the decode path
                           compiled without the bias branch, used only to show
                           what a null bias costs against a build that cannot
                           take one.
"""
from __future__ import annotations

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
SOURCES = ["pa_api.cpp", "pa_decode.hip", "pa_prefill.hip", "pa_prefill_f32x3.hip",
           "pa_prefill_bf16.hip", "pa_cache.hip"]
LIB = os.path.join(HERE, "libpaged_attn.so")
LIB_NOBIAS = os.path.join(HERE, "libpaged_attn_nobias.so")

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared",
    # contraction only where the source asks for it (fmaf): the bias / no-bias
    # score paths must round identically
    "-ffp-contract=off",
    # no packed fp32 instructions
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # keep MFMA accumulators in VGPRs (no AGPR round trips for the softmax
    # rescale of the prefill accumulators)
    "-mllvm", "--amdgpu-mfma-vgpr-form",
    "-Wall", "-Wno-unused-result",
]


def _compile(out: str, extra: list[str]) -> None:
    tmp = out + ".tmp%d" % os.getpid()
    cmd = [HIPCC] + FLAGS + extra + ["-I", INCLUDE, "-I", CSRC, "-o", tmp] + [
        os.path.join(CSRC, s) for s in SOURCES]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        sys.stderr.write(r.stdout + r.stderr)
        raise RuntimeError("hipcc failed building %s" % os.path.basename(out))
    os.replace(tmp, out)


def build(nobias: bool = True) -> list[str]:
    """Compile the library (and the no-bias build). Always recompiles."""
    _compile(LIB, [])
    built = [LIB]
    if nobias:
        _compile(LIB_NOBIAS, ["-DPA_NO_BIAS"])
        built.append(LIB_NOBIAS)
    return built


if __name__ == "__main__":
    for p in build():
        print(p)
