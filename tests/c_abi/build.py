"""Build the plain-C ABI check program (decode_check.c) with gcc against the
library's header and the HIP runtime's C API; it links libpaged_attn.so and
the oracle's liboracle.so from the repository tree (rpath relative to the
binary)."""
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
SRC = os.path.join(HERE, "decode_check.c")
BIN = os.path.join(HERE, "decode_check")
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")


def build() -> str:
    tmp = BIN + ".tmp%d" % os.getpid()
    cmd = ["gcc", "-std=c11", "-O2", "-Wall", "-Wextra", "-D__HIP_PLATFORM_AMD__",
           "-I", os.path.join(ROOT, "include"), "-I", os.path.join(ROOT, "oracle"),
           "-I", os.path.join(ROCM, "include"), SRC, "-o", tmp,
           "-L", os.path.join(ROOT, "sliding_window_mask_amd"), "-lpaged_attn",
           "-L", os.path.join(ROOT, "oracle"), "-loracle",
           "-L", os.path.join(ROCM, "lib"), "-lamdhip64", "-lm",
           "-Wl,-rpath,$ORIGIN/../../sliding_window_mask_amd",
           "-Wl,-rpath,$ORIGIN/../../oracle", "-Wl,-rpath," + os.path.join(ROCM, "lib")]
    subprocess.run(cmd, check=True)
    os.replace(tmp, BIN)
    return BIN


if __name__ == "__main__":
    print(build())
