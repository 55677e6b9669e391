"""Build libconv_check.so (gfx950), the GPU test helper that runs the quantizers' scalar
device functions over ranges of inputs.  Same compiler flags as the library; built in-tree
next to its source by __graft_entry__.build()."""
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
SRC = os.path.join(HERE, "conv_check.hip")
LIB = os.path.join(HERE, "libconv_check.so")
CSRC = os.path.join(ROOT, "unbiased_nvfp4_gradient_amd", "csrc")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")


def build() -> str:
    tmp = LIB + ".tmp"
    subprocess.check_call([HIPCC, "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
                           "-shared", "-ffp-contract=off", "-fno-fast-math", "-Xclang",
                           "-target-feature", "-Xclang", "-packed-fp32-ops", "-Wall",
                           "-I", CSRC, SRC, "-o", tmp], cwd="/tmp")
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build())
