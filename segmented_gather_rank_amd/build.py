"""Build the HIP library for gfx950 in-tree: segmented_gather_rank_amd/liblora_mi355x.so.

One hipcc invocation compiles every HIP source of ``csrc/`` for gfx950 only and
links a shared library exporting the C ABI of ``include/lora_mi355x.h``.
"""
import glob
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "liblora_mi355x.so")
ARCH = "gfx950"

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-shared",
    "-Wall", "-Wno-unused-function",
    # no packed-fp32 instructions in the device code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # the first kernel arguments (the pointers each kernel reads first) arrive
    # preloaded in scalar registers
    "-mllvm", "-amdgpu-kernarg-preload-count=6",
    f"-I{os.path.join(ROOT, 'include')}",
]


def sources():
    return sorted(glob.glob(os.path.join(CSRC, "*.hip")))


def build(out: str = LIB, extra=()) -> str:
    cmd = [HIPCC, *FLAGS, *extra, "-o", out + ".tmp", *sources()]
    subprocess.run(cmd, check=True)
    os.replace(out + ".tmp", out)
    return out


if __name__ == "__main__":
    print(build(extra=sys.argv[1:]))
