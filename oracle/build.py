"""Build the CPU oracle shared library (plain C, gcc, no GPU code).

Test infrastructure only: the oracle is loaded by the tests, the smoke check
and the benchmark's CPU-baseline leg, never by the GPU product path.
"""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "lora_oracle.c")
LIB = os.path.join(HERE, "liblora_oracle.so")


def build(src: str = SRC, out: str = LIB, extra_flags=()) -> str:
    """Compile ``src`` into the shared library ``out`` and return its path.

    -O2 without any fast-math flag: the fp64 summation order written in the
    source is the order that runs.
    """
    cmd = ["gcc", "-std=c99", "-O2", "-fPIC", "-shared", "-Wall", "-Wextra",
           *extra_flags, "-o", out + ".tmp", src]
    subprocess.run(cmd, check=True)
    os.replace(out + ".tmp", out)
    return out


if __name__ == "__main__":
    print(build(*sys.argv[1:2]))
