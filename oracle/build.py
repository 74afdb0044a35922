"""Build the CPU oracle (oracle.c) into liboracle.so with gcc.

Test infrastructure: compiling the checker is part of the build, and only
the tests, the smoke check and the benchmark's CPU-baseline leg load it.
"""
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "oracle.c")
LIB = os.path.join(HERE, "liboracle.so")

# No -ffast-math and no contraction: the oracle's sums are plain IEEE
# double operations in source order.
CFLAGS = ["-O2", "-fopenmp", "-ffp-contract=off", "-fno-fast-math", "-fPIC", "-shared",
          "-std=c11", "-Wall", "-Wextra"]


def build(src: str = SRC, out: str = LIB, extra=()) -> str:
    cmd = ["gcc", *CFLAGS, *extra, src, "-o", out, "-lm"]
    subprocess.run(cmd, check=True)
    return out


def ensure_built() -> str:
    if not os.path.exists(LIB) or os.path.getmtime(LIB) < os.path.getmtime(SRC):
        build()
    return LIB


if __name__ == "__main__":
    print(build())
