"""Compile libdqg.so (the HIP kernels and the C ABI) for gfx950 with hipcc.

The library is built in-tree (dequant_gemv_expert_amd/libdqg.so) so that it
travels with the source tree; nothing is JIT-compiled at run time.
"""
import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
SOURCES = [os.path.join(CSRC, "dqg_kernels.hip"), os.path.join(CSRC, "dqg_api.cpp")]
HEADERS = [os.path.join(CSRC, "dqg_internal.h"), os.path.join(ROOT, "include", "dqg.h")]
LIB = os.path.join(HERE, "libdqg.so")
ARCH = os.environ.get("DQG_OFFLOAD_ARCH", "gfx950")

FLAGS = [
    "-O3", "-std=c++17", "-fPIC", "-shared",
    f"--offload-arch={ARCH}",
    # IEEE f32 arithmetic as written: no contraction beyond the explicit fmaf calls
    "-ffp-contract=off",
    # no packed fp32 instructions are generated
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall",
]


def hipcc() -> str:
    path = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(path):
        raise RuntimeError("hipcc not found")
    return path


def build(out: str = LIB, extra=(), verbose: bool = False) -> str:
    tmp = out + ".tmp"
    cmd = [hipcc(), *FLAGS, *extra, "-x", "hip", *SOURCES, "-o", tmp]
    if verbose:
        print(" ".join(cmd), file=sys.stderr)
    subprocess.run(cmd, check=True)
    os.replace(tmp, out)
    return out


def is_stale(lib: str = LIB) -> bool:
    if not os.path.exists(lib):
        return True
    t = os.path.getmtime(lib)
    return any(os.path.getmtime(p) > t for p in SOURCES + HEADERS)


if __name__ == "__main__":
    # python -m dequant_gemv_expert_amd.build [--out PATH] [-DNAME=VALUE ...]:
    # the library, or a copy at another path (with extra preprocessor
    # definitions) that DQG_LIBRARY=PATH loads instead
    args = sys.argv[1:]
    out = LIB
    if args[:1] == ["--out"]:
        out, args = args[1], args[2:]
    if any(not a.startswith("-D") for a in args):
        raise SystemExit("usage: python -m dequant_gemv_expert_amd.build [--out PATH] [-DNAME=VALUE ...]")
    print(build(out, extra=args, verbose=True))
