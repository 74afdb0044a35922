"""AddressSanitizer and UndefinedBehaviorSanitizer builds of the CPU side.

- The oracle (oracle/oracle.c) built with -fsanitize=address,undefined runs
  every pin of tests/pinlib.py in a child process with the ASan runtime
  preloaded (Python itself is not instrumented; leak checks are off for it).
- The C-ABI layer (dequant_gemv_expert_amd/csrc/dqg_api.cpp), built for the
  host with the same sanitizers against stand-in launchers
  (tests/san/launch_stubs.cpp), runs tests/san/abi_driver.cpp: every
  argument check of every entry point, none of which may reach a launcher;
  leak checks on.

UBSan stops at the first finding (-fno-sanitize-recover), so a finding of
either sanitizer fails the child process.
"""
import os
import shutil
import subprocess
import sys

import pytest

from oracle import build as obuild

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SAN = ["-fsanitize=address,undefined", "-fno-sanitize-recover=undefined", "-fno-omit-frame-pointer", "-g", "-O1"]
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")


def _asan_runtime() -> str:
    out = subprocess.run(["gcc", "-print-file-name=libasan.so"], capture_output=True, text=True, check=True)
    return out.stdout.strip()


def _clean(proc):
    text = proc.stdout + proc.stderr
    assert "ERROR: AddressSanitizer" not in text, text[-4000:]
    assert "ERROR: LeakSanitizer" not in text, text[-4000:]
    assert "runtime error:" not in text, text[-4000:]
    assert proc.returncode == 0, text[-4000:]


@pytest.mark.skipif(shutil.which("gcc") is None, reason="gcc not installed")
def test_oracle_pins_under_asan_ubsan(tmp_path):
    lib = str(tmp_path / "liboracle_san.so")
    flags = [f for f in obuild.CFLAGS if not f.startswith("-O")] + SAN
    subprocess.run(["gcc", *flags, obuild.SRC, "-o", lib, "-lm"], check=True)
    code = (
        "import sys\n"
        f"sys.path.insert(0, {ROOT!r}); sys.path.insert(0, {os.path.join(ROOT, 'tests')!r})\n"
        "import oracle, pinlib\n"
        f"o = oracle.load({lib!r})\n"
        "for p in pinlib.ALL_PINS:\n"
        "    p(o)\n"
        "print('pins', len(pinlib.ALL_PINS))\n"
    )
    env = dict(os.environ, LD_PRELOAD=_asan_runtime(), ASAN_OPTIONS="detect_leaks=0",
               UBSAN_OPTIONS="print_stacktrace=1", OMP_NUM_THREADS="4")
    proc = subprocess.run([sys.executable, "-c", code], env=env, capture_output=True, text=True, timeout=600)
    _clean(proc)
    assert proc.stdout.startswith("pins "), proc.stdout


@pytest.mark.skipif(shutil.which("g++") is None or not os.path.exists(os.path.join(ROCM, "include", "hip")),
                    reason="g++ or the HIP headers not installed")
def test_abi_validation_under_asan_ubsan(tmp_path):
    exe = str(tmp_path / "abi_san")
    srcs = [os.path.join(ROOT, "dequant_gemv_expert_amd", "csrc", "dqg_api.cpp"),
            os.path.join(ROOT, "tests", "san", "launch_stubs.cpp"),
            os.path.join(ROOT, "tests", "san", "abi_driver.cpp")]
    subprocess.run(["g++", "-std=c++17", "-D__HIP_PLATFORM_AMD__", f"-I{ROCM}/include", *SAN, *srcs,
                    f"-L{ROCM}/lib", "-lamdhip64", f"-Wl,-rpath,{ROCM}/lib", "-o", exe], check=True)
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1", UBSAN_OPTIONS="print_stacktrace=1")
    proc = subprocess.run([exe], env=env, capture_output=True, text=True, timeout=300)
    _clean(proc)
    assert " 0 failed" in proc.stdout, proc.stdout
