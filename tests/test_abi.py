"""The C ABI without a GPU: the library loads, exports every symbol the
header declares, and rejects bad arguments before any HIP call."""
import ctypes as C
import os
import re
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "dqg.h")

from dequant_gemv_expert_amd import _lib as L  # noqa: E402
from dequant_gemv_expert_amd import build as B  # noqa: E402


def header_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(dqg_[a-z_0-9]+)\s*\(", text)))


@pytest.fixture(scope="module")
def lib():
    if B.is_stale():
        B.build()
    return L.load()


def test_header_and_binding_agree():
    assert header_functions() == sorted(L.SIGNATURES)


def test_every_declared_symbol_is_exported(lib):
    for name in header_functions():
        assert hasattr(lib, name), name


def _mat(fmt=4, O=64, K=256, gs=32, q=0x10000, q2=0, s=0x20000):
    return L.dqg_matrix(fmt, O, K, gs, q, q2, s)


FAKE_X, FAKE_Y = 0x30000, 0x40000   # never dereferenced: each call below fails validation


@pytest.mark.parametrize("mat,code", [
    (_mat(fmt=3), -2),
    (_mat(fmt=4, gs=48), -2),
    (_mat(fmt=4, gs=16), -2),
    (_mat(fmt=4, K=96, gs=64), -3),
    (_mat(fmt=4, K=100), -3),
    (_mat(fmt=1, K=512, gs=32), -2),
    (_mat(fmt=1, K=520, gs=520), -3),
    (_mat(fmt=5, K=256, gs=32), -2),
    (_mat(fmt=5, K=96, gs=64), -3),
    (_mat(fmt=7, gs=64), -2),
    (_mat(fmt=4, O=0), -3),
    (_mat(q=0), -1),
    (_mat(q=0x10008), -1),
    (_mat(s=0x20002), -1),
    (_mat(fmt=5, gs=64, q2=0), -1),
    # formats without scales: gs 0 or K, scales NULL
    (_mat(fmt=10, K=256, gs=32, s=0), -2),
    (_mat(fmt=11, K=256, gs=256), -1),            # a scales pointer given
    (_mat(fmt=14, K=100, gs=0, s=0), -3),         # K not a multiple of 8
    (_mat(fmt=10, K=6, gs=0, s=0), -3),           # K not a multiple of 4
    # E4M3 blocks: gs 128, K a multiple of 128, scales required
    (_mat(fmt=12, K=256, gs=64), -2),
    (_mat(fmt=12, K=192, gs=128), -3),
    (_mat(fmt=12, K=256, gs=128, s=0), -1),
    # int8 with group scales
    (_mat(fmt=13, K=256, gs=16), -2),
    (_mat(fmt=13, K=256, gs=48), -2),
    (_mat(fmt=13, K=96, gs=64), -3),
    (_mat(fmt=13, K=256, gs=64, s=0), -1),
    (_mat(fmt=9), -2),
    (_mat(fmt=15), -2),
])
def test_matrix_validation(lib, mat, code):
    rc = lib.dqg_matmul(C.byref(mat), FAKE_X, 1, FAKE_Y, None)
    assert rc == code, (rc, lib.dqg_last_error())
    assert lib.dqg_last_error()


def test_vector_validation(lib):
    m = _mat()
    assert lib.dqg_matmul(C.byref(m), 0, 1, FAKE_Y, None) == -1
    assert lib.dqg_matmul(C.byref(m), FAKE_X + 4, 1, FAKE_Y, None) == -1
    assert lib.dqg_matmul(C.byref(m), FAKE_X, 0, FAKE_Y, None) == -1
    assert lib.dqg_dequant(C.byref(m), 0, None) == -1
    g, u = _mat(), _mat(K=512)
    assert lib.dqg_gate_up(C.byref(g), C.byref(u), FAKE_X, 1, FAKE_Y, None) == -3


def test_read_bytes_validation(lib):
    """Argument checks of the streaming-read entry, which launch nothing."""
    assert lib.dqg_read_bytes(None, 1024, FAKE_Y, None) == -1
    assert lib.dqg_read_bytes(FAKE_X + 8, 1024, FAKE_Y, None) == -1      # p not 16-byte aligned
    assert lib.dqg_read_bytes(FAKE_X, 0, FAKE_Y, None) == -1
    assert lib.dqg_read_bytes(FAKE_X, 1000, FAKE_Y, None) == -1          # not a multiple of 1024
    assert lib.dqg_read_bytes(FAKE_X, 1024, None, None) == -1
    assert b"sink" in lib.dqg_last_error()


def test_expert_group_validation(lib):
    assert lib.dqg_expert_group(None, 1, 8, 0x1000, 0x2000, -1, FAKE_X, FAKE_Y, 0x50000, 1 << 20, None) == -1
    assert lib.dqg_expert_group_noalloc(None, 1, 8, 0x1000, 0x2000, -1, FAKE_X, FAKE_Y, None) == -1
    assert b"table is NULL" in lib.dqg_last_error()
    assert lib.dqg_expert_group_scratch_bytes(None, 1, 8) == 0
    t = L.dqg_ticket()
    assert lib.dqg_expert_group_take(C.byref(t)) == -1


FAKE_L, FAKE_IDS, FAKE_W = 0x60000, 0x70000, 0x80000


@pytest.mark.parametrize("S,E,k,mode,renorm,bias,scale,logits,ids,w", [
    (0, 64, 8, 0, 0, None, 1.0, FAKE_L, FAKE_IDS, FAKE_W),          # no tokens
    (1, 0, 1, 0, 0, None, 1.0, FAKE_L, FAKE_IDS, FAKE_W),           # no experts
    (1, 1025, 8, 0, 0, None, 1.0, FAKE_L, FAKE_IDS, FAKE_W),        # more experts than one wave holds
    (1, 64, 0, 0, 0, None, 1.0, FAKE_L, FAKE_IDS, FAKE_W),          # k = 0
    (1, 6, 7, 0, 0, None, 1.0, FAKE_L, FAKE_IDS, FAKE_W),           # k > E
    (1, 256, 65, 0, 0, None, 1.0, FAKE_L, FAKE_IDS, FAKE_W),        # k > 64
    (1, 64, 8, 2, 0, None, 1.0, FAKE_L, FAKE_IDS, FAKE_W),          # unknown mode
    (1, 64, 8, 0, 2, None, 1.0, FAKE_L, FAKE_IDS, FAKE_W),          # renorm not 0/1
    (1, 64, 8, 0, 0, None, float("inf"), FAKE_L, FAKE_IDS, FAKE_W), # scale not finite
    (1, 64, 8, 0, 0, None, float("nan"), FAKE_L, FAKE_IDS, FAKE_W),
    (1, 64, 8, 0, 0, None, 1.0, 0, FAKE_IDS, FAKE_W),               # null logits
    (1, 64, 8, 0, 0, None, 1.0, FAKE_L + 2, FAKE_IDS, FAKE_W),      # misaligned
    (1, 64, 8, 0, 0, 0x90002, 1.0, FAKE_L, FAKE_IDS, FAKE_W),
    (1, 64, 8, 0, 0, None, 1.0, FAKE_L, 0, FAKE_W),
    (1, 64, 8, 0, 0, None, 1.0, FAKE_L, FAKE_IDS, FAKE_W + 1),
])
def test_route_validation(lib, S, E, k, mode, renorm, bias, scale, logits, ids, w):
    lib.dqg_stats_reset()
    rc = lib.dqg_route(logits, S, E, k, mode, renorm, bias, scale, ids, w, None)
    assert rc == -1, (rc, lib.dqg_last_error())
    assert lib.dqg_last_error()
    c = L.dqg_counters()
    lib.dqg_stats(C.byref(c))
    assert c.calls_route == 1 and c.launches == 0


@pytest.mark.parametrize("limit", [0.0, -1.0, float("nan"), float("-inf")])
def test_swiglu_limit_validation(lib, limit):
    g, u = _mat(), _mat()
    assert lib.dqg_gate_up_clamped(C.byref(g), C.byref(u), FAKE_X, 1, limit, FAKE_Y, None) == -1
    assert "limit" in lib.dqg_last_error().decode()
    assert lib.dqg_expert_table_set_swiglu_limit(None, 1.0) == -1


def test_activation_validation(lib):
    assert lib.dqg_expert_table_set_activation(None, L.DQG_ACT_SWIGLU_V4) == -1
    assert "NULL" in lib.dqg_last_error().decode()


def test_table_validation(lib):
    e = L.dqg_expert(_mat(O=32, K=64), _mat(O=32, K=64), _mat(O=64, K=64))   # down must be [64 x 32]
    out = C.c_void_p()
    rc = lib.dqg_expert_table_create(C.byref(e), 1, C.byref(out))
    assert rc == -3 and not out.value
    e = L.dqg_expert(_mat(O=32, K=64), _mat(fmt=7, O=32, K=64), _mat(O=64, K=32))
    assert lib.dqg_expert_table_create(C.byref(e), 1, C.byref(out)) == -3
    assert lib.dqg_expert_table_create(C.byref(e), 0, C.byref(out)) == -1


def test_stats_count_calls(lib):
    lib.dqg_stats_reset()
    m = _mat(fmt=3)
    lib.dqg_matmul(C.byref(m), FAKE_X, 1, FAKE_Y, None)
    c = L.dqg_counters()
    lib.dqg_stats(C.byref(c))
    assert c.calls_matmul == 1 and c.launches == 0


def test_fault_injection_fails_before_launch():
    """DQG_FAULT=1: the first launch attempt returns DQG_ELAUNCH without reaching HIP."""
    code = (
        "import ctypes as C, sys\n"
        f"sys.path.insert(0, {ROOT!r})\n"
        "from dequant_gemv_expert_amd import _lib as L\n"
        "lib = L.load()\n"
        "m = L.dqg_matrix(4, 64, 256, 32, 0x10000, 0, 0x20000)\n"
        "rc = lib.dqg_matmul(C.byref(m), 0x30000, 1, 0x40000, None)\n"
        "print(rc, lib.dqg_last_error().decode())\n"
    )
    env = dict(os.environ, DQG_FAULT="1")
    out = subprocess.run([sys.executable, "-c", code], env=env, capture_output=True, text=True, timeout=120)
    assert out.returncode == 0, out.stderr
    rc, msg = out.stdout.split(" ", 1)
    assert int(rc) == -5 and "DQG_FAULT" in msg


def test_binding_refuses_host_tensors():
    import torch
    with pytest.raises(TypeError):
        L._dev(torch.zeros(4), "x")
