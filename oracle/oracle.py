"""ctypes wrapper over liboracle.so (test infrastructure only).

Matrices are any objects with the fields of ``synth.QMatrix`` (fmt, O, K,
gs, q, q2, scales) holding host numpy arrays.  Every result is float64
except ``dequant`` (float32, the materialised weights).
"""
from __future__ import annotations

import ctypes as C
import math
import os
from typing import Optional, Sequence

import numpy as np

from . import build as _build


class _Mat(C.Structure):
    _fields_ = [("fmt", C.c_int), ("O", C.c_long), ("K", C.c_long), ("gs", C.c_long),
                ("q", C.c_void_p), ("q2", C.c_void_p), ("scales", C.c_void_p)]


_P = C.c_void_p
_L = C.c_long


def _ptr(a: Optional[np.ndarray]):
    return None if a is None else a.ctypes.data_as(C.c_void_p)


NO_SCALES = (10, 11, 14)   # f32, bf16 and f16 rows carry no scales
_QBYTES = {1: 1, 13: 1, 12: 1, 10: 4, 11: 2, 14: 2}   # bytes per input of the one-code-per-input formats


def _check_matrix(m) -> None:
    if not m.q.flags["C_CONTIGUOUS"]:
        raise ValueError("q must be C-contiguous")
    if m.fmt in _QBYTES and m.q.nbytes != m.O * m.K * _QBYTES[m.fmt]:
        raise ValueError(f"fmt {m.fmt}: q holds {m.q.nbytes} bytes, expected {m.O * m.K * _QBYTES[m.fmt]}")
    if m.fmt in NO_SCALES:
        return
    if not m.scales.flags["C_CONTIGUOUS"]:
        raise ValueError("scales must be C-contiguous")
    if m.scales.dtype != np.float32:
        raise ValueError("scales must be float32")
    if m.K % m.gs:
        raise ValueError("K must be a multiple of gs")
    if m.fmt == 12 and (m.gs != 128 or m.scales.size != -(-m.O // 128) * (m.K // 128)):
        raise ValueError("fmt 12 has one scale per 128 x 128 block")
    if m.fmt == 5 and m.q2 is None:
        raise ValueError("fmt 5 needs its 1-bit plane")


def _mat(m) -> _Mat:
    _check_matrix(m)
    scales = None if m.fmt in NO_SCALES else m.scales
    return _Mat(int(m.fmt), int(m.O), int(m.K), int(m.gs), _ptr(m.q), _ptr(m.q2), _ptr(scales))


def _f32(x) -> np.ndarray:
    return np.ascontiguousarray(x, dtype=np.float32)


class OracleLib:
    """One loaded copy of the oracle (the default build, or a test's mutant)."""

    def __init__(self, path: str):
        self.path = path
        lib = C.CDLL(path)
        lib.orc_e2m1.restype = C.c_double
        lib.orc_e2m1.argtypes = [C.c_int]
        lib.orc_minifloat.restype = C.c_double
        lib.orc_minifloat.argtypes = [C.c_uint32, C.c_int, C.c_int, C.c_int]
        lib.orc_code_value.restype = C.c_double
        lib.orc_code_value.argtypes = [C.POINTER(_Mat), _L, _L]
        lib.orc_weight.restype = C.c_double
        lib.orc_weight.argtypes = [C.POINTER(_Mat), _L, _L]
        lib.orc_dequant.restype = None
        lib.orc_dequant.argtypes = [C.POINTER(_Mat), _P]
        lib.orc_gemv.restype = None
        lib.orc_gemv.argtypes = [C.POINTER(_Mat), _P, _L, _P, _P]
        lib.orc_gemv_f64.restype = None
        lib.orc_gemv_f64.argtypes = [C.POINTER(_Mat), _P, _L, _P, _P]
        lib.orc_silu.restype = C.c_double
        lib.orc_silu.argtypes = [C.c_double]
        lib.orc_gate_up.restype = None
        lib.orc_gate_up.argtypes = [C.POINTER(_Mat), C.POINTER(_Mat), _P, _L, _P, _P, _P, _P, _P, _P]
        lib.orc_expert_group.restype = None
        lib.orc_expert_group.argtypes = [_P, _P, _P, _L, _L, _L, _P, _P, _L, _P, _P, _P, _P, _P, _P, _P]
        lib.orc_expert_group_down.restype = None
        lib.orc_expert_group_down.argtypes = [_P, _L, _L, _L, _P, _P, _L, _P, _P, _P]
        lib.orc_gate_up_clamped.restype = None
        lib.orc_gate_up_clamped.argtypes = [C.POINTER(_Mat), C.POINTER(_Mat), _P, _L, C.c_double,
                                            _P, _P, _P, _P, _P, _P]
        lib.orc_expert_group_clamped.restype = None
        lib.orc_expert_group_clamped.argtypes = [_P, _P, _P, _L, _L, _L, _P, _P, _L, _P, C.c_double,
                                                 _P, _P, _P, _P, _P, _P]
        lib.orc_route.restype = None
        lib.orc_route.argtypes = [_P, _L, _L, _L, C.c_int, C.c_int, _P, C.c_double, _P, _P, _P]
        lib.orc_set_threads.restype = None
        lib.orc_round_fmt.restype = C.c_double
        lib.orc_round_fmt.argtypes = [C.c_double, C.c_int, C.c_int]
        lib.orc_v4_block_scale.restype = C.c_double
        lib.orc_v4_block_scale.argtypes = [C.c_double]
        lib.orc_v4_combine.restype = None
        lib.orc_v4_combine.argtypes = [_P, _P, _L, C.c_int, _L, _P]
        lib.orc_expert_group_v4.restype = C.c_long
        lib.orc_expert_group_v4.argtypes = [_P, _P, _P, _L, _L, _L, _P, _P, _L, _P, C.c_double, C.c_double,
                                            C.c_double, C.c_double, _P, _P, _P, _P, _P, _P]
        lib.orc_set_threads.argtypes = [C.c_int]
        lib.orc_get_threads.restype = C.c_int
        lib.orc_get_threads.argtypes = []
        self.lib = lib

    # -- scalar helpers ---------------------------------------------------
    def e2m1(self, code: int) -> float:
        return self.lib.orc_e2m1(int(code))

    def minifloat(self, code: int, ebits: int, mbits: int, ieee: bool) -> float:
        """A binary float code's value from its fields (E4M3: 4, 3, False;
        f16: 5, 10, True; bf16: 8, 7, True)."""
        return self.lib.orc_minifloat(int(code), int(ebits), int(mbits), int(bool(ieee)))

    def silu(self, z: float) -> float:
        return self.lib.orc_silu(float(z))

    def set_threads(self, n: int) -> None:
        self.lib.orc_set_threads(int(n))

    def get_threads(self) -> int:
        return self.lib.orc_get_threads()

    # -- matrices -----------------------------------------------------------
    def code_values(self, m) -> np.ndarray:
        """Signed code values v[o][k] (float64), one call per element."""
        mm = _mat(m)
        out = np.empty((m.O, m.K), dtype=np.float64)
        for o in range(m.O):
            for k in range(m.K):
                out[o, k] = self.lib.orc_code_value(C.byref(mm), o, k)
        return out

    def dequant(self, m) -> np.ndarray:
        out = np.empty((m.O, m.K), dtype=np.float32)
        self.lib.orc_dequant(C.byref(_mat(m)), _ptr(out))
        return out

    def gemv(self, m, x) -> tuple:
        """y[S][O] and its normaliser sum_k |w*x|, for x f32 [S][K] (or f64)."""
        x = np.atleast_2d(x)
        S = x.shape[0]
        if x.shape[1] != m.K:
            raise ValueError("x has the wrong width")
        y = np.empty((S, m.O), dtype=np.float64)
        a = np.empty((S, m.O), dtype=np.float64)
        if x.dtype == np.float64:
            xx = np.ascontiguousarray(x)
            self.lib.orc_gemv_f64(C.byref(_mat(m)), _ptr(xx), S, _ptr(y), _ptr(a))
        else:
            xx = _f32(x)
            self.lib.orc_gemv(C.byref(_mat(m)), _ptr(xx), S, _ptr(y), _ptr(a))
        return y, a

    def gate_up(self, G, U, x, limit: float = math.inf) -> dict:
        """h = silu(min(g, L)) * clamp(u, -L, L) with L = ``limit`` (inf: plain SwiGLU)."""
        x = _f32(np.atleast_2d(x))
        S, I = x.shape[0], G.O
        if G.K != x.shape[1] or U.K != x.shape[1] or U.O != I:
            raise ValueError("gate/up/x shapes disagree")
        out = {n: np.empty((S, I), dtype=np.float64) for n in ("h", "nh", "g", "u", "ag", "au")}
        ptrs = [_ptr(out[n]) for n in ("h", "nh", "g", "u", "ag", "au")]
        if math.isinf(limit) and limit > 0:
            self.lib.orc_gate_up(C.byref(_mat(G)), C.byref(_mat(U)), _ptr(x), S, *ptrs)
        else:
            self.lib.orc_gate_up_clamped(C.byref(_mat(G)), C.byref(_mat(U)), _ptr(x), S, float(limit), *ptrs)
        return out

    def route(self, logits, k: int, mode: int = 0, renorm: bool = False, bias=None,
              w_scale: float = 1.0) -> dict:
        """Router: ids [S][k] int32, w [S][k] float64 and the pick keys [S][E]
        (the logits without a bias, p + bias with one).  mode 0 softmax, 1 sigmoid."""
        lg = np.ascontiguousarray(logits, dtype=np.float32)
        S, E = lg.shape
        if not 1 <= k <= E:
            raise ValueError("k must be in [1, E]")
        b = None if bias is None else np.ascontiguousarray(bias, dtype=np.float32)
        if b is not None and b.shape != (E,):
            raise ValueError("bias must be [E]")
        ids = np.empty((S, k), np.int32)
        w = np.empty((S, k), np.float64)
        key = np.empty((S, E), np.float64)
        self.lib.orc_route(lg.ctypes.data, S, E, k, int(mode), int(bool(renorm)),
                           None if b is None else b.ctypes.data, float(w_scale),
                           ids.ctypes.data, w.ctypes.data, key.ctypes.data)
        return {"ids": ids, "w": w, "key": key}

    def expert_group(self, experts: Sequence, ids, w, shared: Optional[int], x,
                     limit: float = math.inf) -> tuple:
        """y[S][H] and its normaliser for a token batch.

        ``experts`` is a sequence of objects with gate/up/down matrices,
        indexed by expert id.  Only the experts that ``ids`` and ``shared``
        name are handed to the C code (the others are never read).
        """
        ids = np.ascontiguousarray(ids, dtype=np.int32)
        w = _f32(w)
        x = _f32(np.atleast_2d(x))
        S, k = ids.shape
        used = sorted({int(e) for e in ids.ravel() if 0 <= int(e) < len(experts)}
                      | ({int(shared)} if shared is not None and shared >= 0 else set()))
        remap = {e: i for i, e in enumerate(used)}
        # an id outside the table stays outside the compact table too
        cids = np.array([[remap.get(int(e), -1) for e in row] for row in ids], dtype=np.int32)
        cshared = remap[int(shared)] if shared is not None and shared >= 0 else -1
        n = len(used)
        gates = (_Mat * max(n, 1))(*[_mat(experts[e].gate) for e in used])
        ups = (_Mat * max(n, 1))(*[_mat(experts[e].up) for e in used])
        downs = (_Mat * max(n, 1))(*[_mat(experts[e].down) for e in used])
        H = experts[used[0]].down.O
        I = experts[used[0]].gate.O
        y = np.empty((S, H), dtype=np.float64)
        a = np.empty((S, H), dtype=np.float64)
        hw = np.empty(I, dtype=np.float64)
        nw = np.empty(I, dtype=np.float64)
        dw = np.empty(H, dtype=np.float64)
        aw = np.empty(H, dtype=np.float64)
        args = (C.cast(gates, C.c_void_p), C.cast(ups, C.c_void_p), C.cast(downs, C.c_void_p), n, S, k,
                _ptr(cids), _ptr(w), cshared, _ptr(x))
        work = (_ptr(y), _ptr(a), _ptr(hw), _ptr(nw), _ptr(dw), _ptr(aw))
        if math.isinf(limit) and limit > 0:
            self.lib.orc_expert_group(*args, *work)
        else:
            self.lib.orc_expert_group_clamped(*args, float(limit), *work)
        return y, a

    def expert_group_down(self, experts: Sequence, ids, w, shared: Optional[int], h) -> tuple:
        """The group's down and combine on given hidden states h, f32
        [S*k + S][I] in the device scratch's slot order (slot t*k + r, then
        S*k + t for token t's shared expert).  Returns y [S][H] and its
        normaliser sum_r |w| * sum_i |D[o][i] h[i]| (+ the shared row's)."""
        ids = np.ascontiguousarray(ids, dtype=np.int32)
        w = _f32(w)
        S, k = ids.shape
        h = _f32(h)
        used = sorted({int(e) for e in ids.ravel() if 0 <= int(e) < len(experts)}
                      | ({int(shared)} if shared is not None and shared >= 0 else set()))
        if not used:
            raise ValueError("no valid expert id")
        I = experts[used[0]].down.K
        H = experts[used[0]].down.O
        if h.ndim != 2 or h.shape[1] != I or h.shape[0] < S * k + S:
            raise ValueError(f"h must be [S*k + S][I] = [{S * k + S}][{I}], got {h.shape}")
        remap = {e: i for i, e in enumerate(used)}
        cids = np.array([[remap.get(int(e), -1) for e in row] for row in ids], dtype=np.int32)
        cshared = remap[int(shared)] if shared is not None and shared >= 0 else -1
        downs = (_Mat * len(used))(*[_mat(experts[e].down) for e in used])
        y = np.empty((S, H), dtype=np.float64)
        a = np.empty((S, H), dtype=np.float64)
        self.lib.orc_expert_group_down(C.cast(downs, C.c_void_p), len(used), S, k, _ptr(cids), _ptr(w), cshared,
                                       _ptr(h), _ptr(y), _ptr(a))
        return y, a

    def round_fmt(self, v: float, mbits: int, emin: int) -> float:
        return self.lib.orc_round_fmt(float(v), int(mbits), int(emin))

    def v4_block_scale(self, m: float) -> float:
        return self.lib.orc_v4_block_scale(float(m))

    def v4_combine(self, rows, ids, has_shared: bool) -> np.ndarray:
        """One token's rows [k (+1 shared)][H] added as DeepSeek V4's path adds them (f32)."""
        rows = np.ascontiguousarray(rows, dtype=np.float64)
        ids = np.ascontiguousarray(ids, dtype=np.int32)
        k, H = len(ids), rows.shape[1]
        if rows.shape[0] != k + int(bool(has_shared)):
            raise ValueError("rows must hold k rows, then the shared row if any")
        y = np.empty(H, dtype=np.float32)
        self.lib.orc_v4_combine(_ptr(rows), _ptr(ids), k, int(bool(has_shared)), H, _ptr(y))
        return y

    def expert_group_v4(self, experts: Sequence, ids, w, shared: Optional[int], x, limit: float = math.inf,
                        gu_err: float = 0.0, act_rel: float = 0.0, down_err: float = 0.0) -> dict:
        """The expert group with DeepSeek V4's rounding activation.

        Returns h [S*k + S][I] (down's input per slot) with its bounds h_lo,
        h_hi, then y, y_lo, y_hi (f32 [S][H]) and ``open``: the number of
        bf16 decisions before down that a device within the given error
        bounds could take the other way.
        """
        ids = np.ascontiguousarray(ids, dtype=np.int32)
        w = _f32(w)
        x = _f32(np.atleast_2d(x))
        S, k = ids.shape
        used = sorted({int(e) for e in ids.ravel() if 0 <= int(e) < len(experts)}
                      | ({int(shared)} if shared is not None and shared >= 0 else set()))
        remap = {e: i for i, e in enumerate(used)}
        # the compact table keeps the ids' order, so the combine order is unchanged
        cids = np.array([[remap.get(int(e), -1) for e in row] for row in ids], dtype=np.int32)
        cshared = remap[int(shared)] if shared is not None and shared >= 0 else -1
        n = len(used)
        gates = (_Mat * max(n, 1))(*[_mat(experts[e].gate) for e in used])
        ups = (_Mat * max(n, 1))(*[_mat(experts[e].up) for e in used])
        downs = (_Mat * max(n, 1))(*[_mat(experts[e].down) for e in used])
        H = experts[used[0]].down.O
        I = experts[used[0]].gate.O
        if I % 128:
            raise ValueError("DeepSeek V4's activation rounds blocks of 128: I must be a multiple of 128")
        h, h_lo, h_hi = (np.full((S * k + S, I), np.nan) for _ in range(3))
        y, y_lo, y_hi = (np.empty((S, H), dtype=np.float32) for _ in range(3))
        n_open = self.lib.orc_expert_group_v4(
            C.cast(gates, C.c_void_p), C.cast(ups, C.c_void_p), C.cast(downs, C.c_void_p), n, S, k,
            _ptr(cids), _ptr(w), cshared, _ptr(x), float(limit), float(gu_err), float(act_rel),
            float(down_err), _ptr(h), _ptr(h_lo), _ptr(h_hi), _ptr(y), _ptr(y_lo), _ptr(y_hi))
        if n_open < 0:
            raise MemoryError("oracle: out of memory")
        return {"h": h, "h_lo": h_lo, "h_hi": h_hi, "y": y, "y_lo": y_lo, "y_hi": y_hi, "open": int(n_open)}


_default: Optional[OracleLib] = None


def load(path: Optional[str] = None) -> OracleLib:
    """The default oracle (built on demand), or the library at ``path``."""
    global _default
    if path is not None:
        return OracleLib(path)
    if _default is None:
        _default = OracleLib(_build.ensure_built())
    return _default


def e2m1(code):
    return load().e2m1(code)


def minifloat(code, ebits, mbits, ieee):
    return load().minifloat(code, ebits, mbits, ieee)


def silu(z):
    return load().silu(z)


def set_threads(n):
    load().set_threads(n)


def get_threads():
    return load().get_threads()


def code_values(m):
    return load().code_values(m)


def dequant(m):
    return load().dequant(m)


def gemv(m, x):
    return load().gemv(m, x)


def gate_up(G, U, x, limit=math.inf):
    return load().gate_up(G, U, x, limit)


def expert_group(experts, ids, w, shared, x, limit=math.inf):
    return load().expert_group(experts, ids, w, shared, x, limit)


def expert_group_down(experts, ids, w, shared, h):
    return load().expert_group_down(experts, ids, w, shared, h)


def route(logits, k, mode=0, renorm=False, bias=None, w_scale=1.0):
    return load().route(logits, k, mode, renorm, bias, w_scale)


def round_fmt(v, mbits, emin):
    return load().round_fmt(v, mbits, emin)


def v4_block_scale(m):
    return load().v4_block_scale(m)


def v4_combine(rows, ids, has_shared):
    return load().v4_combine(rows, ids, has_shared)


def expert_group_v4(experts, ids, w, shared, x, limit=math.inf, gu_err=0.0, act_rel=0.0, down_err=0.0):
    return load().expert_group_v4(experts, ids, w, shared, x, limit, gu_err, act_rel, down_err)
