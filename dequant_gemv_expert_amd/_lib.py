"""ctypes binding of libdqg.so: the C ABI of include/dqg.h, one Python
function per C entry point, with the same names.

Argument marshalling only: every step of the path runs in the library's
HIP kernels.  PyTorch supplies device memory and the current stream.  There
is no fallback: a missing library or a tensor that is not on a GPU raises.
"""
from __future__ import annotations

import ctypes as C
import os
from typing import Optional, Sequence

import numpy as np
import torch

from . import build as _build

DQG_OK = 0
STATUS = {0: "DQG_OK", -1: "DQG_EINVAL", -2: "DQG_EFORMAT", -3: "DQG_ESHAPE", -4: "DQG_EDEVICE",
          -5: "DQG_ELAUNCH", -6: "DQG_ENOMEM", -7: "DQG_EROUTE"}

DQG_I8_ROW, DQG_I4_ROW, DQG_I4_GS, DQG_I3_G64, DQG_MXFP4 = 1, 2, 4, 5, 7
DQG_F32, DQG_BF16, DQG_FP8_BLOCK, DQG_I8_GS, DQG_F16 = 10, 11, 12, 13, 14
DQG_ROUTE_SOFTMAX, DQG_ROUTE_SIGMOID = 0, 1
DQG_ACT_SWIGLU, DQG_ACT_SWIGLU_V4 = 0, 1


class DqgError(RuntimeError):
    def __init__(self, code: int, message: str):
        super().__init__(f"{STATUS.get(code, code)}: {message}")
        self.code = code


class dqg_matrix(C.Structure):
    _fields_ = [("fmt", C.c_int32), ("O", C.c_int32), ("K", C.c_int32), ("gs", C.c_int32),
                ("q", C.c_void_p), ("q2", C.c_void_p), ("scales", C.c_void_p)]


class dqg_expert(C.Structure):
    _fields_ = [("gate", dqg_matrix), ("up", dqg_matrix), ("down", dqg_matrix)]


class dqg_ticket(C.Structure):
    _fields_ = [("event", C.c_void_p), ("flag", C.c_void_p), ("status", C.c_int32)]


class dqg_counters(C.Structure):
    _fields_ = [("calls_matmul", C.c_uint64), ("calls_gate_up", C.c_uint64),
                ("calls_dequant", C.c_uint64), ("calls_expert_group", C.c_uint64),
                ("launches", C.c_uint64), ("bytes", C.c_uint64), ("calls_route", C.c_uint64)]


class dqg_prof_launch(C.Structure):
    _fields_ = [("kernel", C.c_char * 32), ("ms", C.c_double)]


class dqg_prof_record(C.Structure):
    _fields_ = [("kernel", C.c_char * 32), ("launches", C.c_int64), ("total_ms", C.c_double)]


# Every symbol the header declares, with its ctypes signature.
_P, _I32, _SZ = C.c_void_p, C.c_int32, C.c_size_t
SIGNATURES = {
    "dqg_matmul": (C.c_int, [C.POINTER(dqg_matrix), _P, _I32, _P, _P]),
    "dqg_gate_up": (C.c_int, [C.POINTER(dqg_matrix), C.POINTER(dqg_matrix), _P, _I32, _P, _P]),
    "dqg_gate_up_clamped": (C.c_int, [C.POINTER(dqg_matrix), C.POINTER(dqg_matrix), _P, _I32, C.c_float, _P, _P]),
    "dqg_dequant": (C.c_int, [C.POINTER(dqg_matrix), _P, _P]),
    "dqg_read_bytes": (C.c_int, [_P, C.c_uint64, _P, _P]),
    "dqg_expert_table_create": (C.c_int, [C.POINTER(dqg_expert), _I32, C.POINTER(C.c_void_p)]),
    "dqg_expert_table_destroy": (None, [_P]),
    "dqg_expert_table_set_swiglu_limit": (C.c_int, [_P, C.c_float]),
    "dqg_expert_table_set_activation": (C.c_int, [_P, C.c_int32]),
    "dqg_expert_group_scratch_bytes": (_SZ, [_P, _I32, _I32]),
    "dqg_expert_group": (C.c_int, [_P, _I32, _I32, _P, _P, _I32, _P, _P, _P, _SZ, _P]),
    "dqg_expert_group_issue": (C.c_int, [_P, _I32, _I32, _P, _P, _I32, _P, _P, _P, _SZ, _P,
                                         C.POINTER(dqg_ticket)]),
    "dqg_expert_group_take": (C.c_int, [C.POINTER(dqg_ticket)]),
    "dqg_expert_group_noalloc": (C.c_int, [_P, _I32, _I32, _P, _P, _I32, _P, _P, _P]),
    "dqg_route": (C.c_int, [_P, _I32, _I32, _I32, _I32, _I32, _P, C.c_float, _P, _P, _P]),
    "dqg_prof_begin": (C.c_int, [_I32]),
    "dqg_prof_begin_sampled": (C.c_int, [_I32, _I32]),
    "dqg_prof_end_launches": (C.c_int, [C.POINTER(dqg_prof_launch), _I32, C.POINTER(_I32)]),
    "dqg_prof_end": (C.c_int, [C.POINTER(dqg_prof_record), _I32, C.POINTER(_I32)]),
    "dqg_last_error": (C.c_char_p, []),
    "dqg_stats": (None, [C.POINTER(dqg_counters)]),
    "dqg_stats_reset": (None, []),
}

_lib = None


def library_path() -> str:
    return os.environ.get("DQG_LIBRARY", _build.LIB)


def load() -> C.CDLL:
    """Load libdqg.so (built in-tree by __graft_entry__.build()); raise if absent."""
    global _lib
    if _lib is None:
        path = library_path()
        if not os.path.exists(path):
            raise RuntimeError(f"libdqg.so is not built ({path}); run __graft_entry__.build()")
        lib = C.CDLL(path)
        for name, (res, args) in SIGNATURES.items():
            fn = getattr(lib, name)
            fn.restype = res
            fn.argtypes = args
        _lib = lib
    return _lib


def _check(rc: int) -> None:
    if rc != DQG_OK:
        raise DqgError(rc, load().dqg_last_error().decode())


def _dev(t: Optional[torch.Tensor], name: str, dtype=None):
    if t is None:
        return None
    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise TypeError(f"{name} must be a GPU tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    return t.data_ptr()


def _nbytes(t: torch.Tensor) -> int:
    return t.numel() * t.element_size()


def _need(cond: bool, msg: str) -> None:
    if not cond:
        raise ValueError(msg)


def _same_device(name: str, t: Optional[torch.Tensor], dev: torch.device) -> None:
    if t is not None and t.device != dev:
        raise ValueError(f"{name} is on {t.device}, expected {dev}")


_CODE_BYTES_X8 = {1: 8, 13: 8, 12: 8, 2: 4, 4: 4, 7: 4, 5: 2, 10: 32, 11: 16, 14: 16}   # code bytes per input, x8
_NO_SCALES = (10, 11, 14)


def storage_sizes(fmt: int, O: int, K: int, gs: int):
    """(code bytes, high-plane bytes, scale count) of an [O x K] matrix in format
    ``fmt`` (include/dqg.h's storage table); ValueError for shapes the format
    cannot hold.  fmt 5's code bytes are its 2-bit plane."""
    _need(fmt in _CODE_BYTES_X8, f"unknown format {fmt}")
    _need(O >= 1 and K >= 1, f"O={O} and K={K} must be positive")
    _need(K * _CODE_BYTES_X8[fmt] % 8 == 0, f"K={K} does not fill whole bytes in format {fmt}")
    q = O * K * _CODE_BYTES_X8[fmt] // 8
    if fmt == 5:
        _need(K % 64 == 0, f"K={K} is not a multiple of 64 for format 5")
        return q, O * K // 8, O * (K // 64)
    if fmt in _NO_SCALES:
        return q, 0, 0
    if fmt in (1, 2):
        return q, 0, O
    if fmt == 12:
        _need(K % 128 == 0, f"K={K} is not a multiple of 128 for format 12")
        return q, 0, -(-O // 128) * (K // 128)
    _need(gs >= 1 and K % gs == 0, f"K={K} is not a multiple of gs={gs}")
    return q, 0, O * (K // gs)


def _stream(stream) -> int:
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, torch.cuda.Stream):
        return stream.cuda_stream
    return int(stream)


class Matrix:
    """A resident quantised matrix: device tensors q, q2 (fmt 5), scales
    (None for the formats without scales: 10 f32, 11 bf16, 14 f16)."""

    def __init__(self, fmt: int, O: int, K: int, gs: int, q: torch.Tensor,
                 scales: Optional[torch.Tensor], q2: Optional[torch.Tensor] = None):
        self.fmt, self.O, self.K, self.gs = int(fmt), int(O), int(K), int(gs)
        self.q, self.q2, self.scales = q, q2, scales
        # the kernels read O x K codes through raw pointers: every buffer must hold them
        nq, nq2, ns = storage_sizes(self.fmt, self.O, self.K, self.gs)
        _need(isinstance(q, torch.Tensor) and _nbytes(q) >= nq,
              f"q holds {_nbytes(q) if isinstance(q, torch.Tensor) else 0} bytes, format {fmt} [{O} x {K}] needs {nq}")
        if nq2:
            _need(q2 is not None and _nbytes(q2) >= nq2,
                  f"q2 holds {0 if q2 is None else _nbytes(q2)} bytes, format 5 [{O} x {K}] needs {nq2}")
            _same_device("q2", q2, q.device)
        if ns:
            _need(scales is not None and scales.numel() >= ns,
                  f"scales hold {0 if scales is None else scales.numel()} values, format {fmt} needs {ns}")
            _same_device("scales", scales, q.device)
        else:
            _need(scales is None, f"format {fmt} has no scales (scales must be None)")
        self.struct = dqg_matrix(self.fmt, self.O, self.K, self.gs, _dev(q, "q"),
                                 _dev(q2, "q2"), _dev(scales, "scales", torch.float32))

    @classmethod
    def upload(cls, m, device="cuda") -> "Matrix":
        """Copy a host matrix (fields fmt, O, K, gs, q, q2, scales as numpy) to the GPU."""
        def to(a):
            if a is None:
                return None
            if a.dtype == np.uint16:   # bf16 / f16 bits: same bytes, a dtype torch copies everywhere
                a = a.view(np.int16)
            return torch.from_numpy(np.ascontiguousarray(a)).to(device)
        return cls(m.fmt, m.O, m.K, m.gs, to(m.q), to(m.scales), to(m.q2))

    @property
    def nbytes(self) -> int:
        n = self.q.numel() * self.q.element_size() + (0 if self.scales is None else self.scales.numel() * 4)
        if self.q2 is not None:
            n += self.q2.numel() * self.q2.element_size()
        return n


def _tokens(x: torch.Tensor, K: int, name: str = "x") -> int:
    """S of an activation tensor x [S][K] (S >= 1)."""
    _need(isinstance(x, torch.Tensor) and x.dim() == 2 and x.shape[0] >= 1 and x.shape[1] == K,
          f"{name} must be [S][{K}] with S >= 1, got {tuple(x.shape) if isinstance(x, torch.Tensor) else type(x)}")
    return int(x.shape[0])


def _out(t: Optional[torch.Tensor], n: int, name: str, dev: torch.device) -> None:
    if t is not None:
        _need(isinstance(t, torch.Tensor) and t.numel() >= n, f"{name} holds {t.numel()} values, {n} needed")
        _same_device(name, t, dev)


def dqg_matmul(W: Matrix, x: torch.Tensor, y: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    S = _tokens(x, W.K)
    _same_device("x", x, W.q.device)
    _out(y, S * W.O, "y", x.device)
    if y is None:
        y = torch.empty((S, W.O), dtype=torch.float32, device=x.device)
    _check(load().dqg_matmul(C.byref(W.struct), _dev(x, "x", torch.float32), S,
                             _dev(y, "y", torch.float32), _stream(stream)))
    return y


def _gate_up_shapes(G: Matrix, U: Matrix, x: torch.Tensor, h: Optional[torch.Tensor]) -> int:
    _need((G.O, G.K) == (U.O, U.K), f"gate [{G.O} x {G.K}] and up [{U.O} x {U.K}] differ")
    S = _tokens(x, G.K)
    _same_device("x", x, G.q.device)
    _same_device("up", U.q, G.q.device)
    _out(h, S * G.O, "h", x.device)
    return S


def dqg_gate_up(G: Matrix, U: Matrix, x: torch.Tensor, h: Optional[torch.Tensor] = None,
                stream=None) -> torch.Tensor:
    S = _gate_up_shapes(G, U, x, h)
    if h is None:
        h = torch.empty((S, G.O), dtype=torch.float32, device=x.device)
    _check(load().dqg_gate_up(C.byref(G.struct), C.byref(U.struct), _dev(x, "x", torch.float32), S,
                              _dev(h, "h", torch.float32), _stream(stream)))
    return h


def dqg_gate_up_clamped(G: Matrix, U: Matrix, x: torch.Tensor, limit: float, h: Optional[torch.Tensor] = None,
                        stream=None) -> torch.Tensor:
    S = _gate_up_shapes(G, U, x, h)
    if h is None:
        h = torch.empty((S, G.O), dtype=torch.float32, device=x.device)
    _check(load().dqg_gate_up_clamped(C.byref(G.struct), C.byref(U.struct), _dev(x, "x", torch.float32), S,
                                      float(limit), _dev(h, "h", torch.float32), _stream(stream)))
    return h


def dqg_dequant(W: Matrix, out: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    _out(out, W.O * W.K, "out", W.q.device)
    if out is None:
        out = torch.empty((W.O, W.K), dtype=torch.float32, device=W.q.device)
    _check(load().dqg_dequant(C.byref(W.struct), _dev(out, "out", torch.float32), _stream(stream)))
    return out


def dqg_read_bytes(buf: torch.Tensor, sink: torch.Tensor, nbytes: Optional[int] = None, offset: int = 0,
                   stream=None) -> None:
    """A plain streaming read of nbytes of buf from byte `offset` (the
    measurement ceiling; see dqg.h).  sink: a GPU int32 tensor of one word."""
    n = _nbytes(buf) - offset if nbytes is None else nbytes
    if offset < 0 or n <= 0 or offset + n > _nbytes(buf):
        raise ValueError(f"read_bytes: [{offset}, {offset + n}) outside the buffer's {_nbytes(buf)} bytes")
    _dev(buf, "buf")
    _check(load().dqg_read_bytes(C.c_void_p(buf.data_ptr() + offset), n, _dev(sink, "sink", torch.int32),
                                 _stream(stream)))


class Expert:
    def __init__(self, gate: Matrix, up: Matrix, down: Matrix):
        self.gate, self.up, self.down = gate, up, down

    @classmethod
    def upload(cls, e, device="cuda") -> "Expert":
        return cls(Matrix.upload(e.gate, device), Matrix.upload(e.up, device), Matrix.upload(e.down, device))

    @property
    def nbytes(self) -> int:
        return self.gate.nbytes + self.up.nbytes + self.down.nbytes


class ExpertTable:
    """dqg_expert_table_create / _destroy.  Keeps the experts' tensors alive."""

    def __init__(self, experts: Sequence[Expert]):
        self.experts = list(experts)
        arr = (dqg_expert * len(self.experts))(*[dqg_expert(e.gate.struct, e.up.struct, e.down.struct)
                                                  for e in self.experts])
        handle = C.c_void_p()
        _check(load().dqg_expert_table_create(arr, len(self.experts), C.byref(handle)))
        self.handle = handle
        self.H = self.experts[0].gate.K
        self.I = self.experts[0].gate.O

    def close(self) -> None:
        if self.handle:
            load().dqg_expert_table_destroy(self.handle)
            self.handle = C.c_void_p()

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def set_swiglu_limit(self, limit: float) -> None:
        """dqg_expert_table_set_swiglu_limit (math.inf: the plain SwiGLU)."""
        _check(load().dqg_expert_table_set_swiglu_limit(self.handle, float(limit)))

    def set_activation(self, act: int) -> None:
        """dqg_expert_table_set_activation: DQG_ACT_SWIGLU or DQG_ACT_SWIGLU_V4."""
        _check(load().dqg_expert_table_set_activation(self.handle, int(act)))

    def scratch_bytes(self, S: int, k: int) -> int:
        return load().dqg_expert_group_scratch_bytes(self.handle, S, k)

    def scratch(self, S: int, k: int, device="cuda") -> torch.Tensor:
        """Scratch for calls of up to S tokens (it needs no initialisation)."""
        return torch.empty(self.scratch_bytes(S, k), dtype=torch.uint8, device=device)


def _group_args(table: ExpertTable, ids, w, shared, x, y, scratch):
    _need(isinstance(ids, torch.Tensor) and ids.dim() == 2 and ids.shape[0] >= 1 and ids.shape[1] >= 1,
          "ids must be [S][k] with S, k >= 1")
    S, k = (int(v) for v in ids.shape)
    _need(isinstance(w, torch.Tensor) and tuple(w.shape) == (S, k), f"w must be [{S}][{k}] like ids")
    _need(_tokens(x, table.H) == S, f"x must hold S={S} tokens (one per row of ids)")
    dev = x.device
    for name, t in (("ids", ids), ("w", w)):
        _same_device(name, t, dev)
    _out(y, S * table.H, "y", dev)
    if scratch is not None:
        _same_device("scratch", scratch, dev)
    if y is None:
        y = torch.empty((S, table.H), dtype=torch.float32, device=x.device)
    if scratch is None:
        scratch = table.scratch(S, k, x.device)
    args = (table.handle, S, k, _dev(ids, "ids", torch.int32), _dev(w, "w", torch.float32),
            -1 if shared is None else int(shared), _dev(x, "x", torch.float32),
            _dev(y, "y", torch.float32), _dev(scratch, "scratch"),
            scratch.numel() * scratch.element_size())
    return args, y, scratch


def dqg_expert_group(table: ExpertTable, ids: torch.Tensor, w: torch.Tensor, shared: Optional[int],
                     x: torch.Tensor, y: Optional[torch.Tensor] = None,
                     scratch: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    args, y, _ = _group_args(table, ids, w, shared, x, y, scratch)
    _check(load().dqg_expert_group(*args, _stream(stream)))
    return y


def dqg_expert_group_noalloc(table: ExpertTable, ids: torch.Tensor, w: torch.Tensor, shared: Optional[int],
                             x: torch.Tensor, y: torch.Tensor, stream=None) -> torch.Tensor:
    """dqg_expert_group on the library's static per-device scratch: y must be given
    (nothing is allocated on the path)."""
    _need(y is not None, "y must be given: this call allocates nothing")
    args, y, _ = _group_args(table, ids, w, shared, x, y, torch.empty(0, dtype=torch.uint8, device=x.device))
    _check(load().dqg_expert_group_noalloc(*args[:8], _stream(stream)))
    return y


def dqg_expert_group_issue(table: ExpertTable, ids: torch.Tensor, w: torch.Tensor,
                           shared: Optional[int], x: torch.Tensor, y: Optional[torch.Tensor] = None,
                           scratch: Optional[torch.Tensor] = None, stream=None):
    """Returns (ticket, y, scratch); keep scratch alive until the ticket is taken."""
    args, y, scratch = _group_args(table, ids, w, shared, x, y, scratch)
    ticket = dqg_ticket()
    _check(load().dqg_expert_group_issue(*args, _stream(stream), C.byref(ticket)))
    return ticket, y, scratch


def dqg_expert_group_take(ticket: dqg_ticket) -> None:
    _check(load().dqg_expert_group_take(C.byref(ticket)))


def dqg_route(logits: torch.Tensor, k: int, mode: int = DQG_ROUTE_SOFTMAX, renorm: bool = False,
              bias: Optional[torch.Tensor] = None, w_scale: float = 1.0,
              ids: Optional[torch.Tensor] = None, w: Optional[torch.Tensor] = None, stream=None):
    """Router on the device: returns (ids int32 [S][k], w f32 [S][k])."""
    _need(isinstance(logits, torch.Tensor) and logits.dim() == 2, "logits must be [S][E]")
    S, E = (int(v) for v in logits.shape)
    dev = logits.device
    if bias is not None:
        _need(bias.numel() == E, f"bias must hold E={E} values")
        _same_device("bias", bias, dev)
    _out(ids, S * int(k), "ids", dev)
    _out(w, S * int(k), "w", dev)
    if ids is None:
        ids = torch.empty((S, k), dtype=torch.int32, device=logits.device)
    if w is None:
        w = torch.empty((S, k), dtype=torch.float32, device=logits.device)
    _check(load().dqg_route(_dev(logits, "logits", torch.float32), S, E, int(k), int(mode), int(bool(renorm)),
                            _dev(bias, "bias", torch.float32), float(w_scale),
                            _dev(ids, "ids", torch.int32), _dev(w, "w", torch.float32), _stream(stream)))
    return ids, w


def dqg_last_error() -> str:
    return load().dqg_last_error().decode()


def dqg_stats() -> dict:
    c = dqg_counters()
    load().dqg_stats(C.byref(c))
    return {name: getattr(c, name) for name, _ in dqg_counters._fields_}


def dqg_stats_reset() -> None:
    load().dqg_stats_reset()


def dqg_prof_begin(capacity: int) -> None:
    """Time the next ``capacity`` launches with HIP events on their streams."""
    _check(load().dqg_prof_begin(int(capacity)))


def dqg_prof_begin_sampled(capacity: int, every: int) -> None:
    """Time the launches of every `every`-th call, up to `capacity` launches (host-blocking setup)."""
    _check(load().dqg_prof_begin_sampled(int(capacity), int(every)))


def dqg_prof_end_launches(capacity: int) -> list:
    """[(kernel name, device ms)] of the timed launches in launch order (up to ``capacity``)."""
    recs = (dqg_prof_launch * max(1, int(capacity)))()
    n = C.c_int32()
    _check(load().dqg_prof_end_launches(recs, len(recs), C.byref(n)))
    return [(recs[i].kernel.decode(), recs[i].ms) for i in range(n.value)]


def dqg_prof_end() -> dict:
    """{kernel name: (launches, total device ms)} of the launches timed since dqg_prof_begin."""
    recs = (dqg_prof_record * 16)()
    n = C.c_int32()
    _check(load().dqg_prof_end(recs, 16, C.byref(n)))
    return {recs[i].kernel.decode(): (recs[i].launches, recs[i].total_ms) for i in range(n.value)}
