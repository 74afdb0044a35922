"""Seeded synthetic inputs for the quantised GEMV / expert-MLP path.

This module is shared by the tests, the benchmark and the oracle's callers.
It only draws random storage words, scales, activations and routings with
the shapes and value distributions of the workloads; it holds none of the
method's arithmetic (no decoding, no dot products, no activation).

Storage forms (one per weight format; the format numbers are colibri's
device formats as listed in the expert-tier engine table of "colibri --
Vulkan backend (docs/vulkan.md)"):

  fmt 1  int8, one f32 scale per row
         q: int8 [O][K]                     scales: f32 [O][1]
  fmt 2  int4 pairs, one f32 scale per row
         q: uint8 [O][K/2]                  scales: f32 [O][1]
  fmt 4  int4 pairs, one f32 scale per gs inputs
         q: uint8 [O][K/2]                  scales: f32 [O][K/gs]
  fmt 5  int3, one group per 64 inputs, two bit planes
         q: uint32 [O][K/16] (2-bit plane)  q2: uint32 [O][K/32] (1-bit plane)
         scales: f32 [O][K/64]
  fmt 7  MXFP4: e2m1 nibbles, f32 scale per 32 inputs (pre-expanded e8m0)
         q: uint8 [O][K/2]                  scales: f32 [O][K/32]
  fmt 10 f32 rows, no scales
         q: float32 [O][K]                  scales: None
  fmt 11 bf16 rows, no scales
         q: uint16 [O][K] (bf16 bits)       scales: None
  fmt 12 FP8 E4M3, one f32 scale per block of 128 rows x 128 inputs
         q: uint8 [O][K] (E4M3 bits)        scales: f32 [ceil(O/128)][K/128]
  fmt 13 int8, one f32 scale per gs inputs (gs 64 by default)
         q: int8 [O][K]                     scales: f32 [O][K/gs]
  fmt 14 f16 rows, no scales
         q: uint16 [O][K] (f16 bits)        scales: None

Uniform random words give uniform codes in every field, so drawing words is
the same as drawing codes; no bit of any code is computed here.  The float
forms draw their fields (sign, exponent field in a weight-like range,
uniform fraction) and place them in the word; E4M3 draws a sign and a
non-NaN magnitude byte.
"""
from __future__ import annotations

import dataclasses
from concurrent.futures import ThreadPoolExecutor
from typing import Optional

import numpy as np

FMT_I8_ROW = 1
FMT_I4_ROW = 2
FMT_I4_GS = 4
FMT_I3_G64 = 5
FMT_MXFP4 = 7
FMT_F32 = 10
FMT_BF16 = 11
FMT_FP8_BLOCK = 12
FMT_I8_GS = 13
FMT_F16 = 14

FORMATS = (FMT_I8_ROW, FMT_I4_ROW, FMT_I4_GS, FMT_I3_G64, FMT_MXFP4,
           FMT_F32, FMT_BF16, FMT_FP8_BLOCK, FMT_I8_GS, FMT_F16)
NO_SCALE_FORMATS = (FMT_F32, FMT_BF16, FMT_F16)
FP8_BLOCK = 128   # rows and inputs per E4M3 scale block

BASE_SEED = 20261202


@dataclasses.dataclass
class QMatrix:
    """Host copy of one quantised matrix in its storage form."""
    fmt: int
    O: int
    K: int
    gs: int
    q: np.ndarray
    q2: Optional[np.ndarray]
    scales: Optional[np.ndarray]   # None for the formats without scales

    @property
    def nbytes(self) -> int:
        n = self.q.nbytes + (0 if self.scales is None else self.scales.nbytes)
        if self.q2 is not None:
            n += self.q2.nbytes
        return n


def group_size(fmt: int, K: int, gs: Optional[int] = None) -> int:
    """Inputs per scale for a format (the whole row for the per-row forms
    and for the forms without scales)."""
    if fmt in (FMT_I8_ROW, FMT_I4_ROW) or fmt in NO_SCALE_FORMATS:
        return K
    if fmt == FMT_FP8_BLOCK:
        return FP8_BLOCK
    if fmt == FMT_I8_GS:
        return 64 if gs is None else gs
    if fmt == FMT_I3_G64:
        return 64
    if fmt == FMT_MXFP4:
        return 32
    if fmt == FMT_I4_GS:
        if gs is None:
            raise ValueError("fmt 4 needs a group size")
        return gs
    raise ValueError(f"unknown format {fmt}")


def storage_shapes(fmt: int, O: int, K: int, gs: int):
    """(q shape, q dtype, q2 shape or None, scales shape) of a format."""
    if fmt == FMT_I8_ROW:
        return (O, K), np.int8, None, (O, 1)
    if fmt in (FMT_I4_ROW, FMT_I4_GS, FMT_MXFP4):
        return (O, K // 2), np.uint8, None, (O, K // gs)
    if fmt == FMT_I3_G64:
        return (O, K // 16), np.uint32, (O, K // 32), (O, K // 64)
    if fmt == FMT_F32:
        return (O, K), np.float32, None, None
    if fmt in (FMT_BF16, FMT_F16):
        return (O, K), np.uint16, None, None
    if fmt == FMT_FP8_BLOCK:
        return (O, K), np.uint8, None, (-(-O // FP8_BLOCK), K // FP8_BLOCK)
    if fmt == FMT_I8_GS:
        return (O, K), np.int8, None, (O, K // gs)
    raise ValueError(f"unknown format {fmt}")


def rng_for(*key: int) -> np.random.Generator:
    """Independent PCG64 stream for a tuple of integers (seed, ids...)."""
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence(list(key))))


def _scales(rng: np.random.Generator, fmt: int, shape, kind: str) -> np.ndarray:
    if kind == "pow2_small":
        # powers of two 2^-5 and 2^-4 (with activations on a coarse grid,
        # products and sums that stay exact in f32)
        e = rng.integers(-5, -3, size=shape)
        return np.ldexp(np.ones(shape, dtype=np.float32), e).astype(np.float32)
    if kind == "pow2":
        # e8m0 scales pre-expanded to f32: 2^e with e uniform in {-10..-6}
        e = rng.integers(-10, -5, size=shape)
        return np.ldexp(np.ones(shape, dtype=np.float32), e).astype(np.float32)
    if kind == "row_int8":
        lo, hi = 1e-3, 1e-2
    elif kind == "fp8_block":   # E4M3's largest magnitude 448 maps to about 0.01 to 0.05
        lo, hi = 2e-5, 1e-4
    else:
        lo, hi = 1e-3, 2e-2
    return rng.uniform(lo, hi, size=shape).astype(np.float32)


def default_scale_kind(fmt: int) -> str:
    if fmt in (FMT_I8_ROW, FMT_I8_GS):
        return "row_int8"
    if fmt == FMT_FP8_BLOCK:
        return "fp8_block"
    if fmt == FMT_MXFP4:
        return "pow2"
    return "uniform"


def matrix(fmt: int, O: int, K: int, gs: Optional[int], *key: int,
           scale_kind: Optional[str] = None) -> QMatrix:
    """Draw one quantised matrix from the stream named by ``key``.

    int8 codes are uniform in [-127, 127]; int4, int3 and MXFP4 fields are
    uniform over all their codes.  f32 rows are N(0, 0.02); bf16 and f16
    rows have a uniform sign, an exponent of 2^-12 .. 2^-3 and a uniform
    fraction; E4M3 codes have a uniform sign and a uniform non-NaN
    magnitude.  Scales: int8 rows and groups U[1e-3, 1e-2], int4 and int3
    groups U[1e-3, 2e-2], MXFP4 powers of two 2^U{-10..-6}, E4M3 blocks
    U[2e-5, 1e-4].
    """
    gs = group_size(fmt, K, gs)
    if K % gs:
        raise ValueError("K must be a multiple of the group size")
    qshape, qdtype, q2shape, sshape = storage_shapes(fmt, O, K, gs)
    rng = rng_for(*key)
    if fmt in (FMT_I8_ROW, FMT_I8_GS):
        q = rng.integers(-127, 128, size=qshape, dtype=np.int8)
    elif fmt == FMT_F32:
        q = (rng.standard_normal(size=qshape) * 0.02).astype(np.float32)
    elif fmt in (FMT_BF16, FMT_F16):
        mbits, bias = (7, 127) if fmt == FMT_BF16 else (10, 15)
        sign = rng.integers(0, 2, size=qshape, dtype=np.uint16)
        expo = rng.integers(bias - 12, bias - 2, size=qshape).astype(np.uint16)
        frac = rng.integers(0, 1 << mbits, size=qshape, dtype=np.uint16)
        q = (sign << np.uint16(15)) | (expo << np.uint16(mbits)) | frac
    elif fmt == FMT_FP8_BLOCK:
        sign = rng.integers(0, 2, size=qshape, dtype=np.uint8)
        mag = rng.integers(0, 0x7F, size=qshape, dtype=np.uint8)   # 0x7F is NaN
        q = (sign << np.uint8(7)) | mag
    elif qdtype == np.uint8:
        q = rng.integers(0, 256, size=qshape, dtype=np.uint8)
    else:
        q = rng.integers(0, 2**32, size=qshape, dtype=np.uint32)
    q2 = None
    if q2shape is not None:
        q2 = rng.integers(0, 2**32, size=q2shape, dtype=np.uint32)
    s = None if sshape is None else _scales(rng, fmt, sshape, scale_kind or default_scale_kind(fmt))
    return QMatrix(fmt, O, K, gs, q, q2, s)


def activations(S: int, K: int, *key: int) -> np.ndarray:
    """x[S][K] f32, entries N(0, 1)."""
    return rng_for(*key).standard_normal(size=(S, K)).astype(np.float32)


def activations_e4m3_grid(S: int, K: int, *key: int, max_exp: int = 1) -> np.ndarray:
    """x[S][K] f32 on the E4M3 grid: a uniform sign, fraction 1.000b .. 1.111b
    and exponent 2^-3 .. 2^max_exp (so |x| in [1/8, 1.875 * 2^max_exp],
    multiples of 2^-6), and one entry in ten zero: activations as an engine
    hands them over after rounding them to E4M3 itself."""
    rng = rng_for(*key)
    mant = rng.integers(8, 16, size=(S, K))
    expo = rng.integers(-3, max_exp + 1, size=(S, K))
    sign = rng.choice([-1.0, 1.0], size=(S, K))
    x = sign * np.ldexp(mant.astype(np.float64), expo - 3)
    x[rng.random((S, K)) < 0.1] = 0.0
    return x.astype(np.float32)


def routing(S: int, n_experts: int, k: int, *key: int):
    """Top-k routing of S tokens.

    ids[t]: k expert indices drawn uniformly without replacement.
    w[t]: softmax of the token's k standard-normal logits (f64, shifted by
    the max, stored f32).  These stand in for a router's output.
    """
    rng = rng_for(*key)
    ids = np.empty((S, k), dtype=np.int32)
    w = np.empty((S, k), dtype=np.float32)
    for t in range(S):
        ids[t] = rng.choice(n_experts, size=k, replace=False)
        logits = rng.standard_normal(k)
        e = np.exp(logits - logits.max())
        w[t] = (e / e.sum()).astype(np.float32)
    return ids, w


def router_logits(S: int, n_experts: int, *key: int, spread: float = 2.0) -> np.ndarray:
    """Router logits [S][E] f32: spread * N(0, 1), a stand-in for a router
    projection's output (the workloads' real routers are not available)."""
    rng = rng_for(*key)
    return (rng.standard_normal((S, n_experts)) * spread).astype(np.float32)


def router_bias(n_experts: int, *key: int, spread: float = 0.05) -> np.ndarray:
    """A picking bias [E] f32, uniform in [-spread, spread]."""
    rng = rng_for(*key)
    return rng.uniform(-spread, spread, n_experts).astype(np.float32)


@dataclasses.dataclass
class Expert:
    gate: QMatrix   # [I x H]
    up: QMatrix     # [I x H]
    down: QMatrix   # [H x I]


def expert(fmt: int, H: int, I: int, gs: Optional[int], seed: int, index: int,
           down_fmt: Optional[int] = None, down_gs: Optional[int] = None,
           scale_kind: Optional[str] = None) -> Expert:
    """Expert ``index`` of a seeded set: gate, up [I x H] and down [H x I]."""
    dfmt = fmt if down_fmt is None else down_fmt
    dgs = gs if down_gs is None else down_gs
    if dfmt in (FMT_I8_ROW, FMT_I4_ROW) or dfmt in NO_SCALE_FORMATS or dfmt == FMT_FP8_BLOCK:
        dgs = None
    return Expert(matrix(fmt, I, H, gs, seed, index, 0, scale_kind=scale_kind),
                  matrix(fmt, I, H, gs, seed, index, 1, scale_kind=scale_kind),
                  matrix(dfmt, H, I, dgs, seed, index, 2, scale_kind=scale_kind))


def experts(fmt: int, H: int, I: int, gs: Optional[int], seed: int, n: int,
            threads: int = 8, **kw) -> list:
    """n experts, drawn in parallel (each from its own stream)."""
    with ThreadPoolExecutor(max(1, threads)) as ex:
        return list(ex.map(lambda i: expert(fmt, H, I, gs, seed, i, **kw), range(n)))


# Workloads.  Shapes and distributions of the five configurations the path
# is measured on; seeds are BASE_SEED + workload index.
WORKLOADS = {
    "int8_gemv_256x512": dict(kind="gemv", fmt=FMT_I8_ROW, O=256, K=512, gs=None, S=(1,), seed=BASE_SEED + 0),
    "int4g32_gemv_6144x6144": dict(kind="gemv", fmt=FMT_I4_GS, O=6144, K=6144, gs=32, S=(1, 4), seed=BASE_SEED + 1),
    "int4g32_expert_6144x2048": dict(kind="expert", fmt=FMT_I4_GS, H=6144, I=2048, gs=32, S=(1,), seed=BASE_SEED + 2),
    "int4g32_expert_group_256top8_shared": dict(kind="group", fmt=FMT_I4_GS, H=6144, I=2048, gs=32, E=256, k=8,
                                                shared=True, S=(1, 2, 4), seed=BASE_SEED + 3),
    "mxfp4_expert_group_384top8_s8": dict(kind="group", fmt=FMT_MXFP4, H=7168, I=2048, gs=32, E=384, k=8,
                                          shared=False, S=(8,), seed=BASE_SEED + 4),
    "int3g64_gemv_6144x16384": dict(kind="gemv", fmt=FMT_I3_G64, O=6144, K=16384, gs=64, S=(1,), seed=BASE_SEED + 5),
    # the other device formats on the dense 6144 x 6144 shape
    "f32_gemv_6144x6144": dict(kind="gemv", fmt=FMT_F32, O=6144, K=6144, gs=None, S=(1, 4), seed=BASE_SEED + 6),
    "bf16_gemv_6144x6144": dict(kind="gemv", fmt=FMT_BF16, O=6144, K=6144, gs=None, S=(1, 4), seed=BASE_SEED + 7),
    "fp8b128_gemv_6144x6144": dict(kind="gemv", fmt=FMT_FP8_BLOCK, O=6144, K=6144, gs=None, S=(1, 4),
                                   seed=BASE_SEED + 8),
    "int8gs64_gemv_6144x6144": dict(kind="gemv", fmt=FMT_I8_GS, O=6144, K=6144, gs=64, S=(1, 4), seed=BASE_SEED + 9),
    "f16_gemv_6144x6144": dict(kind="gemv", fmt=FMT_F16, O=6144, K=6144, gs=None, S=(1, 4), seed=BASE_SEED + 10),
    # E4M3 experts in 128 x 128 blocks on the expert-group shape
    "fp8b128_expert_group_256top8_shared": dict(kind="group", fmt=FMT_FP8_BLOCK, H=6144, I=2048, gs=None, E=256,
                                                k=8, shared=True, S=(1, 2, 4), seed=BASE_SEED + 11),
    "fp8b128_expert_6144x2048": dict(kind="expert", fmt=FMT_FP8_BLOCK, H=6144, I=2048, gs=None, S=(1,),
                                     seed=BASE_SEED + 12),
}
