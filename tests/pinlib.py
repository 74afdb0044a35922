"""Pins of the CPU oracle: checks against what the pages and mathematics fix.

Each ``pin_*`` function takes an ``oracle.OracleLib`` and raises
AssertionError when the oracle disagrees with:
  - hand-written fixtures under tests/golden/ (code tables and byte layouts,
    each citing the passage or reading it follows);
  - closed forms (constant codes, one-hot inputs, zero scales, powers of two);
  - exact rational brute force on tiny inputs;
  - a library routine where the operation reduces to one (scipy's expit);
  - invariants of the expert group (zero weights, one expert, permutations).
The same pins run against source-patched mutants of the oracle in
test_oracle_mutants.py, each of which some pin must reject.
"""
from __future__ import annotations

import math
import os
from fractions import Fraction

import numpy as np

import synth

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


# ---------------------------------------------------------------------------
# fixtures
# ---------------------------------------------------------------------------

def _rows(name):
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.split("#", 1)[0].strip()
            if line:
                yield line.split()


def golden_e2m1():
    return {int(r[0]): float(r[2]) for r in _rows("e2m1_values.txt")}


def golden_pairs(name):
    """[(byte, value_even, value_odd)] from a pair fixture."""
    return [(int(r[0], 16), float(r[1]), float(r[2])) for r in _rows(name)]


def golden_int8():
    return [(int(r[0], 16), int(r[1])) for r in _rows("int8_rows.txt")]


def golden_int3():
    low, high, values = None, None, []
    for r in _rows("int3_planes.txt"):
        if r[0] == "low":
            low = [int(v, 16) for v in r[1:]]
        elif r[0] == "high":
            high = [int(v, 16) for v in r[1:]]
        elif r[0] == "values":
            values += [int(v) for v in r[1:]]
    return low, high, values


def golden_minifloats():
    """{kind: [(code, value)]} from the hand-written float code table."""
    out = {}
    for kind, code, val in _rows("minifloat_values.txt"):
        v = float.fromhex(val) if "0x" in val else float(val)
        out.setdefault(kind, []).append((int(code, 16), v))
    return out


def _same_bits(a, b) -> bool:
    if math.isnan(a) or math.isnan(b):
        return math.isnan(a) and math.isnan(b)
    return np.float64(a).tobytes() == np.float64(b).tobytes()


def _same_values(a, b) -> bool:
    """Arrays equal element by element, NaN matching NaN and -0 only -0."""
    a, b = np.asarray(a, np.float64), np.asarray(b, np.float64)
    na, nb = np.isnan(a), np.isnan(b)
    if not np.array_equal(na, nb):
        return False
    return a[~na].tobytes() == b[~nb].tobytes()


def _qm(fmt, O, K, gs, q, scales, q2=None):
    return synth.QMatrix(fmt, O, K, gs, np.ascontiguousarray(q),
                         None if q2 is None else np.ascontiguousarray(q2),
                         None if scales is None else np.ascontiguousarray(scales, dtype=np.float32))


# ---------------------------------------------------------------------------
# decode: code tables and layouts
# ---------------------------------------------------------------------------

def pin_e2m1_table(lib):
    table = golden_e2m1()
    assert len(table) == 16
    for code, val in table.items():
        got = lib.e2m1(code)
        assert _same_bits(got, val), f"e2m1({code}) = {got!r}, expected {val!r}"


def pin_int4_pairs(lib):
    for fmt in (synth.FMT_I4_GS, synth.FMT_I4_ROW):
        rows = golden_pairs("int4_pairs.txt")
        q = np.array([[b for b, _, _ in rows]], dtype=np.uint8)
        K = 2 * q.shape[1]
        m = _qm(fmt, 1, K, K, q, np.ones((1, 1), np.float32))
        got = lib.code_values(m)[0]
        want = np.array([v for _, a, b in rows for v in (a, b)])
        assert np.array_equal(got, want), f"fmt {fmt}: {got} != {want}"


def pin_mxfp4_pairs(lib):
    rows = golden_pairs("mxfp4_pairs.txt")
    pad = (-len(rows)) % 16                 # whole groups of 32 inputs
    q = np.array([[b for b, _, _ in rows] + [0] * pad], dtype=np.uint8)
    K = 2 * q.shape[1]
    m = _qm(synth.FMT_MXFP4, 1, K, 32, q, np.ones((1, K // 32), np.float32))
    got = lib.code_values(m)[0]
    want = [v for _, a, b in rows for v in (a, b)]
    for k, v in enumerate(want):
        assert _same_bits(got[k], v), f"k={k}: {got[k]!r} != {v!r}"


def pin_int8_rows(lib):
    rows = golden_int8()
    q = np.array([[b for b, _ in rows]], dtype=np.uint8).view(np.int8)
    m = _qm(synth.FMT_I8_ROW, 1, q.shape[1], q.shape[1], q, np.ones((1, 1), np.float32))
    got = lib.code_values(m)[0]
    assert np.array_equal(got, [v for _, v in rows]), got


def pin_int3_planes(lib):
    low, high, values = golden_int3()
    m = _qm(synth.FMT_I3_G64, 1, 64, 64, np.array([low], dtype=np.uint32),
            np.ones((1, 1), np.float32), q2=np.array([high], dtype=np.uint32))
    got = lib.code_values(m)[0]
    assert np.array_equal(got, values), f"{got} != {values}"


def pin_exhaustive_codes(lib):
    """Every code of every format decodes to its closed form (value * 1)."""
    # int8: all 256 bytes, two's complement
    q = np.arange(256, dtype=np.uint8).view(np.int8).reshape(1, 256)
    m = _qm(1, 1, 256, 256, q, np.ones((1, 1), np.float32))
    assert np.array_equal(lib.code_values(m)[0], np.arange(256, dtype=np.uint8).view(np.int8))
    # int4: byte b holds (b & 15, b >> 4) -> all 256 combinations
    q = np.arange(256, dtype=np.uint8).reshape(1, 256)
    m = _qm(4, 1, 512, 32, q, np.ones((1, 16), np.float32))
    v = lib.code_values(m)[0]
    b = np.arange(256)
    assert np.array_equal(v[0::2], (b & 15) - 8) and np.array_equal(v[1::2], (b >> 4) - 8)
    # int3: each of the 8 codes at each of the 64 positions of a group
    for code in range(8):
        lo_word = (code & 3) * 0x55555555
        hi_word = 0xFFFFFFFF if code & 4 else 0
        m = _qm(5, 1, 64, 64, np.full((1, 4), lo_word, np.uint32), np.ones((1, 1), np.float32),
                q2=np.full((1, 2), hi_word, np.uint32))
        assert np.array_equal(lib.code_values(m)[0], np.full(64, code - 4)), code


_FLOAT_FMT = {"e4m3": (synth.FMT_FP8_BLOCK, np.uint8), "f16": (synth.FMT_F16, np.uint16),
              "bf16": (synth.FMT_BF16, np.uint16)}


def _float_row(kind, codes):
    """One row of a float format holding ``codes`` (padded to a whole block)."""
    fmt, dt = _FLOAT_FMT[kind]
    K = max(128, -(-len(codes) // 128) * 128)
    q = np.zeros((1, K), dt)
    q[0, :len(codes)] = codes
    scales = np.ones((1, K // 128), np.float32) if fmt == synth.FMT_FP8_BLOCK else None
    return _qm(fmt, 1, K, 128 if fmt == synth.FMT_FP8_BLOCK else K, q, scales)


def pin_minifloat_table(lib):
    """E4M3, f16 and bf16 codes decode to the hand-written table, through the
    field decoder and through a matrix row of each format."""
    ieee = {"e4m3": (4, 3, False), "f16": (5, 10, True), "bf16": (8, 7, True)}
    for kind, rows in golden_minifloats().items():
        for code, val in rows:
            got = lib.minifloat(code, *ieee[kind])
            assert _same_bits(got, val), f"{kind} {code:#x}: {got!r} != {val!r}"
        m = _float_row(kind, [c for c, _ in rows])
        got = lib.code_values(m)[0, :len(rows)]
        assert _same_values(got, [v for _, v in rows]), f"{kind} row: {got}"


def pin_float_formats_exhaustive(lib):
    """Every code of the float formats against a library decode: numpy's
    binary16 for f16, numpy's binary32 of the code in the upper half for
    bf16, torch's float8_e4m3fn for E4M3; f32 rows are their own values."""
    import torch
    f16 = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    assert _same_values(lib.code_values(_float_row("f16", f16))[0], f16.view(np.float16).astype(np.float64))
    bf = np.arange(65536, dtype=np.uint32)
    with np.errstate(invalid="ignore"):   # signalling NaNs widen quietly
        want = (bf << np.uint32(16)).view(np.float32).astype(np.float64)
    assert _same_values(lib.code_values(_float_row("bf16", bf.astype(np.uint16)))[0], want)
    e = np.arange(256, dtype=np.uint8)
    want = torch.from_numpy(e.copy()).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    assert _same_values(lib.code_values(_float_row("e4m3", e))[0, :256], want)
    # f32: random words with the special values mixed in
    w = synth.rng_for(12, 10).integers(0, 2**32, size=(2, 64), dtype=np.uint64).astype(np.uint32)
    w[0, :6] = [0x00000000, 0x80000000, 0x7F800000, 0xFF800000, 0x00000001, 0x7F7FFFFF]
    m = _qm(synth.FMT_F32, 2, 64, 64, w.view(np.float32), None)
    assert _same_values(lib.code_values(m), w.view(np.float32).astype(np.float64))


# ---------------------------------------------------------------------------
# an independent NumPy decoder (vectorised), pinned to the same fixtures,
# used to check the oracle's row and word indexing on large random matrices
# ---------------------------------------------------------------------------

def numpy_values(m) -> np.ndarray:
    O, K = m.O, m.K
    if m.fmt in (1, 13, 10):
        return m.q.astype(np.float64)
    if m.fmt == 11:
        return (m.q.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)
    if m.fmt == 14:
        return m.q.view(np.float16).astype(np.float64)
    if m.fmt == 12:
        import torch
        return torch.from_numpy(np.ascontiguousarray(m.q)).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    if m.fmt in (2, 4, 7):
        lo = (m.q & 0x0F).astype(np.int64)
        hi = (m.q >> 4).astype(np.int64)
        nib = np.stack([lo, hi], axis=-1).reshape(O, K)
        if m.fmt == 7:
            table = golden_e2m1()
            return np.vectorize(lambda c: table[int(c)])(nib).astype(np.float64)
        return (nib - 8).astype(np.float64)
    if m.fmt == 5:
        shifts2 = np.arange(16, dtype=np.uint32) * 2
        lo = ((m.q[:, :, None] >> shifts2) & 3).reshape(O, K).astype(np.int64)
        shifts1 = np.arange(32, dtype=np.uint32)
        hi = ((m.q2[:, :, None] >> shifts1) & 1).reshape(O, K).astype(np.int64)
        return (lo + 4 * hi - 4).astype(np.float64)
    raise ValueError(m.fmt)


def numpy_scales(m) -> np.ndarray:
    if m.fmt in synth.NO_SCALE_FORMATS:
        return np.ones((m.O, m.K))
    if m.fmt == 12:   # 128 x 128 blocks: expand along both axes
        b = np.repeat(m.scales.astype(np.float64), 128, axis=0)[:m.O]
        return np.repeat(b, 128, axis=1)
    return np.repeat(m.scales.astype(np.float64), m.gs, axis=1)


def pin_numpy_decoder_matches_fixtures(lib):
    """The NumPy decoder itself agrees with every fixture (so it can judge)."""
    rows = golden_pairs("int4_pairs.txt")
    q = np.array([[b for b, _, _ in rows]], dtype=np.uint8)
    m = _qm(4, 1, 2 * q.shape[1], 2 * q.shape[1], q, np.ones((1, 1), np.float32))
    assert np.array_equal(numpy_values(m)[0], [v for _, a, b in rows for v in (a, b)])
    low, high, values = golden_int3()
    m = _qm(5, 1, 64, 64, np.array([low], np.uint32), np.ones((1, 1), np.float32),
            q2=np.array([high], np.uint32))
    assert np.array_equal(numpy_values(m)[0], values)


def _random_matrices():
    yield synth.matrix(1, 5, 96, None, 11, 1)
    yield synth.matrix(2, 5, 96, None, 11, 2)
    yield synth.matrix(4, 5, 128, 32, 11, 3)
    yield synth.matrix(4, 3, 256, 64, 11, 4)
    yield synth.matrix(5, 4, 192, 64, 11, 5)
    yield synth.matrix(7, 5, 128, 32, 11, 6)
    yield synth.matrix(10, 3, 64, None, 11, 10)
    yield synth.matrix(11, 4, 96, None, 11, 11)
    yield synth.matrix(12, 130, 256, None, 11, 12)   # two row blocks, the second ragged
    yield synth.matrix(13, 5, 128, 32, 11, 13)
    yield synth.matrix(13, 3, 256, 64, 11, 14)
    yield synth.matrix(14, 4, 96, None, 11, 15)


def pin_random_layouts(lib):
    """Oracle decode == NumPy decode on random multi-row matrices."""
    for m in _random_matrices():
        got = lib.code_values(m)
        want = numpy_values(m)
        assert np.array_equal(got, want), f"fmt {m.fmt}: layout mismatch"


def pin_dequant_rounding_and_scale_index(lib):
    """dequant[o][k] == RNE_f32(v * s[o][k // gs]), with every group's scale distinct."""
    for m in _random_matrices():
        if m.fmt in synth.NO_SCALE_FORMATS:
            assert lib.dequant(m).tobytes() == numpy_values(m).astype(np.float32).tobytes(), m.fmt
            continue
        # distinct scales per (row, group) or block: identifiable if mis-indexed
        shape = m.scales.shape
        s = (1.0 + np.arange(shape[0] * shape[1], dtype=np.float64) / 64.0) * 1e-3
        m.scales = s.reshape(shape).astype(np.float32)
        want = (numpy_values(m) * numpy_scales(m)).astype(np.float32)   # exact product, one rounding
        got = lib.dequant(m)
        assert got.tobytes() == want.tobytes(), f"fmt {m.fmt}: dequant bits differ"


def pin_signed_zero(lib):
    """A zero code times a negative scale gives -0; MXFP4 code 8 gives -0."""
    q = np.full((1, 16), 0x88, np.uint8)            # int4 nibble 8 -> value 0
    m = _qm(4, 1, 32, 32, q, np.full((1, 1), -0.5, np.float32))
    d = lib.dequant(m)
    assert all(math.copysign(1.0, v) < 0 for v in d[0]), "0 * negative scale must be -0"
    m = _qm(7, 1, 32, 32, q, np.full((1, 1), 0.5, np.float32))
    d = lib.dequant(m)
    assert all(v == 0 and math.copysign(1.0, v) < 0 for v in d[0]), "MXFP4 code 8 must be -0"


# ---------------------------------------------------------------------------
# GEMV
# ---------------------------------------------------------------------------

def pin_one_hot_selects_column(lib):
    """x = e_k gives y[o] = w[o][k] exactly, so RNE_f32(y) == dequant.

    Compared by value: a sum of signed zeros starting from +0 is +0, so a
    -0 weight reads back as +0 here (outputs compare equal across signs).
    """
    for m in _random_matrices():
        x = np.eye(m.K, dtype=np.float32)
        y, a = lib.gemv(m, x)                  # y[k][o]
        d = lib.dequant(m)                     # [o][k]
        assert np.array_equal(y.T.astype(np.float32), d), f"fmt {m.fmt}"
        assert np.array_equal(a.T, np.abs(y.T))


def pin_fraction_brute_force(lib):
    """Tiny shapes: oracle y within f64 rounding of the exact rational sum."""
    for m in _random_matrices():
        O, K = min(m.O, 3), m.K
        x = synth.activations(2, K, 99, m.fmt)
        y, a = lib.gemv(m, x)
        assert np.all(np.isfinite(y)) and np.all(np.isfinite(a)), m.fmt
        v = numpy_values(m)
        sc = numpy_scales(m)
        for s in range(2):
            for o in range(O):
                exact = sum(Fraction(v[o, k]) * Fraction(float(sc[o, k])) * Fraction(float(x[s, k]))
                            for k in range(K))
                mag = sum(abs(Fraction(v[o, k]) * Fraction(float(sc[o, k])) * Fraction(float(x[s, k])))
                          for k in range(K))
                assert abs(Fraction(y[s, o]) - exact) <= mag * Fraction(2 * K, 2**53), (m.fmt, s, o)
                assert abs(Fraction(a[s, o]) - mag) <= mag * Fraction(2 * K, 2**53), (m.fmt, s, o)


def _group_sums(x, gs):
    return [math.fsum(float(v) for v in x[g * gs:(g + 1) * gs]) for g in range(len(x) // gs)]


def pin_constant_codes_closed_form(lib):
    """All codes equal c: y[o] = value(c) * sum_g s[o][g] * sum_{k in g} x_k."""
    K = 256
    x = synth.activations(1, K, 77, 1)[0]
    e2m1 = golden_e2m1()
    cases = []
    for c in range(16):   # int4, gs 32 and gs 64
        for gs in (32, 64):
            cases.append((4, gs, np.full((3, K // 2), c | (c << 4), np.uint8), None, c - 8))
    for c in range(16):
        cases.append((7, 32, np.full((3, K // 2), c | (c << 4), np.uint8), None, e2m1[c]))
    for c in (-127, -1, 0, 5, 127):
        cases.append((1, K, np.full((3, K), c, np.int8), None, c))
    for c in range(8):
        cases.append((5, 64, np.full((3, K // 16), (c & 3) * 0x55555555, np.uint32),
                      np.full((3, K // 32), 0xFFFFFFFF if c & 4 else 0, np.uint32), c - 4))
    for c in (-127, -3, 0, 64, 127):   # int8 with group scales
        for gs in (32, 64):
            cases.append((13, gs, np.full((3, K), c, np.int8), None, c))
    for code, val in ((0x38, 1.0), (0xD4, -12.0), (0x7E, 448.0), (0x01, 2.0**-9)):   # E4M3
        cases.append((12, 128, np.full((3, K), code, np.uint8), None, val))
    for fmt, code, val in ((14, 0x3555, 0.333251953125), (14, 0x8001, -2.0**-24), (11, 0x4049, 3.140625),
                           (11, 0xBE00, -0.125)):
        cases.append((fmt, K, np.full((3, K), code, np.uint16), None, val))
    cases.append((10, K, np.full((3, K), -0.375, np.float32), None, -0.375))
    for fmt, gs, q, q2, val in cases:
        G = K // gs
        if fmt in synth.NO_SCALE_FORMATS:
            s, srow = None, lambda o: np.ones(G)
        elif fmt == 12:   # one row block: every row takes block row 0
            s = synth.rng_for(5, fmt, gs).uniform(1e-3, 2e-2, size=(1, G)).astype(np.float32)
            srow = lambda o: s[0]
        else:
            s = synth.rng_for(5, fmt, gs).uniform(1e-3, 2e-2, size=(3, G)).astype(np.float32)
            srow = lambda o: s[o]
        m = _qm(fmt, 3, K, gs, q, s, q2=q2)
        y, _ = lib.gemv(m, x[None, :])
        xs = _group_sums(x, gs)
        xa = _group_sums(np.abs(x), gs)
        for o in range(3):
            sr = srow(o)
            want = val * math.fsum(float(sr[g]) * xs[g] for g in range(G))
            ref = abs(val) * math.fsum(float(sr[g]) * xa[g] for g in range(G))
            assert abs(y[0, o] - want) <= 2 * K * 2.0**-52 * ref, (fmt, gs, val, o, y[0, o], want)


def pin_fp8_block_scales_closed_form(lib):
    """E4M3 blocks: all codes 1.0, scale of block (i, j) 2^-(4i + j), x = 1:
    y[o] = 128 * sum_j 2^-(4 (o // 128) + j), exactly (three row blocks, the
    last ragged, three column blocks)."""
    O, K = 300, 384
    q = np.full((O, K), 0x38, np.uint8)
    s = np.array([[2.0 ** -(4 * i + j) for j in range(3)] for i in range(3)], np.float32)
    y, _ = lib.gemv(_qm(12, O, K, 128, q, s), np.ones((1, K), np.float32))
    for o in range(O):
        want = 128.0 * sum(2.0 ** -(4 * (o // 128) + j) for j in range(3))
        assert y[0, o] == want, (o, y[0, o], want)


def pin_zero_scales(lib):
    for m in _random_matrices():
        if m.fmt in synth.NO_SCALE_FORMATS:
            continue
        m.scales = np.zeros_like(m.scales)
        y, a = lib.gemv(m, synth.activations(2, m.K, 3))
        assert np.all(y == 0) and np.all(a == 0), m.fmt


def pin_power_of_two_scaling(lib):
    """Scaling x by 2^j scales y by 2^j bit for bit (no rounding changes)."""
    for m in _random_matrices():
        x = synth.activations(2, m.K, 4)
        y0, _ = lib.gemv(m, x)
        for j in (3, -5):
            y1, _ = lib.gemv(m, np.ldexp(x, j).astype(np.float32))
            assert np.array_equal(y1, np.ldexp(y0, j)), (m.fmt, j)


def pin_normaliser_bounds(lib):
    for m in _random_matrices():
        y, a = lib.gemv(m, synth.activations(3, m.K, 5))
        assert np.all(a >= np.abs(y)) and np.all(a > 0)


def pin_token_rows_independent(lib):
    """Row s of a batch equals the single-token result for x[s] (no transposition)."""
    for m in _random_matrices():
        x = synth.activations(3, m.K, 6)
        y, a = lib.gemv(m, x)
        for s in range(3):
            y1, a1 = lib.gemv(m, x[s:s + 1])
            assert np.array_equal(y[s], y1[0]) and np.array_equal(a[s], a1[0]), (m.fmt, s)


# ---------------------------------------------------------------------------
# SwiGLU and gate_up
# ---------------------------------------------------------------------------

def pin_silu(lib):
    from scipy.special import expit
    assert lib.silu(0.0) == 0.0
    for z in np.linspace(-30, 30, 241):
        want = z * expit(z)
        got = lib.silu(z)
        assert abs(got - want) <= 4e-16 * max(abs(want), 1e-300) + 1e-300, (z, got, want)
        # silu(z) - silu(-z) = z
        assert abs(lib.silu(z) - lib.silu(-z) - z) <= 1e-15 * max(abs(z), 1.0)
    assert abs(lib.silu(50.0) - 50.0) < 1e-18 * 50
    assert lib.silu(-800.0) == 0.0 or abs(lib.silu(-800.0)) < 1e-300


def pin_gate_up_one_hot(lib):
    """x = e_k: g = w_gate[i][k], u = w_up[i][k], h = g * expit(g) * u."""
    from scipy.special import expit
    for fmt, gs in ((4, 32), (7, 32), (1, None), (5, 64)):
        K = 128
        G = synth.matrix(fmt, 6, K, gs, 21, fmt, 0)
        U = synth.matrix(fmt, 6, K, gs, 21, fmt, 1)
        # larger scales so silu works away from its linear part
        G.scales = (G.scales * 200).astype(np.float32)
        dg = lib.dequant(G).astype(np.float64)
        du = lib.dequant(U).astype(np.float64)
        for k in (0, 1, 31, 64, 127):
            x = np.zeros((1, K), np.float32)
            x[0, k] = 1.0
            r = lib.gate_up(G, U, x)
            g = lib.gemv(G, x)[0][0]
            assert np.allclose(r["g"][0], g, rtol=0, atol=0)
            assert np.allclose(np.float32(r["g"][0]), dg[:, k], rtol=0, atol=0)
            assert np.allclose(np.float32(r["u"][0]), du[:, k], rtol=0, atol=0)
            want = r["g"][0] * expit(r["g"][0]) * r["u"][0]
            assert np.allclose(r["h"][0], want, rtol=1e-15, atol=0), (fmt, k)


def pin_gate_up_zero(lib):
    G = synth.matrix(4, 8, 64, 32, 22, 0)
    U = synth.matrix(4, 8, 64, 32, 22, 1)
    x = synth.activations(2, 64, 22)
    Gz = _qm(4, 8, 64, 32, G.q, np.zeros_like(G.scales))
    Uz = _qm(4, 8, 64, 32, U.q, np.zeros_like(U.scales))
    assert np.all(lib.gate_up(Gz, U, x)["h"] == 0)
    assert np.all(lib.gate_up(G, Uz, x)["h"] == 0)
    r = lib.gate_up(G, U, x)
    assert np.all(r["nh"] >= 0)


def pin_gate_up_rows(lib):
    """h[s][i] uses gate row i and up row i with token s (gate and up not swapped)."""
    from scipy.special import expit
    G = synth.matrix(4, 8, 64, 32, 23, 0)
    U = synth.matrix(4, 8, 64, 32, 23, 1)
    G.scales = (G.scales * 50).astype(np.float32)
    x = synth.activations(3, 64, 23)
    r = lib.gate_up(G, U, x)
    g, _ = lib.gemv(G, x)
    u, _ = lib.gemv(U, x)
    assert np.array_equal(r["g"], g) and np.array_equal(r["u"], u)
    assert np.allclose(r["h"], g * expit(g) * u, rtol=1e-14, atol=0)


# ---------------------------------------------------------------------------
# expert group
# ---------------------------------------------------------------------------

def _tiny_experts(n, fmt=4, gs=32, H=64, I=32, seed=31):
    return [synth.expert(fmt, H, I, gs, seed, i) for i in range(n)]


def _mlp(lib, ex, x):
    h = lib.gate_up(ex.gate, ex.up, x)["h"]
    y, _ = lib.gemv(ex.down, h)
    return y


def pin_group_shared_only(lib):
    exs = _tiny_experts(6)
    x = synth.activations(2, 64, 32)
    ids = np.array([[0, 1, 2], [3, 4, 1]], np.int32)
    w = np.zeros((2, 3), np.float32)
    y, a = lib.expert_group(exs, ids, w, 5, x)
    want = _mlp(lib, exs[5], x)
    assert np.allclose(y, want, rtol=1e-13, atol=1e-15)
    y0, _ = lib.expert_group(exs, ids, w, -1, x)
    assert np.all(y0 == 0)


def pin_group_single_expert(lib):
    exs = _tiny_experts(6)
    x = synth.activations(2, 64, 33)
    ids = np.array([[0, 1, 2], [3, 4, 1]], np.int32)
    for t, r in ((0, 1), (1, 2)):
        w = np.zeros((2, 3), np.float32)
        w[t, r] = 1.0
        y, _ = lib.expert_group(exs, ids, w, 5, x)
        want = _mlp(lib, exs[5], x)
        want[t] += _mlp(lib, exs[int(ids[t, r])], x[t:t + 1])[0]
        assert np.allclose(y, want, rtol=1e-13, atol=1e-15), (t, r)


def pin_group_weights_scale_outputs(lib):
    """w[t][r] multiplies expert r's output: doubling one weight adds that output once more."""
    exs = _tiny_experts(5)
    x = synth.activations(1, 64, 34)
    ids = np.array([[4, 0, 2]], np.int32)
    w = np.array([[0.25, 0.5, 0.125]], np.float32)
    y1, _ = lib.expert_group(exs, ids, w, -1, x)
    w2 = w.copy()
    w2[0, 1] *= 2
    y2, _ = lib.expert_group(exs, ids, w2, -1, x)
    d = _mlp(lib, exs[0], x)[0] * 0.5
    assert np.allclose(y2[0] - y1[0], d, rtol=1e-12, atol=1e-15)


def pin_group_identical_experts(lib):
    """Every expert the same: y = (sum w) * MLP(x) + MLP_shared(x)."""
    base = _tiny_experts(1)[0]
    shared = _tiny_experts(1, seed=35)[0]
    exs = [base] * 7 + [shared]
    S, k = 3, 4
    ids, w = synth.routing(S, 7, k, 36)
    x = synth.activations(S, 64, 36)
    y, _ = lib.expert_group(exs, ids, w, 7, x)
    want = w.astype(np.float64).sum(axis=1)[:, None] * _mlp(lib, base, x) + _mlp(lib, shared, x)
    assert np.allclose(y, want, rtol=1e-12, atol=1e-15)


def pin_group_permutation(lib):
    exs = _tiny_experts(9)
    S, k = 2, 4
    ids, w = synth.routing(S, 8, k, 37)
    x = synth.activations(S, 64, 37)
    y, a = lib.expert_group(exs, ids, w, 8, x)
    perm = [2, 0, 3, 1]
    y2, a2 = lib.expert_group(exs, ids[:, perm], w[:, perm], 8, x)
    assert np.all(np.abs(y - y2) <= 1e-13 * a)
    assert np.allclose(a, a2, rtol=1e-13)


def pin_group_tokens_independent(lib):
    """Token t of a batch equals the batch of just token t."""
    exs = _tiny_experts(9)
    S, k = 3, 4
    ids, w = synth.routing(S, 8, k, 38)
    x = synth.activations(S, 64, 38)
    y, a = lib.expert_group(exs, ids, w, 8, x)
    for t in range(S):
        y1, a1 = lib.expert_group(exs, ids[t:t + 1], w[t:t + 1], 8, x[t:t + 1])
        assert np.array_equal(y[t], y1[0]) and np.array_equal(a[t], a1[0]), t


def pin_group_bad_id_is_nan(lib):
    exs = _tiny_experts(4)
    x = synth.activations(2, 64, 39)
    ids = np.array([[0, 9], [1, 2]], np.int32)
    w = np.full((2, 2), 0.5, np.float32)
    y, _ = lib.expert_group(exs, ids, w, 3, x)
    assert np.all(np.isnan(y[0])) and np.all(np.isfinite(y[1]))


def pin_group_normaliser(lib):
    exs = _tiny_experts(9)
    ids, w = synth.routing(2, 8, 4, 40)
    x = synth.activations(2, 64, 40)
    y, a = lib.expert_group(exs, ids, w, 8, x)
    assert np.all(a >= np.abs(y)) and np.all(a > 0)


def pin_gate_up_error_reach(lib):
    """nh is the first-order reach of errors eps * A_g in g and eps * A_u in u:
    the largest change of silu(g) * u over the four sign corners, over eps
    (a spare factor, a dropped term or a wrong silu slope moves it)."""
    from scipy.special import expit
    G = synth.matrix(4, 96, 256, 32, 7200, 0)
    U = synth.matrix(4, 96, 256, 32, 7200, 1)
    G.scales = (G.scales * 40).astype(np.float32)   # g over silu's curved range
    x = synth.activations(3, 256, 7200, 2)
    r = lib.gate_up(G, U, x)
    g, u, ag, au, nh = r["g"], r["u"], r["ag"], r["au"], r["nh"]
    assert np.ptp(g) > 4, "g should span silu's curved range"
    eps = 1e-7

    def swiglu(gv, uv):
        return gv * expit(gv) * uv

    h0 = swiglu(g, u)
    reach = np.zeros_like(h0)
    for sg in (-1.0, 1.0):
        for su in (-1.0, 1.0):
            reach = np.maximum(reach, np.abs(swiglu(g + sg * eps * ag, u + su * eps * au) - h0))
    reach /= eps
    assert np.allclose(reach, nh, rtol=1e-3, atol=1e-9 * float(nh.max())), float(np.max(np.abs(reach - nh) / nh))


def pin_group_normaliser_decomposes(lib):
    """The group's propagated normaliser is, per row, |w| times the down row's
    own sum |D h| plus sum |D| nh (the reach of h's errors), summed over the
    ranks, plus the shared expert's (weight 1)."""
    exs = _tiny_experts(5)
    x = synth.activations(1, 64, 44)
    ids = np.array([[1, 3]], np.int32)
    w = np.array([[0.75, -0.5]], np.float32)
    _, a = lib.expert_group(exs, ids, w, 4, x)
    want = np.zeros(64)
    for e, wr in ((1, 0.75), (3, -0.5), (4, 1.0)):
        r = lib.gate_up(exs[e].gate, exs[e].up, x)
        _, ah = lib.gemv(exs[e].down, r["h"])    # sum_i |D[o][i] h[i]|, h in f64
        _, an = lib.gemv(exs[e].down, r["nh"])   # sum_i |D[o][i]| nh[i], nh >= 0
        want += abs(wr) * (ah[0] + an[0])
    assert np.allclose(a[0], want, rtol=1e-12, atol=0)


def pin_group_down_brute_force(lib):
    """Down and combine on given hidden states: within f64 rounding of the exact
    rational sum, slot t*k + r for (token t, rank r), the shared slot S*k + t
    last with weight 1, signed weights, an expert twice in one token."""
    exs = _tiny_experts(6)   # down [64 x 32], int4-g32
    S, k, H, I = 2, 3, 64, 32
    ids = np.array([[0, 3, 0], [2, 1, 4]], np.int32)
    w = np.array([[0.5, -0.25, 0.125], [-1.0, 0.75, 0.3]], np.float32)
    h = synth.activations(S * k + S, I, 41)
    y, a = lib.expert_group_down(exs, ids, w, 5, h)
    dec = {e: (numpy_values(exs[e].down), numpy_scales(exs[e].down)) for e in range(6)}

    def row(e, o, slot):
        v, sc = dec[e]
        terms = [Fraction(v[o, i]) * Fraction(float(sc[o, i])) * Fraction(float(h[slot, i])) for i in range(I)]
        return sum(terms), sum(abs(t) for t in terms)

    for t in range(S):
        for o in range(H):
            exact, mag = Fraction(0), Fraction(0)
            for r in range(k):
                d, m = row(int(ids[t, r]), o, t * k + r)
                exact += Fraction(float(w[t, r])) * d
                mag += abs(Fraction(float(w[t, r]))) * m
            d, m = row(5, o, S * k + t)
            exact += d
            mag += m
            tol = mag * Fraction(4 * (I + k + 1), 2**53)
            assert abs(Fraction(y[t, o]) - exact) <= tol, (t, o)
            assert abs(Fraction(a[t, o]) - mag) <= tol, (t, o)


def pin_group_down_edge_cases(lib):
    """No shared expert and zero weights give 0 exactly; a bad id makes only its
    token's row NaN."""
    exs = _tiny_experts(4)
    h = synth.activations(6, 32, 42)
    ids = np.array([[0, 2], [1, 3]], np.int32)
    y, a = lib.expert_group_down(exs, ids, np.zeros((2, 2), np.float32), None, h)
    assert np.all(y == 0) and np.all(a == 0)
    ids[0, 1] = 9
    y, _ = lib.expert_group_down(exs, ids, np.full((2, 2), 0.5, np.float32), 3, h)
    assert np.all(np.isnan(y[0])) and np.all(np.isfinite(y[1]))


def pin_group_down_matches_group(lib):
    """On the oracle's own hidden states, rounded to f32, the two-stage form is
    the one-stage group within that rounding; the propagated normaliser is at
    least the strict one."""
    exs = _tiny_experts(9)
    S, k, I = 2, 4, 32
    ids, w = synth.routing(S, 8, k, 43)
    x = synth.activations(S, 64, 43)
    y, a = lib.expert_group(exs, ids, w, 8, x)
    h = np.zeros((S * k + S, I), np.float32)
    for t in range(S):
        for r in range(k):
            e = exs[int(ids[t, r])]
            h[t * k + r] = lib.gate_up(e.gate, e.up, x[t:t + 1])["h"][0]
        h[S * k + t] = lib.gate_up(exs[8].gate, exs[8].up, x[t:t + 1])["h"][0]
    y2, a2 = lib.expert_group_down(exs, ids, w, 8, h)
    assert np.all(np.abs(y2 - y) <= 2.0**-23 * a2 + 1e-300)
    assert np.all(a >= a2 * (1 - 2.0**-20))


# ---------------------------------------------------------------------------
# clamped SwiGLU (swiglu_limit)
# ---------------------------------------------------------------------------

def _gu_pair(seed=7100, I=96, H=256):
    G = synth.matrix(4, I, H, 32, seed, 0)
    U = synth.matrix(4, I, H, 32, seed, 1)
    x = synth.activations(3, H, seed, 2)
    return G, U, x


def pin_clamp_huge_limit_is_plain(lib):
    """A limit above every |g| and |u| changes nothing, bit for bit."""
    G, U, x = _gu_pair()
    plain = lib.gate_up(G, U, x)
    for L in (1e3, 1e300):
        r = lib.gate_up(G, U, x, L)
        assert np.array_equal(r["h"], plain["h"]), L
        assert np.array_equal(r["nh"], plain["nh"]), L


def pin_clamp_regions(lib):
    """Against the plain SwiGLU (pinned above), region by region:
    g < L and |u| <= L: unchanged; g < L and |u| > L: scaled by L/|u|;
    g >= L: h / clamp(u) is one value for every output (silu(L))."""
    G, U, x = _gu_pair(7101)
    plain = lib.gate_up(G, U, x)
    g, u = plain["g"], plain["u"]
    L = float(np.median(np.abs(u)))
    r = lib.gate_up(G, U, x, L)
    h, hp = r["h"], plain["h"]
    free = (g < L) & (np.abs(u) <= L)
    assert free.any() and np.array_equal(h[free], hp[free])
    cut = (g < L) & (np.abs(u) > L)
    assert cut.any() and np.allclose(h[cut], hp[cut] * L / np.abs(u[cut]), rtol=1e-14, atol=0)
    sat = (g >= L) & (np.abs(u) > 1e-6)
    assert sat.sum() > 3
    ratio = h[sat] / np.clip(u[sat], -L, L)
    assert np.allclose(ratio, ratio[0], rtol=1e-14, atol=0)
    assert ratio[0] > 0


def pin_clamp_is_odd_in_up(lib):
    """Negating the up weights negates h exactly, clamped or not."""
    G, U, x = _gu_pair(7102)
    Un = synth.QMatrix(U.fmt, U.O, U.K, U.gs, U.q, U.q2, (-U.scales).astype(np.float32))
    for L in (math.inf, 0.3, 0.01):
        a = lib.gate_up(G, U, x, L)["h"]
        b = lib.gate_up(G, Un, x, L)["h"]
        assert np.array_equal(a, -b), L


def pin_clamp_tiny_limit_zeroes_outputs(lib):
    """The pages: a limit of 0 zeroes every expert's output; as L -> 0+ so does h and y."""
    G, U, x = _gu_pair(7103)
    r = lib.gate_up(G, U, x, 1e-150)
    assert np.all(np.abs(r["h"]) <= 1e-150)
    ex = _tiny_experts(4)
    ids = np.array([[0, 2], [3, 1]], np.int32)
    w = np.array([[0.7, 0.3], [0.5, 0.5]], np.float32)
    xg = synth.activations(2, 64, 7104)
    y, _ = lib.expert_group(ex, ids, w, 1, xg, 1e-150)
    assert np.all(np.abs(y) < 1e-140)
    y_plain, _ = lib.expert_group(ex, ids, w, 1, xg)
    assert np.abs(y_plain).max() > 1e-3


def pin_clamp_group_uses_limit(lib):
    """The group applies the limit in every expert, shared included: each token's y equals the
    weighted sum of the clamped single-expert MLPs."""
    ex = _tiny_experts(3)
    xg = synth.activations(1, 64, 7105)
    L = 0.05
    ys = []
    for e in range(3):
        y1, _ = lib.expert_group(ex, np.array([[e]], np.int32), np.array([[1.0]], np.float32), None, xg, L)
        ys.append(y1[0])
    y, _ = lib.expert_group(ex, np.array([[0, 1]], np.int32), np.array([[0.25, 0.75]], np.float32), 2, xg, L)
    want = np.float64(np.float32(0.25)) * ys[0] + np.float64(np.float32(0.75)) * ys[1] + ys[2]
    assert np.allclose(y[0], want, rtol=1e-12, atol=1e-15)
    y_plain, _ = lib.expert_group(ex, np.array([[0, 1]], np.int32), np.array([[0.25, 0.75]], np.float32), 2, xg)
    assert not np.allclose(y[0], y_plain[0])


# ---------------------------------------------------------------------------
# router
# ---------------------------------------------------------------------------

def golden_routes():
    """The hand-worked router cases of tests/golden/route_examples.txt."""
    cases, cur = [], None
    for r in _rows("route_examples.txt"):
        if r[0] == "case":
            f = dict(zip(r[2::2], r[3::2]))
            cur = {"name": r[1], "mode": int(f["mode"]), "k": int(f["k"]), "renorm": bool(int(f["renorm"])),
                   "scale": float(f["scale"])}
            cases.append(cur)
        elif r[0] == "logits":
            cur["logits"] = np.array([[float(v) for v in r[1:]]], np.float32)
        elif r[0] == "bias":
            cur["bias"] = None if r[1] == "none" else np.array([float(v) for v in r[1:]], np.float32)
        elif r[0] == "ids":
            cur["ids"] = [int(v) for v in r[1:]]
        elif r[0] == "w":
            cur["w"] = [float(v) for v in r[1:]]
    return cases


def pin_route_golden(lib):
    for c in golden_routes():
        r = lib.route(c["logits"], c["k"], c["mode"], c["renorm"], c["bias"], c["scale"])
        assert r["ids"][0].tolist() == c["ids"], (c["name"], r["ids"])
        assert np.allclose(r["w"][0], c["w"], rtol=1e-6, atol=0), (c["name"], r["w"])


def _logits(S, E, seed, spread=2.0):
    return (synth.rng_for(seed, S, E).standard_normal((S, E)) * spread).astype(np.float32)


def pin_route_softmax_is_library_softmax(lib):
    """k = E without renormalising: the weights, read back by id, are scipy's softmax."""
    from scipy.special import softmax
    lg = _logits(5, 37, 7001)
    r = lib.route(lg, 37, 0)
    for t in range(5):
        ref = softmax(lg[t].astype(np.float64))
        got = np.empty(37)
        got[r["ids"][t]] = r["w"][t]
        assert np.allclose(got, ref, rtol=1e-13, atol=0)
        assert sorted(r["ids"][t].tolist()) == list(range(37))


def pin_route_sigmoid_is_library_expit(lib):
    from scipy.special import expit
    lg = _logits(4, 19, 7002, spread=6.0)
    r = lib.route(lg, 19, 1)
    for t in range(4):
        got = np.empty(19)
        got[r["ids"][t]] = r["w"][t]
        assert np.allclose(got, expit(lg[t].astype(np.float64)), rtol=1e-14, atol=0)


def pin_route_topk_brute_force(lib):
    """Selection against a sort by (-key, index), with many equal logits."""
    rng = synth.rng_for(7003)
    for mode in (0, 1):
        for E, k in ((6, 1), (9, 4), (33, 8), (64, 10), (70, 70)):
            lg = rng.integers(-3, 4, size=(6, E)).astype(np.float32) * np.float32(0.5)
            r = lib.route(lg, k, mode)
            for t in range(6):
                want = sorted(range(E), key=lambda e: (-float(lg[t, e]), e))[:k]
                assert r["ids"][t].tolist() == want, (mode, E, k, t)


def pin_route_bias_picks_only(lib):
    """A bias changes which experts are picked, never their weights."""
    from scipy.special import expit
    lg = _logits(3, 16, 7004)
    bias = np.zeros(16, np.float32)
    bias[5] = 10.0   # expert 5 is always picked first
    bias[11] = 9.0   # then expert 11
    for mode in (0, 1):
        r = lib.route(lg, 4, mode, False, bias)
        for t in range(3):
            assert r["ids"][t][:2].tolist() == [5, 11]
            if mode == 1:
                assert np.allclose(r["w"][t][:2], expit(lg[t, [5, 11]].astype(np.float64)), rtol=1e-14)
            key = r["key"][t]
            picked = set(r["ids"][t].tolist())
            worst = min(key[e] for e in picked)
            assert all(key[e] <= worst for e in range(16) if e not in picked)


def pin_route_renorm_and_scale(lib):
    lg = _logits(6, 40, 7005)
    for mode in (0, 1):
        r = lib.route(lg, 6, mode, True, None, 2.5)
        assert np.allclose(r["w"].sum(axis=1), 2.5, rtol=1e-14)
        plain = lib.route(lg, 6, mode, False, None, 1.0)
        ratio = r["w"] / plain["w"]
        assert np.allclose(ratio, ratio[:, :1], rtol=1e-13)   # one factor per token


def pin_route_tokens_independent(lib):
    lg = _logits(7, 24, 7006)
    r = lib.route(lg, 5, 0, True)
    for t in range(7):
        one = lib.route(lg[t:t + 1], 5, 0, True)
        assert one["ids"][0].tolist() == r["ids"][t].tolist()
        assert np.array_equal(one["w"][0], r["w"][t])



# ---------------------------------------------------------------------------
# DeepSeek V4's rounding activation
# ---------------------------------------------------------------------------

def _torch():
    import torch
    return torch


def _bf16_torch(v):
    """f32 values rounded to bf16 by torch's cast (nearest-even)."""
    torch = _torch()
    return torch.from_numpy(np.asarray(v, np.float32)).to(torch.bfloat16).to(torch.float64).numpy()


def _e4m3_torch(v):
    """f32 values rounded to E4M3 (the fn variant: no infinities) by torch's cast."""
    torch = _torch()
    return torch.from_numpy(np.asarray(v, np.float32)).to(torch.float8_e4m3fn).to(torch.float64).numpy()


def _f32_ties(rng, n, low_bits, exp_lo, exp_hi):
    """f32 values whose low ``low_bits`` bits are exactly half a unit of the
    shorter format (a tie), the rest random, exponents in [exp_lo, exp_hi)."""
    mant = rng.integers(0, 1 << 23, size=n, dtype=np.int64)
    mant = (mant >> low_bits << low_bits) | (1 << (low_bits - 1))
    e = rng.integers(exp_lo, exp_hi, size=n)
    bits = (rng.integers(0, 2, size=n) << 31) | ((e + 127) << 23) | mant
    return bits.astype(np.uint32).view(np.float32)


def pin_bf16_rounding_is_library_cast(lib):
    """bf16 nearest-even on f32 values (random, exact ties, bf16 subnormals) is torch's cast."""
    rng = np.random.default_rng(7300)
    vals = np.concatenate([
        (rng.standard_normal(600) * np.exp2(rng.integers(-30, 30, 600))).astype(np.float32),
        _f32_ties(rng, 400, 16, -20, 20),
        (rng.uniform(-1, 1, 100) * 2.0 ** -128).astype(np.float32),   # below bf16's smallest normal
        np.array([0.0, -0.0, 1.0, 1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, -(1.0 + 2 ** -8)], np.float32)])
    want = _bf16_torch(vals)
    got = np.array([lib.round_fmt(float(v), 7, -126) for v in vals])
    assert np.array_equal(got, want), np.flatnonzero(got != want)[:5]


def pin_e4m3_rounding_is_library_cast(lib):
    """E4M3 nearest-even on f32 values below 448 (random, ties, subnormals) is torch's cast."""
    rng = np.random.default_rng(7301)
    vals = np.concatenate([
        rng.uniform(-440, 440, 500).astype(np.float32),
        (rng.standard_normal(400) * np.exp2(rng.integers(-9, 6, 400))).astype(np.float32),
        _f32_ties(rng, 300, 20, -6, 8),            # ties between normal E4M3 values
        (rng.integers(-32, 33, 100) * 2.0 ** -10).astype(np.float32),   # ties in the subnormal range
        np.array([448.0, 447.9, 0.0, 2 ** -6, 2 ** -9, 2 ** -10, 3 * 2 ** -11, 0.0625 * 1.0625], np.float32)])
    vals = vals[np.abs(vals) <= 448.0]
    want = _e4m3_torch(vals)
    got = np.array([lib.round_fmt(float(v), 3, -6) for v in vals])
    assert np.array_equal(got, want), [(float(v), a, b) for v, a, b in zip(vals, got, want) if a != b][:5]


def pin_v4_block_scale(lib):
    """The scale is the smallest power of two that takes the block's maximum below 448."""
    hand = {448.0: 2.0, 447.0: 1.0, 224.0: 1.0, 223.9: 0.5, 1.0: 2.0 ** -8, 0.0: 1.0,
            896.0: 4.0, 2.0 ** -20: 2.0 ** -28, 1000.0: 4.0}
    for m, s in hand.items():
        assert lib.v4_block_scale(m) == s, (m, lib.v4_block_scale(m), s)
    rng = np.random.default_rng(7302)
    for m in np.exp2(rng.uniform(-40, 40, 300)):
        s = lib.v4_block_scale(float(m))
        assert math.frexp(s)[0] == 0.5            # a power of two
        assert m / s < 448.0 <= m / (s / 2.0)


def pin_v4_combine_order(lib):
    """Rows join in ascending expert id, equal ids in rank order, the shared row last, in f32:
    1 + 1 + 2^24 is 2^24 + 2 in f32 while 2^24 + 1 + 1 is 2^24 (1 is half an ulp there)."""
    big = 2.0 ** 24
    rows = np.array([[big], [1.0], [1.0]])
    assert lib.v4_combine(rows, [7, 3, 5], False)[0] == big + 2      # ids 3, 5 before 7
    assert lib.v4_combine(rows, [1, 3, 5], False)[0] == big
    rows = np.array([[1.0], [big], [1.0]])
    assert lib.v4_combine(rows, [4, 4, 2], False)[0] == big + 2      # id 2, then id 4's ranks 0, 1
    rows = np.array([[1.0], [1.0], [big]])
    assert lib.v4_combine(rows, [1, 2], True)[0] == big + 2          # the shared row after the routed ones
    rows = np.array([[1.0, -3.0], [2.0, 0.5]])
    assert lib.v4_combine(rows, [9, 8], False).tolist() == [3.0, -2.5]


def _f32_expert(H, I, seed, gate_rows):
    """An expert of f32 rows (format 10): gate row i all gate_rows[i]; up rows all 1/H; down random."""
    rng = np.random.default_rng(seed)

    def mat(v, O, K):
        return _qm(10, O, K, K, np.ascontiguousarray(v, np.float32), None)

    class Ex:
        pass
    ex = Ex()
    ex.gate = mat(np.repeat(np.asarray(gate_rows, np.float32)[:, None], H, axis=1), I, H)
    ex.up = mat(np.full((I, H), 1.0 / H, np.float32), I, H)
    ex.down = mat(rng.standard_normal((H, I)).astype(np.float32), H, I)
    return ex


def pin_v4_group_closed_form(lib):
    """x all ones and constant gate and up rows make g[i] = H * gate_rows[i] and u[i] = 1 exactly;
    every later step is then a library cast, a closed-form scale or an exact rational sum."""
    H, I = 64, 256
    rng = np.random.default_rng(7303)
    gate_rows = (rng.choice([-1, 1], I) * np.exp2(rng.uniform(-16, 3, I))).astype(np.float32)
    gate_rows[:128] = gate_rows[:128] * np.float32(2.0 ** -9)   # block 0: |g| < 1
    gate_rows[200] = 0.12    # block 1's largest activation sits in its second half
    gate_rows[130] = 0.02
    # block 0's largest: g just under a limit of 6.99 whose bf16 rounding (7) is above it; a
    # route weight for which clamping before the rounding would change its E4M3 value
    L = 6.99
    gate_rows[17] = np.float32(6.986 / H)
    g17 = float(_bf16_torch(H * np.float64(gate_rows[17])))

    def e4_of(gc, wr):
        a = float(_bf16_torch(gc / (1.0 + math.exp(-gc)) * float(wr)))
        s = 2.0 ** (math.floor(math.log2(a / 448.0)) + 1)
        return float(_e4m3_torch(a / s)) * s
    wr = next(w for w in (np.float32(0.7 + j / 4096) for j in range(400))
              if e4_of(min(g17, L), w) != e4_of(g17, w))
    ex = _f32_expert(H, I, 7304, gate_rows)
    x = np.ones((1, H), np.float32)
    for limit in (math.inf, L):
        r = lib.expert_group_v4([ex], np.array([[0]], np.int32), np.array([[wr]], np.float32), None, x, limit)
        assert r["open"] == 0
        _v4_closed_form_check(r, ex, gate_rows, H, I, wr, limit)


def _v4_closed_form_check(r, ex, gate_rows, H, I, wr, limit):
    g = np.minimum(_bf16_torch(H * gate_rows.astype(np.float64)), limit)   # clamped after the rounding
    hv = np.array([gi / (1.0 + math.exp(-gi)) for gi in g]) * float(wr)   # u = 1 exactly
    a = _bf16_torch(hv)
    e4 = np.empty(I)
    for b0 in range(0, I, 128):
        blk = a[b0:b0 + 128]
        m = np.max(np.abs(blk))
        s = 2.0 ** (math.floor(math.log2(m / 448.0)) + 1)
        e4[b0:b0 + 128] = _e4m3_torch(blk / s) * s
    assert np.array_equal(r["h"][0], e4)
    Wd = ex.down.q.astype(np.float64)
    d = np.array([float(sum(Fraction(float(Wd[o, k])) * Fraction(float(e4[k])) for k in range(I)))
                  for o in range(H)])
    assert np.array_equal(r["y"][0].astype(np.float64), _bf16_torch(d))


def pin_v4_zero_weight_slot_adds_nothing(lib):
    """A routed slot of weight 0 leaves every row of y as the group without it (bit for bit)."""
    ex = _tiny_experts(3, fmt=7, gs=32, H=64, I=128)
    x = synth.activations(2, 64, 7305)
    ids = np.array([[0, 1], [2, 1]], np.int32)
    r2 = lib.expert_group_v4(ex, ids, np.array([[0.0, 0.6], [0.3, 0.0]], np.float32), 2, x)
    for t, keep in ((0, 1), (1, 0)):
        r1 = lib.expert_group_v4(ex, ids[t:t + 1, keep:keep + 1],
                                 np.array([[(0.6, 0.3)[t]]], np.float32), 2, x[t:t + 1])
        assert np.array_equal(r2["y"][t], r1["y"][0])


def pin_v4_group_near_plain_group(lib):
    """The roundings move y by at most a few percent of the plain group's normaliser
    (E4M3 keeps 4 significant bits), and the weights, the shared expert and the limit act
    as in the plain group."""
    ex = _tiny_experts(4, fmt=7, gs=32, H=64, I=256)
    x = synth.activations(3, 64, 7306) * np.float32(8.0)
    ids = np.array([[0, 1], [2, 0], [1, 2]], np.int32)
    w = np.array([[0.6, 0.4], [0.9, 0.1], [0.5, 0.5]], np.float32)
    for limit in (math.inf, 0.02):
        y, a = lib.expert_group(ex, ids, w, 3, x, limit)
        r = lib.expert_group_v4(ex, ids, w, 3, x, limit)
        err = np.abs(r["y"].astype(np.float64) - y)
        assert np.all(err <= 0.08 * a + 1e-30), float(np.max(err / a))
        assert np.max(np.abs(y)) > 0 and np.mean(err) < 0.02 * np.mean(a)


def pin_v4_h_rows_are_e4m3_blocks(lib):
    """Each block of 128 in a slot's h is a power of two times E4M3 values, the largest under 448."""
    ex = _tiny_experts(2, fmt=7, gs=32, H=64, I=256)
    x = synth.activations(2, 64, 7307) * np.float32(8.0)
    r = lib.expert_group_v4(ex, np.array([[0], [1]], np.int32), np.array([[0.8], [0.25]], np.float32), 0, x)
    for row in r["h"]:
        for b0 in range(0, row.size, 128):
            blk = row[b0:b0 + 128]
            m = np.max(np.abs(blk))
            assert m > 0
            s = lib.v4_block_scale(m)
            assert np.array_equal(_e4m3_torch(blk / s), blk / s) and m / s < 448.0



def pin_v4_bounds(lib):
    """The bounds for a device's error hold the exact-arithmetic result and collapse onto it
    when the allowed errors are zero; a draw of this size has open decisions to bound."""
    ex = _tiny_experts(3, fmt=7, gs=32, H=256, I=512)
    x = synth.activations(2, 256, 7308) * np.float32(4.0)
    ids = np.array([[0, 1], [2, 0]], np.int32)
    w = np.array([[0.7, 0.3], [0.45, 0.55]], np.float32)
    exact = lib.expert_group_v4(ex, ids, w, 2, x)
    for key in ("h", "y"):
        assert np.array_equal(exact[key + "_lo"], exact[key]) and np.array_equal(exact[key + "_hi"], exact[key])
    r = lib.expert_group_v4(ex, ids, w, 2, x, math.inf, 0.0, 2.0 ** -12, 2.0 ** -14)
    assert r["open"] > 0
    assert np.array_equal(r["h"], exact["h"]) and np.array_equal(r["y"], exact["y"])
    assert np.all(r["h_lo"] <= r["h"]) and np.all(r["h"] <= r["h_hi"]) and np.any(r["h_lo"] < r["h_hi"])
    assert np.all(r["y_lo"] <= r["y"]) and np.all(r["y"] <= r["y_hi"]) and np.any(r["y_lo"] < r["y_hi"])


ALL_PINS = [v for k, v in sorted(globals().items()) if k.startswith("pin_") and callable(v)]
