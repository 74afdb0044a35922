"""Parity of formats 10 (f32 rows), 11 (bf16 rows), 12 (E4M3 with 128 x 128
block scales), 13 (int8 with group scales) and 14 (f16 rows) with the CPU
oracle, through the C ABI.

Bars as for the other formats: dequantised weights bit for bit (NaN codes
compare as NaN, whatever their payload), and every output within 1e-5 of its
row's normaliser sum_k |w*x|.  The shapes have ragged rows (and ragged
128-row scale blocks), K that is not a multiple of a wave's 64 chunks, and
batches on both sides of the matrix-core cut-overs (matmul from 9 tokens,
gate_up from 8, 9 for formats 1 and 13; formats 10 and 11 stay on the per-row
route).
"""
import numpy as np
import pytest
import torch

import oracle
import synth
from gpu_helpers import assert_close, check_group, dev_f32, host, log

pytestmark = pytest.mark.gpu

if torch.cuda.is_available():
    import dequant_gemv_expert_amd as dq
else:   # collected on CPU-only hosts, never run there
    dq = None


@pytest.fixture(autouse=True)
def _announce(request):
    log(f"[gpu] start {request.node.nodeid}")
    yield
    torch.cuda.synchronize()
    log(f"[gpu] done  {request.node.nodeid}")


def up(m):
    return dq.Matrix.upload(m)


def same_bits_or_nan(a: np.ndarray, b: np.ndarray) -> bool:
    """f32 arrays with NaN in the same places and the same bits elsewhere."""
    na, nb = np.isnan(a), np.isnan(b)
    return np.array_equal(na, nb) and a[~na].view(np.uint32).tobytes() == b[~nb].view(np.uint32).tobytes()


SPECS = [  # (fmt, O, K, gs)
    (10, 1, 4, None), (10, 77, 1028, None), (10, 130, 2048, None),
    (11, 1, 8, None), (11, 130, 1032, None), (11, 64, 4096, None),
    (12, 1, 128, None), (12, 130, 1152, None), (12, 300, 2048, None),
    (13, 1, 32, 32), (13, 77, 1056, 32), (13, 64, 2048, 64), (13, 50, 1024, 128),
    (14, 1, 8, None), (14, 130, 1032, None), (14, 300, 2048, None),
]
IDS = [f"fmt{s[0]}_{s[1]}x{s[2]}" + (f"_gs{s[3]}" if s[3] else "") for s in SPECS]


def _m(i, spec):
    fmt, O, K, gs = spec
    return synth.matrix(fmt, O, K, gs, 6000 + i, fmt)


# ---------------------------------------------------------------------------
# dequant
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("i,spec", list(enumerate(SPECS)), ids=IDS)
def test_dequant_bits_random(i, spec):
    m = _m(i, spec)
    got = host(dq.dqg_dequant(up(m)))
    assert same_bits_or_nan(got, oracle.dequant(m)), f"{spec}: dequant bits differ"


def test_dequant_every_code():
    """Every f16 and bf16 code (65536 of each), every E4M3 code in two row
    blocks with signed scales, f32 specials, int8 with group scales."""
    cases = []
    codes16 = np.arange(65536, dtype=np.uint32).astype(np.uint16).reshape(256, 256)
    for fmt in (synth.FMT_F16, synth.FMT_BF16):
        cases.append(synth.QMatrix(fmt, 256, 256, 256, codes16.copy(), None, None))
    e = np.arange(256, dtype=np.uint8)
    q8 = np.stack([np.roll(e, r) for r in range(130)])                  # 130 rows: two row blocks
    s = np.array([[0.5, -3e-3], [-2.0 ** -20, 7e-5]], np.float32)
    cases.append(synth.QMatrix(synth.FMT_FP8_BLOCK, 130, 256, 128, q8, None, s))
    w = synth.rng_for(6100).integers(0, 2**32, size=(4, 64), dtype=np.uint64).astype(np.uint32)
    w[0, :8] = [0, 0x80000000, 0x7F800000, 0xFF800000, 1, 0x807FFFFF, 0x7F7FFFFF, 0x7FC00000]
    cases.append(synth.QMatrix(synth.FMT_F32, 4, 64, 64, w.view(np.float32), None, None))
    qi = np.tile(np.arange(256, dtype=np.uint8).view(np.int8), (2, 1))
    si = synth.rng_for(6101).uniform(-1e-2, 1e-2, size=(2, 8)).astype(np.float32)
    cases.append(synth.QMatrix(synth.FMT_I8_GS, 2, 256, 32, qi, None, si))
    for m in cases:
        got = host(dq.dqg_dequant(up(m)))
        assert same_bits_or_nan(got, oracle.dequant(m)), f"fmt {m.fmt}: dequant bits differ"


# ---------------------------------------------------------------------------
# matmul
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("i,spec", list(enumerate(SPECS)), ids=IDS)
def test_one_hot_is_exact(i, spec):
    """x = e_k: y[o] is the dequantised weight exactly (block and group
    scales land on the right rows and inputs)."""
    m = _m(i, spec)
    K = m.K
    ks = sorted(set([0, 1, K - 1, K // 2] + list(synth.rng_for(6200, i).integers(0, K, 12))))
    x = np.zeros((len(ks), K), np.float32)
    for j, k in enumerate(ks):
        x[j, k] = 1.0
    y = host(dq.dqg_matmul(up(m), dev_f32(x)))
    d = oracle.dequant(m)
    for j, k in enumerate(ks):
        assert np.array_equal(y[j], d[:, k]), f"{spec}: column {k}"


@pytest.mark.parametrize("S", [1, 2, 3, 4, 5, 8, 9, 16, 20, 33])
@pytest.mark.parametrize("i,spec", list(enumerate(SPECS)), ids=IDS)
def test_matmul_matches_oracle(i, spec, S):
    m = _m(i, spec)
    x = synth.activations(S, m.K, 6300 + i, S)
    y = host(dq.dqg_matmul(up(m), dev_f32(x)))
    yr, a = oracle.gemv(m, x)
    assert_close(y, yr, a, f"matmul {spec} S={S}")


GEMM = [(12, 130, 1024, None), (12, 256, 4096, None), (13, 77, 2048, 64), (13, 130, 1024, 32),
        (14, 77, 1024, None), (14, 300, 2080, None)]


@pytest.mark.parametrize("S", [8, 9, 16, 47, 64, 65, 96, 130, 200])
@pytest.mark.parametrize("spec", GEMM, ids=lambda s: f"fmt{s[0]}_{s[1]}x{s[2]}")
def test_gemm_route_matches_oracle(spec, S):
    """Both sides of the cut-over, the matrix-core route with token tiles of
    16, 32 and 64 per block."""
    fmt, O, K, gs = spec
    m = synth.matrix(fmt, O, K, gs, 6400, fmt, O, K)
    x = synth.activations(S, K, 6401, S, K)
    y = host(dq.dqg_matmul(up(m), dev_f32(x)))
    yr, a = oracle.gemv(m, x)
    assert_close(y, yr, a, f"gemm {spec} S={S}")


@pytest.mark.parametrize("fmt", [10, 11, 12, 13, 14])
def test_matmul_batch_invariant(fmt):
    """Per-row route: each token's row has the same bits alone and in a batch of 8."""
    spec = [s for s in SPECS if s[0] == fmt][1]
    m = _m(100 + fmt, spec)
    W = up(m)
    x = synth.activations(8, m.K, 6500 + fmt)
    yb = host(dq.dqg_matmul(W, dev_f32(x)))
    for t in range(8):
        y1 = host(dq.dqg_matmul(W, dev_f32(x[t:t + 1])))
        assert yb[t].tobytes() == y1[0].tobytes(), (spec, t)


@pytest.mark.parametrize("fmt", [1, 11, 12, 13, 14])
def test_matmul_6144_one_token_in_batch(fmt):
    """K = 6144 of 16-input chunks (int8, E4M3, int8-gs) or 8-input ones (bf16, f16): one token
    alone takes the one-row kernel (6 or 12 steps), a batch of 8 the general row kernel; each token
    has the same bits either way, and each token alone matches the oracle."""
    m = synth.matrix(fmt, 300, 6144, 64 if fmt == 13 else None, 6950, fmt)
    W = up(m)
    x = synth.activations(8, 6144, 6951, fmt)
    yb = host(dq.dqg_matmul(W, dev_f32(x)))
    yr, a = oracle.gemv(m, x)
    for t in range(8):
        y1 = host(dq.dqg_matmul(W, dev_f32(x[t:t + 1])))
        assert yb[t].tobytes() == y1[0].tobytes(), (fmt, t)
        assert_close(y1, yr[t:t + 1], a[t:t + 1], f"fmt {fmt} 6144 token {t}")


# ---------------------------------------------------------------------------
# gate_up and the expert group
# ---------------------------------------------------------------------------

GU = [(10, 77, 1028, None), (11, 130, 1032, None), (12, 130, 1024, None), (13, 64, 2048, 64),
      (14, 77, 1024, None)]


@pytest.mark.parametrize("S", [1, 2, 4, 5, 8, 32, 40])
@pytest.mark.parametrize("spec", GU, ids=lambda s: f"fmt{s[0]}_{s[1]}x{s[2]}")
def test_gate_up_matches_oracle(spec, S):
    fmt, I, H, gs = spec
    G = synth.matrix(fmt, I, H, gs, 6600, fmt, 0)
    U = synth.matrix(fmt, I, H, gs, 6600, fmt, 1)
    x = synth.activations(S, H, 6601, S)
    h = host(dq.dqg_gate_up(up(G), up(U), dev_f32(x)))
    r = oracle.gate_up(G, U, x)
    assert_close(h, r["h"], r["nh"], f"gate_up {spec} S={S}")


@pytest.mark.parametrize("fmt", [11, 12, 13, 14])
def test_gate_up_6144_one_token_in_batch(fmt):
    """gate_up over 6144 inputs: one token alone takes the one-row kernel (6 or 12 steps), a batch
    of 4 the general row kernel (from 8 tokens E4M3 and f16 take the matrix cores); each token has
    the same bits either way and matches the oracle."""
    gs = 64 if fmt == 13 else None
    G = synth.matrix(fmt, 200, 6144, gs, 6960, fmt, 0)
    U = synth.matrix(fmt, 200, 6144, gs, 6960, fmt, 1)
    x = synth.activations(4, 6144, 6961, fmt)
    hb = host(dq.dqg_gate_up(up(G), up(U), dev_f32(x)))
    r = oracle.gate_up(G, U, x)
    for t in range(4):
        h1 = host(dq.dqg_gate_up(up(G), up(U), dev_f32(x[t:t + 1])))
        assert hb[t].tobytes() == h1[0].tobytes(), (fmt, t)
        assert_close(h1, r["h"][t:t + 1], r["nh"][t:t + 1], f"gate_up fmt {fmt} 6144 token {t}")


@pytest.mark.parametrize("S", [1, 40])
@pytest.mark.parametrize("fmt", [11, 12])
def test_gate_up_clamped(fmt, S):
    G = synth.matrix(fmt, 130, 1024, None, 6700, 0)
    U = synth.matrix(fmt, 130, 1024, None, 6700, 1)
    x = synth.activations(S, 1024, 6701, S) * np.float32(30.0)
    limit = 0.5
    h = host(dq.dqg_gate_up_clamped(up(G), up(U), dev_f32(x), limit))
    r = oracle.gate_up(G, U, x, limit)
    assert_close(h, r["h"], r["nh"], f"clamped gate_up fmt {fmt} S={S}")


@pytest.mark.parametrize("S", [1, 40])
@pytest.mark.parametrize("fmt", [4, 12])
def test_gate_up_far_negative_gate(fmt, S):
    """Gate values far below -88.7, where exp(-g) is beyond f32: silu(g)
    keeps its subnormal value instead of collapsing to -0."""
    G = synth.matrix(fmt, 130, 1024, 32 if fmt == 4 else None, 6750, 0)
    U = synth.matrix(fmt, 130, 1024, 32 if fmt == 4 else None, 6750, 1)
    x = synth.activations(S, 1024, 6751, S) * np.float32(80.0 if fmt == 4 else 400.0)
    h = host(dq.dqg_gate_up(up(G), up(U), dev_f32(x)))
    r = oracle.gate_up(G, U, x)
    g = r["g"]
    log(f"  gates in (-104, -88.7): {int(((g > -104) & (g < -88.7)).sum())} of {g.size}")
    assert_close(h, r["h"], r["nh"], f"far negative gate fmt {fmt} S={S}")


GROUPS = [  # (gate/up fmt, gs, down fmt, down gs)
    (10, None, 10, None), (11, None, 11, None), (12, None, 12, None), (13, 64, 13, 64),
    (14, None, 14, None), (4, 32, 13, 32), (12, None, 4, 32), (11, None, 12, None),
]


@pytest.mark.parametrize("S", [1, 2, 3])
@pytest.mark.parametrize("fmts", GROUPS, ids=lambda f: f"fmt{f[0]}_down{f[2]}")
def test_group_matches_oracle(fmts, S):
    fmt, gs, dfmt, dgs = fmts
    E, k, H, I = 9, 3, 256, 384
    hs = [synth.expert(fmt, H, I, gs, 6800, i, down_fmt=dfmt, down_gs=dgs) for i in range(E + 1)]
    table = dq.ExpertTable([dq.Expert.upload(h) for h in hs])
    ids, w = synth.routing(S, E, k, 6801, S)
    x = synth.activations(S, H, 6802, S)
    check_group(hs, table, ids, w, E, x, f"group {fmts} S={S}")
    table.close()


# ---------------------------------------------------------------------------
# full size: 6144 x 6144 dense, every output against the oracle
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("S", [1, 4])
@pytest.mark.parametrize("fmt", [11, 12, 13, 14])
def test_full_size_6144(fmt, S):
    m = synth.matrix(fmt, 6144, 6144, 64 if fmt == 13 else None, 6900, fmt)
    x = synth.activations(S, 6144, 6901, S)
    y = host(dq.dqg_matmul(up(m), dev_f32(x)))
    yr, a = oracle.gemv(m, x)
    log(f"  worst normalised error {assert_close(y, yr, a, f'fmt {fmt} 6144 S={S}'):.2e}")


def test_full_size_fp8_group_256top8_shared():
    """The E4M3 expert group on the 6144 x 2048 shape, 257 experts, 2 tokens."""
    import gc
    from gpu_helpers import HostExperts, dev_i32, upload_experts
    c = synth.WORKLOADS["fp8b128_expert_group_256top8_shared"]
    S = 2
    ids, w = synth.routing(S, c["E"], c["k"], c["seed"], S)
    keep = set(ids.ravel().tolist()) | {c["E"]}
    log(f"  drawing {c['E'] + 1} E4M3 experts ({len(keep)} kept on the host)")
    dev, hosts = upload_experts(c["fmt"], c["H"], c["I"], c["gs"], c["seed"], c["E"] + 1, keep=keep)
    table = dq.ExpertTable(dev)
    x = synth.activations(S, c["H"], c["seed"], 300)
    check_group(HostExperts(c["E"] + 1, hosts), table, ids, w, c["E"], x, "fp8 group S=2")
    table.close()
    del dev, table
    gc.collect()
    torch.cuda.empty_cache()
