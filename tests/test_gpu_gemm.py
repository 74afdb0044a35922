"""Parity of the matrix-core GEMM route with the CPU oracle.

dqg_matmul (from 32 tokens for int4 and MXFP4, 48 for int8) and
dqg_gate_up (from 32) take the route when K is a multiple of 32; the sizes
below straddle the cut-overs, so both routes are checked at 16..130 tokens.  Bar: as for
the GEMV route, every output within 1e-5 of its row's normaliser
sum_k |w*x|.  The route's own error
terms are far below it: x is split as f16 hi + lo (x - hi - lo < 2^-22 |x|),
the products of f16 patterns and f16 parts are exact in the matrix cores,
and the sums run in f32.
"""
import numpy as np
import pytest
import torch

import oracle
import synth
from gpu_helpers import assert_close, dev_f32, host, log

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


SHAPES = [  # (fmt, O, K, gs): ragged rows, K not a multiple of the 128-input step, group sizes
    (1, 77, 512, None), (1, 130, 2080, None),
    (2, 45, 96, None), (2, 300, 2240, None),
    (4, 1, 32, 32), (4, 77, 2240, 32), (4, 130, 4128, 32), (4, 64, 2048, 64), (4, 50, 1024, 128),
    (7, 77, 2240, 32), (7, 300, 4128, 32),
]


@pytest.mark.parametrize("S", [16, 31, 32, 33, 47, 48, 64, 100])
@pytest.mark.parametrize("spec", SHAPES, ids=lambda s: f"fmt{s[0]}_{s[1]}x{s[2]}")
def test_gemm_matmul_matches_oracle(spec, S):
    fmt, O, K, gs = spec
    m = synth.matrix(fmt, O, K, gs, 9000, fmt, O, K)
    x = synth.activations(S, K, 9001, S, K)
    y = host(dq.dqg_matmul(up(m), dev_f32(x)))
    yr, a = oracle.gemv(m, x)
    assert_close(y, yr, a, f"gemm {spec} S={S}")


@pytest.mark.parametrize("S", [16, 40, 64, 65, 130])
@pytest.mark.parametrize("spec", [(1, 96, 512, None), (4, 77, 2240, 32), (4, 130, 2048, 64), (7, 64, 2240, 32)],
                         ids=lambda s: f"fmt{s[0]}_{s[1]}x{s[2]}")
def test_gemm_gate_up_matches_oracle(spec, S):
    fmt, I, H, gs = spec
    G = synth.matrix(fmt, I, H, gs, 9100, 0)
    U = synth.matrix(fmt, I, H, gs, 9100, 1)
    x = synth.activations(S, H, 9101, S)
    h = host(dq.dqg_gate_up(up(G), up(U), dev_f32(x)))
    r = oracle.gate_up(G, U, x)
    assert_close(h, r["h"], r["nh"], f"gemm gate_up {spec} S={S}")


@pytest.mark.parametrize("scale", [1e-8, 1.0, 3e4, 1e7])
def test_gemm_wide_activation_range(scale):
    """x scaled into f16 range per token and step: tiny, large, and beyond f16's max."""
    m = synth.matrix(4, 130, 2048, 32, 9200, 0)
    x = synth.activations(40, 2048, 9201) * np.float32(scale)
    x[3, :100] *= np.float32(1e4)    # one token with a few large inputs
    x[5] = 0.0                       # an all-zero token
    y = host(dq.dqg_matmul(up(m), dev_f32(x)))
    yr, a = oracle.gemv(m, x)
    assert np.all(y[5] == 0)
    assert_close(y, yr, a, f"gemm x scale {scale}")


def test_gemm_batch_invariant():
    """Within the GEMM route a token's outputs have the same bits whatever the batch."""
    m = synth.matrix(4, 200, 4096, 32, 9300, 0)
    x = synth.activations(96, 4096, 9301)
    y96 = host(dq.dqg_matmul(up(m), dev_f32(x)))
    for lo, n in ((0, 32), (16, 40), (40, 56)):
        yn = host(dq.dqg_matmul(up(m), dev_f32(x[lo:lo + n])))
        assert yn.tobytes() == y96[lo:lo + n].tobytes(), (lo, n)


def test_gemm_zero_scales():
    m = synth.matrix(4, 64, 1024, 32, 9400, 0)
    m.scales[:] = 0
    x = synth.activations(48, 1024, 9401)
    y = host(dq.dqg_matmul(up(m), dev_f32(x)))
    assert np.all(y == 0)


def test_gemm_full_size_int4_6144():
    """The dense int4-g32 6144 x 6144 matrix at a 256-token prefill; sampled rows of the oracle."""
    c = synth.WORKLOADS["int4g32_gemv_6144x6144"]
    m = synth.matrix(c["fmt"], c["O"], c["K"], c["gs"], c["seed"], 0)
    x = synth.activations(256, c["K"], c["seed"], 256)
    y = host(dq.dqg_matmul(up(m), dev_f32(x)))
    rows = [0, 1, 7, 127, 128, 3071, 6143]
    sub = synth.QMatrix(m.fmt, len(rows), m.K, m.gs, m.q[rows], None if m.q2 is None else m.q2[rows],
                        m.scales[rows])
    toks = [0, 1, 63, 64, 200, 255]
    yr, a = oracle.gemv(sub, x[toks])
    assert_close(y[np.ix_(toks, rows)], yr, a, "gemm 6144 S=256 sampled")
