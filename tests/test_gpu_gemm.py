"""Parity of the matrix-core GEMM route with the CPU oracle.

dqg_matmul (from 9 tokens) and dqg_gate_up (from 8, 9 for int8 codes) take
the route when K is a multiple of 32; the batches below straddle the
cut-overs and the token-tile sizes.  Bar: as for the GEMV route, every
output within 1e-5 of its row's normaliser sum_k |w*x|.  The route's own
error terms are far below it: x is split as f16 hi + lo (x - hi - lo <
2^-22 |x|), the products of f16 patterns and f16 parts are exact in the
matrix cores, and the sums run in f32.

The sum over K is taken per 512-input chunk and the chunk sums are added in
order; a grid too small for the chip computes the chunks in separate blocks
(split-K) and adds them in a second kernel.  Small matrices and batches take
the split path; the large-grid tests below take the other one, and the bits
of both agree.
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


@pytest.mark.parametrize("S", [8, 9, 16, 31, 33, 64, 65, 100])
@pytest.mark.parametrize("spec", SHAPES, ids=lambda s: f"fmt{s[0]}_{s[1]}x{s[2]}")
def test_gemm_matmul_matches_oracle(spec, S):
    fmt, O, K, gs = spec
    m = synth.matrix(fmt, O, K, gs, 9000, fmt, O, K)
    x = synth.activations(S, K, 9001, S, K)
    y = host(dq.dqg_matmul(up(m), dev_f32(x)))
    yr, a = oracle.gemv(m, x)
    assert_close(y, yr, a, f"gemm {spec} S={S}")


@pytest.mark.parametrize("S", [7, 8, 9, 40, 65, 130])
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
    """x scaled into f16 range per token and 32-input window: tiny, large, and beyond f16's max."""
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
    for lo, n in ((0, 32), (16, 40), (40, 56), (5, 9), (80, 16)):
        yn = host(dq.dqg_matmul(up(m), dev_f32(x[lo:lo + n])))
        assert yn.tobytes() == y96[lo:lo + n].tobytes(), (lo, n)


# One tile of up to 16 tokens with 4-bit codes, a scale per 32 inputs and K
# of whole 512-input chunks: the split-K chunks take the small-batch kernel
# (16-byte code loads, a transpose across lane groups to the matrix cores'
# layout), whose bits must be those of the general kernel's chunks (a
# 48-token batch).  Row counts ragged against its 256-row (gate/up: 128) blocks.
SMALL = [(4, 77, 1024), (4, 300, 2048), (7, 513, 1536), (7, 40, 512 * 5), (4, 6144, 6144)]


@pytest.mark.parametrize("spec", SMALL, ids=lambda s: f"fmt{s[0]}_{s[1]}x{s[2]}")
def test_gemm_small_batch_kernel(spec):
    fmt, O, K = spec
    i = SMALL.index(spec)
    m = synth.matrix(fmt, O, K, 32, 9900 + i, fmt)
    x = synth.activations(48, K, 9950 + i)
    W = up(m)
    y48 = host(dq.dqg_matmul(W, dev_f32(x)))
    for lo, n in ((0, 9), (9, 16), (30, 13)):
        yn = host(dq.dqg_matmul(W, dev_f32(x[lo:lo + n])))
        assert yn.tobytes() == y48[lo:lo + n].tobytes(), (spec, lo, n)
    rows = list(range(O)) if O <= 600 else [0, 1, 255, 256, 3000, O - 1]
    yr, a = oracle.gemv(_sampled_rows(m, rows), x[9:25])
    assert_close(y48[9:25][:, rows], yr, a, f"small-batch gemm {spec} S=16")


@pytest.mark.parametrize("spec", [(4, 300, 2048), (7, 129, 1024)], ids=lambda s: f"fmt{s[0]}_{s[1]}x{s[2]}")
def test_gemm_gate_up_small_batch_kernel(spec):
    fmt, O, K = spec
    G = synth.matrix(fmt, O, K, 32, 9960, 0)
    U = synth.matrix(fmt, O, K, 32, 9960, 1)
    x = synth.activations(48, K, 9961)
    g, u = up(G), up(U)
    h48 = host(dq.dqg_gate_up(g, u, dev_f32(x)))
    for lo, n in ((0, 9), (20, 16)):
        hn = host(dq.dqg_gate_up(g, u, dev_f32(x[lo:lo + n])))
        assert hn.tobytes() == h48[lo:lo + n].tobytes(), (spec, lo, n)
    r = oracle.gate_up(G, U, x[20:36])
    assert_close(h48[20:36], r["h"], r["nh"], f"small-batch gemm gate_up {spec} S=16")


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


def _sampled_rows(m, rows):
    return synth.QMatrix(m.fmt, len(rows), m.K, m.gs, m.q[rows], None if m.q2 is None else m.q2[rows],
                         None if m.scales is None else m.scales[rows])


@pytest.mark.parametrize("fmt", [4, 7])
def test_gemm_unsplit_matches_split(fmt):
    """8192 x 2080 (five K chunks, the last one 32 inputs) at 1024 tokens fills
    the chip without split-K (64 x 16 blocks); 64 of those tokens alone take
    split-K.  Same bits, and the large batch agrees with the oracle on sampled
    rows and tokens."""
    m = synth.matrix(fmt, 8192, 2080, 32, 9500, fmt)
    x = synth.activations(1024, 2080, 9501, fmt)
    W = up(m)
    y = host(dq.dqg_matmul(W, dev_f32(x)))
    for lo in (0, 500, 960):
        ys = host(dq.dqg_matmul(W, dev_f32(x[lo:lo + 64])))
        assert ys.tobytes() == y[lo:lo + 64].tobytes(), lo
    rows = [0, 1, 127, 128, 4095, 8191]
    toks = [0, 15, 16, 511, 1000, 1023]
    yr, a = oracle.gemv(_sampled_rows(m, rows), x[toks])
    assert_close(y[np.ix_(toks, rows)], yr, a, f"gemm fmt{fmt} 8192x2080 S=1024 sampled")


def test_gemm_gate_up_unsplit_matches_split():
    """gate_up: 4096 x 1056 (chunks 512, 512, 32) at 1024 tokens (64 x 16
    blocks, no split) against 64-token batches (split-K), and the oracle."""
    G = synth.matrix(4, 4096, 1056, 32, 9600, 0)
    U = synth.matrix(4, 4096, 1056, 32, 9600, 1)
    x = synth.activations(1024, 1056, 9601)
    g, u = up(G), up(U)
    h = host(dq.dqg_gate_up(g, u, dev_f32(x)))
    for lo in (0, 700):
        hs = host(dq.dqg_gate_up(g, u, dev_f32(x[lo:lo + 64])))
        assert hs.tobytes() == h[lo:lo + 64].tobytes(), lo
    rows = [0, 63, 64, 2047, 4095]
    toks = [0, 17, 640, 1023]
    r = oracle.gate_up(_sampled_rows(G, rows), _sampled_rows(U, rows), x[toks])
    assert_close(h[np.ix_(toks, rows)], r["h"], r["nh"], "gemm gate_up 4096x1056 S=1024 sampled")


def test_gemm_streams_share_the_split_workspace():
    """Split-K calls on two streams, interleaved, share the library's partials
    buffer and give the bits of the same calls made one at a time."""
    ms = [synth.matrix(4, 1024, 2048, 32, 9700, i) for i in range(2)]
    Ws = [up(m) for m in ms]
    xs = [dev_f32(synth.activations(S, 2048, 9701, S)) for S in (32, 96, 200)]
    want = {(i, j): host(dq.dqg_matmul(Ws[i], xs[j])) for i in range(2) for j in range(3)}
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    outs = {}
    torch.cuda.synchronize()
    for j in range(3):
        for i in range(2):
            with torch.cuda.stream(streams[i]):
                outs[i, j] = dq.dqg_matmul(Ws[i], xs[j])
    torch.cuda.synchronize()
    for key, y in outs.items():
        assert host(y).tobytes() == want[key].tobytes(), key


def test_gemm_graph_capture_replays():
    """A captured dqg_matmul (a stream under capture takes the unsplit kernel)
    replays with the eager call's bits, with eager split-K calls between
    replays and new inputs copied in."""
    m = synth.matrix(4, 1024, 2048, 32, 9800, 0)
    W = up(m)
    x_np = [synth.activations(48, 2048, 9801, r) for r in range(3)]
    x = dev_f32(x_np[0])
    y = torch.empty((48, 1024), dtype=torch.float32, device="cuda")
    dq.dqg_matmul(W, x, y)       # warm the library on this shape
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        dq.dqg_matmul(W, x, y)
    other = dev_f32(synth.activations(64, 2048, 9802))
    for r in range(3):
        x.copy_(dev_f32(x_np[r]))
        want = host(dq.dqg_matmul(W, x))          # eager, split-K
        y.zero_()
        g.replay()
        dq.dqg_matmul(W, other)                    # eager work between replays
        torch.cuda.synchronize()
        assert host(y).tobytes() == want.tobytes(), r
