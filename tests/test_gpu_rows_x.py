"""Parity of the one- to four-token row kernel (x staged once per block,
every load of a wave issued before its arithmetic) with the CPU oracle,
through the C ABI.

It takes K of one to four whole steps of 64 code chunks, so the shapes below
set K = n * 64 * (inputs per chunk) for n = 1..4 in every format (int3 at one
token only), with row counts ragged against its blocks (8 rows below 6144
rows, 24 from there up).  Bars as for the other
matmul tests: every output within 1e-5 of its row's normaliser, and a
token's bits the same alone and inside a batch of 8 (which takes the
general per-row kernel).
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


# inputs per code chunk, and a group size where the format has one
CHUNK = {1: (16, None), 2: (32, None), 4: (32, 32), 5: (64, 64), 7: (32, 32), 10: (4, None), 11: (8, None),
         12: (16, None), 13: (16, 64), 14: (8, None)}
CASES = [(fmt, n, O) for fmt in CHUNK for n, O in ((1, 37), (2, 24), (3, 61), (4, 5))]
# from 6144 rows up the blocks are 12 waves x 1 row at one token (int3 and several tokens:
# 12 x 2 and 8 x 3); these leave the last block ragged
CASES += [(4, 1, 6161), (7, 2, 6150), (1, 3, 6170), (5, 1, 6151), (11, 4, 6145), (13, 4, 6157)]
IDS = [f"fmt{f}_steps{n}_O{o}" for f, n, o in CASES]


def _bits_equal(a, b):
    return a.view(np.uint32).tobytes() == b.view(np.uint32).tobytes()


@pytest.mark.parametrize("case", CASES, ids=IDS)
def test_rows_x_matmul(case):
    fmt, n, O = case
    cw, gs = CHUNK[fmt]
    K = n * 64 * cw
    i = CASES.index(case)
    m = synth.matrix(fmt, O, K, gs, 7000 + i, fmt)
    W = dq.Matrix.upload(m)
    x = synth.activations(8, K, 7100 + i)
    yb = host(dq.dqg_matmul(W, dev_f32(x)))
    for S in (1, 2, 3, 4):
        y = host(dq.dqg_matmul(W, dev_f32(x[:S])))
        yr, a = oracle.gemv(m, x[:S])
        assert_close(y, yr, a, f"rows_x matmul {case} S={S}")
        for t in range(S):
            assert _bits_equal(y[t], yb[t]), (case, S, t)


@pytest.mark.parametrize("case", CASES[::3], ids=IDS[::3])
def test_rows_x_gate_up(case):
    fmt, n, O = case
    cw, gs = CHUNK[fmt]
    K = n * 64 * cw
    i = CASES.index(case)
    G = synth.matrix(fmt, O, K, gs, 7200 + i, 0)
    U = synth.matrix(fmt, O, K, gs, 7200 + i, 1)
    x = synth.activations(4, K, 7300 + i)
    for S in (1, 2, 4):
        h = host(dq.dqg_gate_up(dq.Matrix.upload(G), dq.Matrix.upload(U), dev_f32(x[:S])))
        r = oracle.gate_up(G, U, x[:S])
        assert_close(h, r["h"], r["nh"], f"rows_x gate_up {case} S={S}")
