"""Parity of the clamped SwiGLU (swiglu_limit) with the CPU oracle, through the C ABI.

dqg_gate_up_clamped on the per-row and GEMM routes, and dqg_expert_group
with the table's limit.  Bar: as for the plain SwiGLU, within 1e-5 of the
propagated normaliser (the clamps are 1-Lipschitz, so the oracle's
normaliser, taken at the clamped values, still bounds the error's reach).
A limit of +inf gives the plain SwiGLU's bits.
"""
import math

import numpy as np
import pytest
import torch

import oracle
import synth
from gpu_helpers import assert_close, check_group, dev_f32, dev_i32, host, log

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


SPECS = [(1, 96, 512, None), (4, 77, 2240, 32), (5, 64, 4160, 64), (7, 130, 2240, 32)]


@pytest.mark.parametrize("limit", [0.05, 0.5, 2.0])
@pytest.mark.parametrize("S", [1, 4, 8, 40])   # 40 tokens: the GEMM route (int8, int4, MXFP4)
@pytest.mark.parametrize("spec", SPECS, ids=lambda s: f"fmt{s[0]}_{s[1]}x{s[2]}")
def test_gate_up_clamped_matches_oracle(spec, S, limit):
    fmt, I, H, gs = spec
    G = synth.matrix(fmt, I, H, gs, 9500, 0)
    U = synth.matrix(fmt, I, H, gs, 9500, 1)
    x = synth.activations(S, H, 9501, S)
    h = host(dq.dqg_gate_up_clamped(up(G), up(U), dev_f32(x), limit))
    r = oracle.gate_up(G, U, x, limit)
    plain = oracle.gate_up(G, U, x)
    clamped = np.mean((plain["g"] > limit) | (np.abs(plain["u"]) > limit))
    assert clamped > 0.05, f"limit {limit} clamps too little of this draw ({clamped:.2f})"
    assert_close(h, r["h"], r["nh"], f"clamped gate_up {spec} S={S} L={limit}")


@pytest.mark.parametrize("S", [1, 40])
def test_gate_up_clamped_inf_is_plain(S):
    G = synth.matrix(4, 77, 2240, 32, 9510, 0)
    U = synth.matrix(4, 77, 2240, 32, 9510, 1)
    x = synth.activations(S, 2240, 9511, S)
    a = host(dq.dqg_gate_up_clamped(up(G), up(U), dev_f32(x), math.inf))
    b = host(dq.dqg_gate_up(up(G), up(U), dev_f32(x)))
    assert a.tobytes() == b.tobytes()


@pytest.mark.parametrize("S", [1, 3, 5])
def test_group_with_table_limit(S):
    E, k, H, I = 10, 4, 256, 128
    hs = [synth.expert(4, H, I, 32, 9600, i) for i in range(E + 1)]
    table = dq.ExpertTable([dq.Expert.upload(h) for h in hs])
    ids, w = synth.routing(S, E, k, 9601, S)
    x = synth.activations(S, H, 9602, S)
    for limit in (0.3, 1.0):
        table.set_swiglu_limit(limit)
        check_group(hs, table, ids, w, E, x, f"group S={S} L={limit}", limit=limit)
    table.set_swiglu_limit(math.inf)
    check_group(hs, table, ids, w, E, x, f"group S={S} back to the plain SwiGLU")
    with pytest.raises(dq.DqgError):
        table.set_swiglu_limit(0.0)
    table.close()
