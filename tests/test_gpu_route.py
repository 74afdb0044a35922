"""Parity of the device router (dqg_route) with the CPU oracle, through the C ABI.

Bars:
- Without a bias the pick compares the f32 logits themselves on both sides,
  so ids must match bit for bit, ties included (lower index first).
- Weights: |w_gpu - w_ref| <= 1e-5 * |w_ref| + 1e-37.  The bound comes from
  the f32 arithmetic: expf within 2 ulp, the softmax sum over at most 16
  values per lane plus a 6-level wave tree, one division, the renormalising
  sum over at most 64 picks, one division and one product: under 100 ulp
  (6e-6) in all.  The absolute term covers scores that underflow f32.
- With a bias the pick key is the f32 p + bias on the device and the f64 one
  in the oracle, so near-ties may fall either way.  The test checks what is
  unique: every picked expert's f64 key is at least every unpicked one's
  minus 4e-6 (the key's rounding bound: 2e-6 on p, 1.2e-7 on the f32 add),
  the picks are distinct, and they come in key order within the same band.
"""
import numpy as np
import pytest
import torch

import oracle
import synth
from gpu_helpers import assert_close, dev_f32, dev_i32, host, log, scratch_h

pytestmark = pytest.mark.gpu

if torch.cuda.is_available():
    import dequant_gemv_expert_amd as dq
else:   # collected on CPU-only hosts, never run there
    dq = None

W_RTOL, W_ATOL = 1e-5, 1e-37
KEY_BAND = 4e-6


@pytest.fixture(autouse=True)
def _announce(request):
    log(f"[gpu] start {request.node.nodeid}")
    yield
    torch.cuda.synchronize()
    log(f"[gpu] done  {request.node.nodeid}")


def _route_gpu(lg, k, mode, renorm=False, bias=None, w_scale=1.0):
    ids, w = dq.dqg_route(dev_f32(lg), k, mode, renorm, None if bias is None else dev_f32(bias), w_scale)
    return host(ids), host(w)


def _check_weights(w_gpu, w_ref, what):
    w_gpu = w_gpu.astype(np.float64)
    bad = np.abs(w_gpu - w_ref) > W_RTOL * np.abs(w_ref) + W_ATOL
    assert not bad.any(), f"{what}: {int(bad.sum())} weights off; gpu {w_gpu[bad][:4]} ref {w_ref[bad][:4]}"


SHAPES = [  # (S, E, k): E spans 1..16 values per lane, ragged E, k up to 64 and k = E
    (1, 8, 1), (1, 64, 8), (3, 256, 8), (5, 384, 8), (2, 512, 10), (4, 1000, 16), (3, 1024, 64),
    (2, 70, 64), (6, 33, 33), (1, 1, 1),
]


@pytest.mark.parametrize("mode", [0, 1])
@pytest.mark.parametrize("renorm", [False, True])
@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: f"S{s[0]}_E{s[1]}_k{s[2]}")
def test_route_matches_oracle(mode, renorm, shape):
    S, E, k = shape
    lg = synth.router_logits(S, E, 8000, S, E, k)
    w_scale = 2.5 if renorm else 1.0
    ids, w = _route_gpu(lg, k, mode, renorm, None, w_scale)
    r = oracle.route(lg, k, mode, renorm, None, w_scale)
    assert np.array_equal(ids, r["ids"]), f"ids differ: gpu {ids[:2]} ref {r['ids'][:2]}"
    _check_weights(w, r["w"], f"route mode {mode} renorm {renorm} {shape}")


@pytest.mark.parametrize("mode", [0, 1])
def test_route_ties_go_to_lower_index(mode):
    lg = np.zeros((3, 200), np.float32)
    lg[1, 150:] = 1.0                               # 50 equal leaders at the end
    lg[2] = np.repeat(np.arange(20, dtype=np.float32), 10)[::-1]   # blocks of 10 equal values
    ids, w = _route_gpu(lg, 12, mode, True)
    r = oracle.route(lg, 12, mode, True)
    assert np.array_equal(ids, r["ids"])
    assert ids[0].tolist() == list(range(12))
    assert ids[1].tolist() == list(range(150, 162))
    _check_weights(w, r["w"], "ties")


@pytest.mark.parametrize("mode", [0, 1])
def test_route_extreme_logits(mode):
    rng = synth.rng_for(8100, mode)
    lg = (rng.standard_normal((4, 96)) * 200).astype(np.float32)   # exp over- and underflows
    lg[3] = 1e4
    lg[3, 7] = 1e4 + 1
    ids, w = _route_gpu(lg, 8, mode, False)
    r = oracle.route(lg, 8, mode, False)
    assert np.array_equal(ids, r["ids"])
    assert np.all(np.isfinite(w))
    _check_weights(w, r["w"], "extreme logits")


def _check_picks(ids, key, k, what):
    S, E = key.shape
    for t in range(S):
        picked = [int(e) for e in ids[t]]
        assert len(set(picked)) == k and all(0 <= e < E for e in picked), (what, t, picked)
        rest = [e for e in range(E) if e not in set(picked)]
        low = min(key[t, e] for e in picked)
        high = max((key[t, e] for e in rest), default=-np.inf)
        assert low >= high - KEY_BAND, (what, t, low, high)
        for a, b in zip(picked, picked[1:]):
            assert key[t, a] >= key[t, b] - KEY_BAND, (what, t, a, b)


@pytest.mark.parametrize("mode", [0, 1])
@pytest.mark.parametrize("renorm", [False, True])
@pytest.mark.parametrize("shape", [(4, 64, 8), (3, 384, 8), (2, 1024, 32)], ids=lambda s: f"S{s[0]}_E{s[1]}_k{s[2]}")
def test_route_with_bias(mode, renorm, shape):
    S, E, k = shape
    lg = synth.router_logits(S, E, 8200, S, E, k)
    bias = synth.router_bias(E, 8201, E)
    ids, w = _route_gpu(lg, k, mode, renorm, bias)
    r = oracle.route(lg, k, mode, renorm, bias)
    _check_picks(ids, r["key"], k, f"bias mode {mode}")
    # the weights of the device's own picks: the oracle's scores of those ids
    full = oracle.route(lg, E, mode, False)
    p = np.empty((S, E))
    for t in range(S):
        p[t, full["ids"][t]] = full["w"][t]
    want = np.take_along_axis(p, ids.astype(np.int64), axis=1)
    if renorm:
        want = want / want.sum(axis=1, keepdims=True)
    _check_weights(w, want, f"bias weights mode {mode}")


def test_route_batch_invariant():
    lg = synth.router_logits(9, 384, 8300)
    ids, w = _route_gpu(lg, 8, 0, True)
    for t in range(9):
        i1, w1 = _route_gpu(lg[t:t + 1], 8, 0, True)
        assert np.array_equal(i1[0], ids[t])
        assert w1[0].tobytes() == w[t].tobytes()


def test_route_then_expert_group_on_device():
    """logits -> dqg_route -> dqg_expert_group with no host step, against the oracle's chain."""
    E, k, S, H, I = 16, 4, 3, 256, 128
    hs = [synth.expert(4, H, I, 32, 8400, i) for i in range(E + 1)]
    table = dq.ExpertTable([dq.Expert.upload(h) for h in hs])
    lg = synth.router_logits(S, E, 8401)
    x = synth.activations(S, H, 8402)
    ids_d, w_d = dq.dqg_route(dev_f32(lg), k, dq.DQG_ROUTE_SOFTMAX, True)
    scratch = table.scratch(S, k)
    y = host(dq.dqg_expert_group(table, ids_d, w_d, E, dev_f32(x), scratch=scratch))
    r = oracle.route(lg, k, 0, True)
    assert np.array_equal(host(ids_d), r["ids"])
    # the oracle's group on the device's f32 weights (the weights' own check is above)
    yd, ad = oracle.expert_group_down(hs, r["ids"], host(w_d), E, scratch_h(scratch, S, k, I))
    assert_close(y, yd, ad, "route then group: down and combine on the device's h")
    yr, a = oracle.expert_group(hs, r["ids"], host(w_d), E, x)
    assert_close(y, yr, a, "route then group")
    table.close()


def test_route_full_size_mxfp4_router():
    """The MXFP4 workload's router shape: 8 tokens, 384 experts, top-8, renormalised."""
    lg = synth.router_logits(8, 384, 8500)
    ids, w = _route_gpu(lg, 8, 0, True)
    r = oracle.route(lg, 8, 0, True)
    assert np.array_equal(ids, r["ids"])
    _check_weights(w, r["w"], "384 experts")
    assert np.allclose(w.sum(axis=1), 1.0, rtol=1e-6)
