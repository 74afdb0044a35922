"""Parity of the HIP path with the CPU oracle, through the C ABI.

Bars: dequantised weights bit for bit; outputs within 1e-5 of the per-row
normaliser sum_k |w*x|.  For the expert group that is the down rows' own
normaliser: the device's y against the oracle's down and combine applied to
the device's own h, normalised by sum_r |w| sum_i |D h| (+ the shared row's);
h itself within 1e-5 of its first-order error reach; and, as a second check,
the oracle's whole group with that reach carried through down.
"""
import gc
import math

import numpy as np
import pytest
import torch

import oracle
import pinlib
import synth
from gpu_helpers import (HostExperts, TOL, assert_close, check_group, dev_f32, dev_i32, host, log,
                         scratch_h, upload_experts)

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


def bits_equal(a: np.ndarray, b: np.ndarray) -> bool:
    return a.view(np.uint32).tobytes() == b.view(np.uint32).tobytes()


SMALL = [  # (fmt, O, K, gs)
    (1, 1, 16, None), (1, 77, 512, None), (1, 33, 2064, None),
    (2, 45, 96, None), (2, 300, 2240, None),
    (4, 1, 32, 32), (4, 77, 2240, 32), (4, 130, 4128, 32), (4, 64, 2048, 64), (4, 50, 1024, 128),
    (5, 3, 64, 64), (5, 77, 4160, 64), (5, 129, 8192, 64),
    (7, 1, 32, 32), (7, 77, 2240, 32), (7, 300, 4128, 32),
]


def _small(i, spec):
    fmt, O, K, gs = spec
    return synth.matrix(fmt, O, K, gs, 1000 + i, fmt)


# ---------------------------------------------------------------------------
# dequant: bits
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("i,spec", list(enumerate(SMALL)), ids=[f"fmt{s[0]}_{s[1]}x{s[2]}" for s in SMALL])
def test_dequant_bits_random(i, spec):
    m = _small(i, spec)
    got = host(dq.dqg_dequant(up(m)))
    want = oracle.dequant(m)
    assert bits_equal(got, want), f"{spec}: dequant bits differ"


def test_dequant_bits_all_codes_and_signed_zero():
    cases = []
    q = np.tile(np.arange(256, dtype=np.uint8), (2, 1))                  # every byte, K = 512
    for fmt, gs in ((4, 32), (4, 64), (2, 512), (7, 32)):
        s = synth.rng_for(3, fmt).uniform(-2e-2, 2e-2, size=(2, 512 // gs)).astype(np.float32)
        cases.append(synth.QMatrix(fmt, 2, 512, gs, q.copy(), None, s))
    q8 = np.tile(np.arange(256, dtype=np.uint8).view(np.int8), (2, 1))  # int8, with -128
    cases.append(synth.QMatrix(1, 2, 256, 256, q8, None, np.array([[3e-3], [-7e-3]], np.float32)))
    for code in range(8):                                                 # int3, every code
        lo = np.full((2, 4), (code & 3) * 0x55555555, np.uint32)
        hi = np.full((2, 2), 0xFFFFFFFF if code & 4 else 0, np.uint32)
        cases.append(synth.QMatrix(5, 2, 64, 64, lo, hi, np.array([[1e-2], [-1e-2]], np.float32)))
    low, high, _ = pinlib.golden_int3()
    cases.append(synth.QMatrix(5, 1, 64, 64, np.array([low], np.uint32), np.array([high], np.uint32),
                               np.array([[0.25]], np.float32)))
    for m in cases:
        got = host(dq.dqg_dequant(up(m)))
        want = oracle.dequant(m)
        assert bits_equal(got, want), f"fmt {m.fmt}: dequant bits differ"


# ---------------------------------------------------------------------------
# GEMV
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("i,spec", list(enumerate(SMALL)), ids=[f"fmt{s[0]}_{s[1]}x{s[2]}" for s in SMALL])
def test_one_hot_is_exact(i, spec):
    """x = e_k: the GPU's y[o] equals the dequantised weight exactly."""
    m = _small(i, spec)
    K = m.K
    ks = sorted(set([0, 1, K - 1, K // 2] + list(synth.rng_for(4, i).integers(0, K, 12))))
    x = np.zeros((len(ks), K), np.float32)
    for j, k in enumerate(ks):
        x[j, k] = 1.0
    y = host(dq.dqg_matmul(up(m), dev_f32(x)))
    d = oracle.dequant(m)
    for j, k in enumerate(ks):
        assert np.array_equal(y[j], d[:, k]), f"{spec}: column {k}"


@pytest.mark.parametrize("S", [1, 2, 3, 4, 5, 8, 9, 13])
@pytest.mark.parametrize("i,spec", list(enumerate(SMALL)), ids=[f"fmt{s[0]}_{s[1]}x{s[2]}" for s in SMALL])
def test_matmul_matches_oracle(i, spec, S):
    m = _small(i, spec)
    x = synth.activations(S, m.K, 2000 + i, S)
    y = host(dq.dqg_matmul(up(m), dev_f32(x)))
    yr, a = oracle.gemv(m, x)
    assert_close(y, yr, a, f"matmul {spec} S={S}")


def test_matmul_batch_invariant():
    """Each token's row has the same bits alone and inside a batch (of 8: the
    per-row route's largest)."""
    for i, spec in enumerate(SMALL[::3]):
        m = _small(i, spec)
        W = up(m)
        x = synth.activations(8, m.K, 2100 + i)
        yb = host(dq.dqg_matmul(W, dev_f32(x)))
        for t in range(8):
            y1 = host(dq.dqg_matmul(W, dev_f32(x[t:t + 1])))
            assert bits_equal(yb[t], y1[0]), (spec, t)


def test_zero_scales_give_zero():
    for i, spec in enumerate(SMALL[::2]):
        m = _small(i, spec)
        m.scales = np.zeros_like(m.scales)
        y = host(dq.dqg_matmul(up(m), dev_f32(synth.activations(3, m.K, 5))))
        assert np.all(y == 0), spec


# ---------------------------------------------------------------------------
# gate_up
# ---------------------------------------------------------------------------

GU = [(4, 64, 2048, 32), (4, 77, 96, 32), (7, 130, 2240, 32), (1, 50, 512, None), (5, 33, 4160, 64),
      (4, 2048, 6144, 32)]


@pytest.mark.parametrize("S", [1, 2, 4, 5, 8])
@pytest.mark.parametrize("spec", GU, ids=[f"fmt{s[0]}_{s[1]}x{s[2]}" for s in GU])
def test_gate_up_matches_oracle(spec, S):
    fmt, I, H, gs = spec
    G = synth.matrix(fmt, I, H, gs, 3000, 0)
    U = synth.matrix(fmt, I, H, gs, 3000, 1)
    x = synth.activations(S, H, 3001, S)
    h = host(dq.dqg_gate_up(up(G), up(U), dev_f32(x)))
    r = oracle.gate_up(G, U, x)
    assert_close(h, r["h"], r["nh"], f"gate_up {spec} S={S}")


# ---------------------------------------------------------------------------
# expert group (small)
# ---------------------------------------------------------------------------

def _small_group(n, fmt=4, gs=32, H=256, I=128, seed=4000, **kw):
    hs = [synth.expert(fmt, H, I, gs, seed, i, **kw) for i in range(n)]
    table = dq.ExpertTable([dq.Expert.upload(h) for h in hs])
    return hs, table


@pytest.mark.parametrize("S", [1, 2, 3, 4, 5, 8])
@pytest.mark.parametrize("shared", [True, False])
def test_group_small(S, shared):
    E, k = 12, 4
    hs, table = _small_group(E + 1)
    ids, w = synth.routing(S, E, k, 4100 + S)
    x = synth.activations(S, 256, 4200 + S)
    check_group(hs, table, ids, w, E if shared else None, x, f"group S={S} shared={shared}")


@pytest.mark.parametrize("fmts", [(7, 32, 4, 32), (4, 64, 1, None), (1, None, 7, 32), (5, 64, 4, 32)])
def test_group_mixed_formats(fmts):
    fmt, gs, dfmt, dgs = fmts
    hs, table = _small_group(7, fmt=fmt, gs=gs, down_fmt=dfmt, down_gs=dgs, seed=4300)
    ids, w = synth.routing(3, 6, 3, 4301)
    x = synth.activations(3, 256, 4302)
    check_group(hs, table, ids, w, 6, x, f"group mixed {fmts}")


def test_group_many_slots():
    """S*k > 64: the dedup ballots span several windows."""
    hs, table = _small_group(20)
    ids, w = synth.routing(20, 19, 8, 4400)
    x = synth.activations(20, 256, 4401)
    check_group(hs, table, ids, w, 19, x, "group S=20 k=8")


def test_group_repeated_id_in_a_token():
    hs, table = _small_group(8)
    ids = np.array([[3, 3, 5, 7], [5, 1, 3, 3]], np.int32)
    w = np.array([[0.4, 0.3, 0.2, 0.1], [0.25, 0.25, 0.25, 0.25]], np.float32)
    x = synth.activations(2, 256, 4500)
    check_group(hs, table, ids, w, 0, x, "group repeated ids")


def test_group_batch_invariant():
    hs, table = _small_group(13)
    ids, w = synth.routing(5, 12, 4, 4600)
    x = synth.activations(5, 256, 4601)
    yb = host(dq.dqg_expert_group(table, dev_i32(ids), dev_f32(w), 12, dev_f32(x)))
    for t in range(5):
        y1 = host(dq.dqg_expert_group(table, dev_i32(ids[t:t + 1]), dev_f32(w[t:t + 1]), 12,
                                      dev_f32(x[t:t + 1])))
        assert bits_equal(yb[t], y1[0]), t


# One token with k routed experts (6 to 8) and a shared one, I of 64 code
# chunks: the down launch that deals the shared expert's rows over the
# waves.  H is ragged against its 12-row blocks.
SPLIT_CASES = [(8, 160, 4, 32, 2048), (7, 224, 7, 32, 2048), (6, 64, 4, 32, 2048), (8, 80, 1, None, 1024)]


@pytest.mark.parametrize("case", SPLIT_CASES)
def test_group_one_token_split_down(case):
    k, H, fmt, gs, I = case
    E = k + 2
    seed = 4800 + SPLIT_CASES.index(case)
    hs, table = _small_group(E, fmt=fmt, gs=gs, H=H, I=I, seed=seed)
    ids, w = synth.routing(3, E - 1, k, seed)
    ids[1, k - 1] = ids[1, 0]   # an expert twice in one token
    x = synth.activations(3, H, seed)
    for t in range(3):
        check_group(hs, table, ids[t:t + 1], w[t:t + 1], E - 1, x[t:t + 1], f"split down {case} token {t}")
    # batch invariance: three tokens (the general down launch) against one at a time
    yb = host(dq.dqg_expert_group(table, dev_i32(ids), dev_f32(w), E - 1, dev_f32(x)))
    for t in range(3):
        y1 = host(dq.dqg_expert_group(table, dev_i32(ids[t:t + 1]), dev_f32(w[t:t + 1]), E - 1,
                                      dev_f32(x[t:t + 1])))
        assert bits_equal(yb[t], y1[0]), (case, t)
    # a bad id: the token's outputs are NaN and the call reports it
    bad = ids[:1].copy()
    bad[0, k // 2] = E + 5
    ticket, y, _ = dq.dqg_expert_group_issue(table, dev_i32(bad), dev_f32(w[:1]), E - 1, dev_f32(x[:1]))
    with pytest.raises(dq.DqgError) as ei:
        dq.dqg_expert_group_take(ticket)
    assert ei.value.code == -7
    assert np.all(np.isnan(host(y)))
    table.close()


# Several tokens with at least 8 units and I of 64 code chunks, H ragged
# against the down launch's 12-row blocks (14-row blocks for H of 6145 to
# 7168: 6176 and 7008), one expert named by two tokens.
MULTI_CASES = [(2, 8, True, 4, 32, 2048, 416), (3, 4, False, 4, 32, 2048, 224),
              (2, 6, True, 7, 32, 2048, 6176), (5, 3, True, 1, None, 1024, 160),
              (3, 4, False, 4, 32, 2048, 7008)]


@pytest.mark.parametrize("case", MULTI_CASES)
def test_group_multi_token_down(case):
    S, k, with_shared, fmt, gs, I, H = case
    E = 2 * k + 3
    seed = 4900 + MULTI_CASES.index(case)
    hs, table = _small_group(E, fmt=fmt, gs=gs, H=H, I=I, seed=seed)
    ids, w = synth.routing(S, E - 1, k, seed)
    ids[S - 1, k - 1] = ids[0, 0]   # one expert named by two tokens
    shared = E - 1 if with_shared else None
    x = synth.activations(S, H, seed)
    check_group(hs, table, ids, w, shared, x, f"multi-token down {case}")
    # batch invariance: the batch against one token at a time
    yb = host(dq.dqg_expert_group(table, dev_i32(ids), dev_f32(w), shared, dev_f32(x)))
    for t in range(S):
        y1 = host(dq.dqg_expert_group(table, dev_i32(ids[t:t + 1]), dev_f32(w[t:t + 1]), shared,
                                      dev_f32(x[t:t + 1])))
        assert bits_equal(yb[t], y1[0]), (case, t)
    # a bad id: that token's outputs are NaN, the others finite, and the call reports it
    bad = ids.copy()
    bad[S - 1, 1] = E + 9
    ticket, y, _ = dq.dqg_expert_group_issue(table, dev_i32(bad), dev_f32(w), shared, dev_f32(x))
    with pytest.raises(dq.DqgError) as ei:
        dq.dqg_expert_group_take(ticket)
    assert ei.value.code == -7
    yh = host(y)
    assert np.all(np.isnan(yh[S - 1])) and np.all(np.isfinite(yh[:S - 1]))
    table.close()


# One token routed to one expert with no shared expert (a single expert
# MLP), H and I whole multiples of 64 code chunks (1 to 4 of them per lane, or
# 6 and 12 for 6144 inputs of 16- and 8-input chunks):
# the group's unit launches, whose bits must be those of the general group
# launches (a batch of two tokens, one expert each).  H = 8192 leaves the
# down launch's last 24-row block ragged; int4 down at I = 1024 takes the
# general down launch after the unit gate/up launch.
UNIT_CASES = [  # gate/up format and group size, down's, H, I
    (4, 32, 4, 32, 2048, 2048), (4, 32, 4, 32, 8192, 2048), (4, 32, 4, 32, 6144, 1024),
    (7, 32, 7, 32, 6144, 2048), (5, 64, 4, 32, 4096, 2048), (1, None, 12, None, 3072, 1024),
    (13, 64, 13, 64, 4096, 1024), (11, None, 14, None, 1024, 512), (10, None, 10, None, 1024, 256),
    (12, None, 12, None, 6144, 2048), (14, None, 14, None, 6144, 1024),
]


@pytest.mark.parametrize("case", UNIT_CASES, ids=lambda c: f"fmt{c[0]}_down{c[2]}_H{c[4]}_I{c[5]}")
def test_group_single_expert(case):
    fmt, gs, dfmt, dgs, H, I = case
    seed = 5100 + UNIT_CASES.index(case)
    hs, table = _small_group(3, fmt=fmt, gs=gs, H=H, I=I, seed=seed, down_fmt=dfmt, down_gs=dgs)
    ids = np.array([[2], [0]], np.int32)
    w = np.array([[0.6180339], [1.0]], np.float32)
    x = synth.activations(2, H, seed)
    y1 = [check_group(hs, table, ids[t:t + 1], w[t:t + 1], None, x[t:t + 1], f"single expert {case} token {t}")[0]
          for t in range(2)]
    yb = host(dq.dqg_expert_group(table, dev_i32(ids), dev_f32(w), None, dev_f32(x)))
    for t in range(2):
        assert bits_equal(yb[t], y1[t][0]), (case, t)
    if case == UNIT_CASES[0]:
        table.set_swiglu_limit(0.5)
        check_group(hs, table, ids[:1], w[:1], None, x[:1], f"single expert {case} limit 0.5", limit=0.5)
        table.set_swiglu_limit(math.inf)
    # a bad id: every output NaN, and the call reports it; the next call clears the flag
    ticket, y, _ = dq.dqg_expert_group_issue(table, dev_i32(np.array([[7]], np.int32)), dev_f32(w[:1]), None,
                                             dev_f32(x[:1]))
    with pytest.raises(dq.DqgError) as ei:
        dq.dqg_expert_group_take(ticket)
    assert ei.value.code == -7
    assert np.all(np.isnan(host(y)))
    ticket, y, _ = dq.dqg_expert_group_issue(table, dev_i32(ids[:1]), dev_f32(w[:1]), None, dev_f32(x[:1]))
    dq.dqg_expert_group_take(ticket)
    assert bits_equal(host(y)[0], y1[0][0])
    table.close()


def test_group_bad_id_is_reported():
    hs, table = _small_group(6)
    ids = np.array([[0, 1, 2], [1, 99, 4]], np.int32)
    w = np.full((2, 3), 1 / 3, np.float32)
    x = synth.activations(2, 256, 4700)
    ticket, y, scratch = dq.dqg_expert_group_issue(table, dev_i32(ids), dev_f32(w), 5, dev_f32(x))
    with pytest.raises(dq.DqgError) as ei:
        dq.dqg_expert_group_take(ticket)
    assert ei.value.code == -7
    yh = host(y)
    assert np.all(np.isnan(yh[1])) and np.all(np.isfinite(yh[0]))
    yd, ad = oracle.expert_group_down(hs, ids, w, 5, scratch_h(scratch, 2, 3, table.I))
    assert np.all(np.isnan(yd[1]))
    assert_close(yh[:1], yd[:1], ad[:1], "row beside a bad id: down and combine on the device's h")
    yr, a = oracle.expert_group(hs, ids[:1], w[:1], 5, x[:1])
    assert_close(yh[:1], yr, a, "row beside a bad id")
    # the next good call clears the flag
    ids[1, 1] = 3
    ticket, y, scratch = dq.dqg_expert_group_issue(table, dev_i32(ids), dev_f32(w), 5, dev_f32(x),
                                                   scratch=scratch)
    dq.dqg_expert_group_take(ticket)


def test_group_scratch_reused_across_calls():
    """One scratch, consecutive calls of different sizes: each matches the oracle."""
    hs, table = _small_group(13)
    scratch = table.scratch(6, 4)
    for i, S in enumerate([3, 1, 6, 2, 6, 1]):
        ids, w = synth.routing(S, 12, 4, 4900 + i)
        x = synth.activations(S, 256, 4950 + i)
        sc = scratch[: table.scratch_bytes(S, 4)]
        check_group(hs, table, ids, w, 12 if i % 2 else None, x, f"reused scratch call {i} S={S}", scratch=sc,
                    issue=False)


def test_group_zero_weights_and_no_shared():
    hs, table = _small_group(6)
    ids, _ = synth.routing(2, 5, 3, 4800)
    w = np.zeros((2, 3), np.float32)
    x = synth.activations(2, 256, 4801)
    y = host(dq.dqg_expert_group(table, dev_i32(ids), dev_f32(w), None, dev_f32(x)))
    assert np.all(y == 0)


# ---------------------------------------------------------------------------
# the measured workloads at full size
# ---------------------------------------------------------------------------

def test_workload_int8_gemv_256x512():
    c = synth.WORKLOADS["int8_gemv_256x512"]
    m = synth.matrix(c["fmt"], c["O"], c["K"], c["gs"], c["seed"], 0)
    x = synth.activations(1, c["K"], c["seed"], 1)
    y = host(dq.dqg_matmul(up(m), dev_f32(x)))
    yr, a = oracle.gemv(m, x)
    log(f"  worst normalised error {assert_close(y, yr, a, 'int8 256x512'):.2e}")


@pytest.mark.parametrize("S", [1, 4])
def test_workload_int4g32_gemv_6144(S):
    c = synth.WORKLOADS["int4g32_gemv_6144x6144"]
    m = synth.matrix(c["fmt"], c["O"], c["K"], c["gs"], c["seed"], 0)
    x = synth.activations(S, c["K"], c["seed"], S)
    y = host(dq.dqg_matmul(up(m), dev_f32(x)))
    yr, a = oracle.gemv(m, x)
    log(f"  worst normalised error {assert_close(y, yr, a, f'int4 6144 S={S}'):.2e}")


def test_workload_int3g64_gemv_6144x16384():
    c = synth.WORKLOADS["int3g64_gemv_6144x16384"]
    m = synth.matrix(c["fmt"], c["O"], c["K"], c["gs"], c["seed"], 0)
    x = synth.activations(1, c["K"], c["seed"], 1)
    y = host(dq.dqg_matmul(up(m), dev_f32(x)))
    yr, a = oracle.gemv(m, x)
    log(f"  worst normalised error {assert_close(y, yr, a, 'int3 6144x16384'):.2e}")


def test_workload_single_expert_mlp():
    c = synth.WORKLOADS["int4g32_expert_6144x2048"]
    e = synth.expert(c["fmt"], c["H"], c["I"], c["gs"], c["seed"], 0)
    x = synth.activations(1, c["H"], c["seed"], 1)
    d = dq.Expert.upload(e)
    h = dq.dqg_gate_up(d.gate, d.up, dev_f32(x))
    y = host(dq.dqg_matmul(d.down, h))
    hh = host(h)
    r = oracle.gate_up(e.gate, e.up, x)
    assert_close(hh, r["h"], r["nh"], "expert MLP: h")
    yd, ad = oracle.gemv(e.down, hh)   # down on the device's own h, the GEMV's own normaliser
    log(f"  worst strict error {assert_close(y, yd, ad, 'expert MLP: down on the device h'):.2e}")
    yr, a = oracle.expert_group([e], np.zeros((1, 1), np.int32), np.ones((1, 1), np.float32), None, x)
    assert_close(y, yr, a, "expert MLP end to end (propagated normaliser)")
    table = dq.ExpertTable([d])
    check_group([e], table, np.zeros((1, 1), np.int32), np.ones((1, 1), np.float32), None, x,
                "expert MLP via expert_group")


@pytest.fixture(scope="module")
def group256():
    c = synth.WORKLOADS["int4g32_expert_group_256top8_shared"]
    routes = {S: synth.routing(S, c["E"], c["k"], c["seed"], S) for S in c["S"]}
    keep = set(np.concatenate([r[0].ravel() for r in routes.values()]).tolist()) | {c["E"]}
    log(f"  drawing {c['E'] + 1} experts ({len(keep)} kept on the host)")
    dev, hosts = upload_experts(c["fmt"], c["H"], c["I"], c["gs"], c["seed"], c["E"] + 1, keep=keep)
    table = dq.ExpertTable(dev)
    yield c, routes, table, HostExperts(c["E"] + 1, hosts)
    table.close()
    del dev, table
    gc.collect()
    torch.cuda.empty_cache()


@pytest.mark.parametrize("S", [1, 2, 4])
def test_workload_group_256top8_shared(group256, S):
    c, routes, table, hosts = group256
    ids, w = routes[S]
    x = synth.activations(S, c["H"], c["seed"], 100 + S)
    check_group(hosts, table, ids, w, c["E"], x, f"group256 S={S}")


def test_workload_mxfp4_group_384top8_s8():
    c = synth.WORKLOADS["mxfp4_expert_group_384top8_s8"]
    S = 8
    ids, w = synth.routing(S, c["E"], c["k"], c["seed"], S)
    keep = set(ids.ravel().tolist())   # every token's experts (at most 64) stay on the host
    log(f"  drawing {c['E']} MXFP4 experts ({len(keep)} kept on the host)")
    dev, hosts = upload_experts(c["fmt"], c["H"], c["I"], c["gs"], c["seed"], c["E"], keep=keep)
    table = dq.ExpertTable(dev)
    x = synth.activations(S, c["H"], c["seed"], 200)
    check_group(HostExperts(c["E"], hosts), table, ids, w, None, x, "mxfp4 group S=8")
    table.close()
    del dev, table
    gc.collect()
    torch.cuda.empty_cache()


def test_event_timing_all_and_sampled():
    """dqg_prof_begin times every launch; dqg_prof_begin_sampled(capacity, 3)
    the launches of calls 0, 3, 6, ... counted from the begin."""
    m = _small(0, SMALL[0])
    W = up(m)
    x = dev_f32(synth.activations(2, m.K, 2200))
    dq.dqg_prof_begin(16)
    for _ in range(7):
        dq.dqg_matmul(W, x)
    prof = dq.dqg_prof_end()
    assert prof["matmul"][0] == 7 and prof["matmul"][1] > 0
    dq.dqg_prof_begin_sampled(16, 3)
    for _ in range(7):
        dq.dqg_matmul(W, x)
    prof = dq.dqg_prof_end()
    assert prof["matmul"][0] == 3 and prof["matmul"][1] > 0
    dq.dqg_prof_begin_sampled(2, 1)   # capacity caps the timed launches
    for _ in range(5):
        dq.dqg_matmul(W, x)
    assert dq.dqg_prof_end()["matmul"][0] == 2
    dq.dqg_prof_begin(8)              # launch by launch, in launch order
    for _ in range(3):
        dq.dqg_matmul(W, x)
    dq.dqg_dequant(W, torch.empty((m.O, m.K), dtype=torch.float32, device="cuda"))
    each = dq.dqg_prof_end_launches(8)
    assert [k for k, _ in each] == ["matmul"] * 3 + ["dequant"] and all(ms > 0 for _, ms in each)
