"""Parity of DeepSeek V4's rounding activation (dqg_expert_table_set_activation)
with the CPU oracle, through the C ABI.

Inputs as the pages' engine hands them over to its experts: x already on
the E4M3 grid (multiples of 2^-6 up to 3.75), MXFP4 experts (DeepSeek V4's
expert format), here with power-of-two scales of 2^-5 and 2^-4.  Then every
product of gate and up is exact in f32 and every partial sum is a multiple
of 2^-12 below 6 * 2^-4 * 3.75 * H < 2^24 * 2^-12, so the device forms g and
u exactly, in any order, and rounds the same values the oracle rounds.
(Larger scales put |g| where f32's silu(g) is g itself, and g * u * w then
often sits on a bf16 tie that the exact value misses by less than f32
resolves.)  The silu and the route weight leave the device within 2^-19 of
the exact activation; a draw in which the oracle finds a bf16 decision that
close to a rounding boundary is redrawn (the seed moves on), so down's
input (h in the scratch) must match the oracle bit for bit.  Each of down's
outputs is a chain of at most 32 fused multiply-adds per chunk of 32
inputs, one scaled add per chunk a lane holds (I / 2048 of them, rounded
up) and six adds across the wave, so its f32 sum strays from the exact one
by at most (40 + I / 2048) 2^-24 sum |w_k h_k| (first order; 48 is used):
y must lie in the oracle's [y_lo, y_hi] (the rows' lower and upper bf16
candidates added in the same order), which pins it bit for bit wherever
the two coincide.
"""
import math

import numpy as np
import pytest
import torch

import oracle
import synth
from gpu_helpers import dev_f32, dev_i32, host, log

pytestmark = pytest.mark.gpu

if torch.cuda.is_available():
    import dequant_gemv_expert_amd as dq
else:   # collected on CPU-only hosts, never run there
    dq = None

H_OFFSET = 1024      # DQG_SCRATCH_H_OFFSET
ACT_REL = 2.0 ** -19


@pytest.fixture(autouse=True)
def _announce(request):
    log(f"[gpu] start {request.node.nodeid}")
    yield
    torch.cuda.synchronize()
    log(f"[gpu] done  {request.node.nodeid}")


def _exact_inputs(hs, x, H):
    """The conditions under which g and u are exact in f32 (see the module text)."""
    assert np.all(x * 64 == np.round(x * 64))
    for h in hs:
        for m in (h.gate, h.up):
            assert set(np.unique(m.scales).tolist()) <= {2.0 ** -5, 2.0 ** -4}
    assert 6 * 2.0 ** -4 * float(np.max(np.abs(x))) * H * 2 ** 12 < 2 ** 24


def _draw(E, H, I, S, k, seed, limit, shared, dup):
    """Experts from ``seed``; x and the routing redrawn until no bf16 decision
    before down lies within ACT_REL of a boundary."""
    hs = [synth.expert(synth.FMT_MXFP4, H, I, 32, seed, i, scale_kind="pow2_small") for i in range(E)]
    for s in range(seed, seed + 40):
        x = synth.activations_e4m3_grid(S, H, s, 1)
        ids, w = synth.routing(S, E - 1, k, s, 2)
        if dup:
            ids[0, k - 1] = ids[0, 0]   # one expert twice in a token: rank order among equal ids
        r = oracle.expert_group_v4(hs, ids, w, shared, x, limit, 0.0, ACT_REL, (48 + -(-I // 2048)) * 2.0 ** -24)
        if r["open"] == 0:
            return hs, x, ids, w, r
        log(f"  seed {s}: {r['open']} bf16 decisions within 2^-19 of a boundary, redrawn")
    raise AssertionError("no draw without open decisions")


CASES = [
    # E, H, I, S, k, limit, shared, dup
    (16, 1024, 256, 1, 6, math.inf, True, False),
    (16, 1024, 256, 1, 6, 10.0, True, False),
    (8, 512, 128, 4, 3, math.inf, True, True),
    (12, 2048, 512, 1, 8, 7.0, False, False),
    (6, 256, 128, 7, 3, 1.0, True, True),
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: f"E{c[0]}_H{c[1]}_I{c[2]}_S{c[3]}_k{c[4]}_L{c[5]}"
                         + ("_sh" if c[6] else "") + ("_dup" if c[7] else ""))
def test_v4_group_matches_oracle(case):
    E, H, I, S, k, limit, with_shared, dup = case
    shared = E - 1 if with_shared else None
    hs, x, ids, w, r = _draw(E, H, I, S, k, 9800 + 50 * CASES.index(case), limit, shared, dup)
    _exact_inputs(hs, x, H)
    table = dq.ExpertTable([dq.Expert.upload(h) for h in hs])
    table.set_activation(dq.DQG_ACT_SWIGLU_V4)
    if not math.isinf(limit):
        table.set_swiglu_limit(limit)
    scratch = table.scratch(S, k)
    y = host(dq.dqg_expert_group(table, dev_i32(ids), dev_f32(w), shared, dev_f32(x), scratch=scratch))
    hdev = host(scratch[H_OFFSET: H_OFFSET + (S * k + S) * I * 4].view(torch.float32)).reshape(S * k + S, I)
    slots = list(range(S * k)) + ([S * k + t for t in range(S)] if with_shared else [])
    for q in slots:
        bad = np.flatnonzero(hdev[q].astype(np.float64) != r["h"][q])
        assert bad.size == 0, f"h slot {q}: {bad.size} of {I} differ, first {bad[:4]}: " \
                              f"{hdev[q][bad[:4]]} vs {r['h'][q][bad[:4]]}"
    lo, hi = r["y_lo"], r["y_hi"]
    out = (y < lo) | (y > hi) | np.isnan(y)
    assert not out.any(), f"{int(out.sum())} of {y.size} outside [y_lo, y_hi], first {np.argwhere(out)[:4].tolist()}"
    pinned = lo == hi
    log(f"  h: {len(slots) * I} values bit for bit; y: {int(pinned.sum())} of {y.size} pinned to one value, "
        f"{int(np.sum(y == r['y']))} equal to the oracle's nearest")
    table.close()


def test_v4_toggles_back_to_plain():
    """Switching a table to DeepSeek V4's activation and back gives the plain SwiGLU's bits again."""
    E, H, I, S, k = 6, 512, 256, 2, 3
    hs = [synth.expert(synth.FMT_MXFP4, H, I, 32, 9900, i) for i in range(E)]
    x = synth.activations(S, H, 9901)
    ids, w = synth.routing(S, E, k, 9902)
    table = dq.ExpertTable([dq.Expert.upload(h) for h in hs])
    args = (table, dev_i32(ids), dev_f32(w), 0, dev_f32(x))
    y0 = host(dq.dqg_expert_group(*args))
    table.set_activation(dq.DQG_ACT_SWIGLU_V4)
    y1 = host(dq.dqg_expert_group(*args))
    table.set_activation(dq.DQG_ACT_SWIGLU)
    y2 = host(dq.dqg_expert_group(*args))
    assert np.array_equal(y0, y2)
    assert not np.array_equal(y0, y1)
    yr, a = oracle.expert_group(hs, ids, w, 0, x)
    assert np.max(np.abs(y1 - yr) / a) < 0.1   # the roundings move y, within E4M3's reach
    table.close()


def test_v4_needs_blocks_of_128():
    hs = [synth.expert(synth.FMT_MXFP4, 256, 192, 32, 9910, i) for i in range(2)]
    table = dq.ExpertTable([dq.Expert.upload(h) for h in hs])
    with pytest.raises(dq.DqgError):
        table.set_activation(dq.DQG_ACT_SWIGLU_V4)
    with pytest.raises(dq.DqgError):
        table.set_activation(7)
    table.close()


def test_v4_bad_id_is_nan_and_reported():
    """An id outside the table makes its token's row NaN; the other tokens keep their values."""
    E, H, I, S, k = 6, 256, 128, 3, 2
    hs, x, ids, w, r = _draw(E, H, I, S, k, 9920, math.inf, E - 1, False)
    bad = ids.copy()
    bad[1, 1] = E + 3
    table = dq.ExpertTable([dq.Expert.upload(h) for h in hs])
    table.set_activation(dq.DQG_ACT_SWIGLU_V4)
    ticket, y, _ = dq.dqg_expert_group_issue(table, dev_i32(bad), dev_f32(w), E - 1, dev_f32(x))
    with pytest.raises(dq.DqgError):
        dq.dqg_expert_group_take(ticket)
    y = host(y)
    assert np.all(np.isnan(y[1]))
    for t in (0, 2):
        assert np.all((y[t] >= r["y_lo"][t]) & (y[t] <= r["y_hi"][t]))
    table.close()


def test_v4_group_full_size():
    """The one-token group shape the benchmark times (H 6144, I 2048, top-8 + shared), on MXFP4
    experts with x on the E4M3 grid up to 0.9375 (so g and u stay exact at this H).  With 18432
    activations no draw avoids open bf16 decisions, so h is checked against the oracle's bounds:
    bit for bit where they coincide, inside them where a decision is open."""
    E, H, I, k = 10, 6144, 2048, 8
    hs = [synth.expert(synth.FMT_MXFP4, H, I, 32, 9950, i, scale_kind="pow2_small") for i in range(E)]
    x = synth.activations_e4m3_grid(1, H, 9951, max_exp=-1)
    ids, w = synth.routing(1, E - 1, k, 9952)
    _exact_inputs(hs, x, H)
    r = oracle.expert_group_v4(hs, ids, w, E - 1, x, math.inf, 0.0, ACT_REL, (48 + -(-I // 2048)) * 2.0 ** -24)
    table = dq.ExpertTable([dq.Expert.upload(h) for h in hs])
    table.set_activation(dq.DQG_ACT_SWIGLU_V4)
    scratch = table.scratch(1, k)
    y = host(dq.dqg_expert_group(table, dev_i32(ids), dev_f32(w), E - 1, dev_f32(x), scratch=scratch))
    hdev = host(scratch[H_OFFSET: H_OFFSET + (k + 1) * I * 4].view(torch.float32)).reshape(k + 1, I).astype(np.float64)
    lo, hi = r["h_lo"], r["h_hi"]
    fixed = lo == hi
    assert np.array_equal(hdev[fixed], r["h"][fixed]), f"{int(np.sum(hdev[fixed] != r['h'][fixed]))} fixed values differ"
    assert np.all((hdev >= lo) & (hdev <= hi))
    out = (y < r["y_lo"]) | (y > r["y_hi"]) | np.isnan(y)
    assert not out.any(), f"{int(out.sum())} of {y.size} outside [y_lo, y_hi]"
    log(f"  {r['open']} open decisions; h: {int(fixed.sum())} of {fixed.size} fixed, "
        f"{int(np.sum(hdev == r['h']))} equal to the nearest; y: {int(np.sum(r['y_lo'] == r['y_hi']))} of {y.size} "
        f"pinned")
    table.close()


@pytest.mark.parametrize("limit", [math.inf, 7.0])
def test_v4_single_expert(limit):
    """One token routed to one expert with no shared expert (the group's unit launches), H 2048,
    I 2048, route weight 0.75: h within the oracle's bf16 bounds and bit for bit where they
    coincide, y within [y_lo, y_hi]."""
    E, H, I = 4, 2048, 2048
    hs = [synth.expert(synth.FMT_MXFP4, H, I, 32, 9970, i, scale_kind="pow2_small") for i in range(E)]
    x = synth.activations_e4m3_grid(1, H, 9971, 1)
    ids, w = np.array([[2]], np.int32), np.array([[0.75]], np.float32)
    _exact_inputs(hs, x, H)
    r = oracle.expert_group_v4(hs, ids, w, None, x, limit, 0.0, ACT_REL, (48 + -(-I // 2048)) * 2.0 ** -24)
    table = dq.ExpertTable([dq.Expert.upload(h) for h in hs])
    table.set_activation(dq.DQG_ACT_SWIGLU_V4)
    if not math.isinf(limit):
        table.set_swiglu_limit(limit)
    scratch = table.scratch(1, 1)
    y = host(dq.dqg_expert_group(table, dev_i32(ids), dev_f32(w), None, dev_f32(x), scratch=scratch))
    hdev = host(scratch[H_OFFSET: H_OFFSET + I * 4].view(torch.float32)).reshape(1, I).astype(np.float64)
    lo, hi = r["h_lo"][:1], r["h_hi"][:1]
    fixed = lo == hi
    assert np.array_equal(hdev[fixed], r["h"][:1][fixed])
    assert np.all((hdev >= lo) & (hdev <= hi))
    out = (y < r["y_lo"]) | (y > r["y_hi"]) | np.isnan(y)
    assert not out.any(), f"{int(out.sum())} of {y.size} outside [y_lo, y_hi]"
    log(f"  {r['open']} open decisions; h: {int(fixed.sum())} of {fixed.size} fixed; "
        f"y: {int(np.sum(r['y_lo'] == r['y_hi']))} of {y.size} pinned")
    table.close()


@pytest.mark.parametrize("S", [1, 2])
@pytest.mark.parametrize("act", ["swiglu", "v4"])
def test_group_graph_capture_replays(act, S):
    """A captured dqg_expert_group (two launches; three with DeepSeek V4's activation, none of them
    a memset) replays with the eager call's bits, with new routings and activations copied in and
    eager calls between the replays, at one token (the one-token gate/up kernel) and two."""
    E, H, I, k = 10, 512, 256, 4
    hs = [synth.expert(synth.FMT_MXFP4, H, I, 32, 9960, i) for i in range(E)]
    table = dq.ExpertTable([dq.Expert.upload(h) for h in hs])
    if act == "v4":
        table.set_activation(dq.DQG_ACT_SWIGLU_V4)
    draws = [synth.routing(S, E - 1, k, 9961, r) for r in range(3)]
    xs = [synth.activations(S, H, 9962, r) for r in range(3)]
    ids, w, x = dev_i32(draws[0][0]), dev_f32(draws[0][1]), dev_f32(xs[0])
    y = torch.empty((S, H), dtype=torch.float32, device="cuda")
    scratch = table.scratch(S, k)
    dq.dqg_expert_group(table, ids, w, E - 1, x, y=y, scratch=scratch)   # warm the library
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        dq.dqg_expert_group(table, ids, w, E - 1, x, y=y, scratch=scratch)
    for r in range(3):
        ids.copy_(dev_i32(draws[r][0]))
        w.copy_(dev_f32(draws[r][1]))
        x.copy_(dev_f32(xs[r]))
        want = host(dq.dqg_expert_group(table, ids, w, E - 1, x))   # eager, its own scratch
        y.zero_()
        g.replay()
        dq.dqg_expert_group(table, ids, w, 0, x)                    # eager work between replays
        torch.cuda.synchronize()
        assert host(y).tobytes() == want.tobytes(), r
    table.close()
