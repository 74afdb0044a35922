"""Helpers of the GPU parity tests: upload seeded inputs, compare with the oracle."""
from __future__ import annotations

import math
import sys
from concurrent.futures import ThreadPoolExecutor

import numpy as np
import torch

import synth
from dequant_gemv_expert_amd import (Expert, ExpertTable, Matrix, dqg_expert_group, dqg_expert_group_issue,
                                     dqg_expert_group_take)

TOL = 1e-5   # max |y_gpu - y_ref| / sum|w*x| per row


def log(msg: str) -> None:
    print(msg, file=sys.stderr, flush=True)


def dev_f32(a) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).cuda()


def dev_i32(a) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).cuda()


def host(t: torch.Tensor) -> np.ndarray:
    return t.detach().cpu().numpy()


ATOL = float(np.finfo(np.float32).tiny)   # 2^-126, the smallest normal f32


def assert_close(y_gpu, y_ref, absn, what: str, tol: float = TOL) -> float:
    """Every |y_gpu - y_ref| <= tol * absn + ATOL.

    ATOL is the smallest normal f32: below it an f32 result has no relative
    precision left (an exact value under 2^-149 can only be 0), so no
    normalised bar holds there.  Returns the largest normalised error seen.
    """
    y = np.asarray(y_gpu, dtype=np.float64)
    assert y.shape == y_ref.shape, (what, y.shape, y_ref.shape)
    assert np.all(np.isfinite(y)), f"{what}: non-finite output"
    err = np.abs(y - y_ref)
    rel = err / (absn + ATOL / tol)   # rel > tol  <=>  err > tol * absn + ATOL
    bad = rel > tol
    worst = float(rel.max()) if rel.size else 0.0
    if bad.any():
        idx = np.unravel_index(np.argmax(rel), rel.shape)
        raise AssertionError(f"{what}: {int(bad.sum())} of {bad.size} outputs beyond tol {tol}; worst "
                             f"{worst:.3e} at {idx}: gpu {y[idx]!r} ref {y_ref[idx]!r} absn {absn[idx]!r}")
    return worst


def upload_experts(fmt, H, I, gs, seed, n, keep=(), threads=16, **kw):
    """Draw n experts, upload each, keep host copies only of the ids in ``keep``.

    Returns (device experts, {id: host expert}).  Host memory stays bounded
    by the batch being uploaded plus the kept experts.
    """
    keep = set(int(i) for i in keep)
    dev, hosts = [None] * n, {}
    batch = max(1, threads)
    with ThreadPoolExecutor(threads) as ex:
        for b0 in range(0, n, batch):
            ids = list(range(b0, min(n, b0 + batch)))
            hs = list(ex.map(lambda i: synth.expert(fmt, H, I, gs, seed, i, **kw), ids))
            for i, h in zip(ids, hs):
                dev[i] = Expert.upload(h)
                if i in keep:
                    hosts[i] = h
    return dev, hosts


class HostExperts:
    """Sequence view for oracle.expert_group: only kept experts are readable."""

    def __init__(self, n, hosts):
        self.n, self.hosts = n, hosts

    def __len__(self):
        return self.n

    def __getitem__(self, i):
        return self.hosts[int(i)]


H_OFFSET = 1024   # DQG_SCRATCH_H_OFFSET: h's byte offset in an expert-group scratch


def scratch_h(scratch: torch.Tensor, S: int, k: int, I: int) -> np.ndarray:
    """The hidden states h [S*k + S][I] an expert-group call left in its scratch."""
    n = (S * k + S) * I
    return host(scratch[H_OFFSET:H_OFFSET + 4 * n].view(torch.float32)).reshape(S * k + S, I)


def check_group(hs, table, ids, w, shared, x, what, limit=math.inf, scratch=None, issue=True,
                slot_h=True):
    """One expert-group call (through issue/take, or the plain call) against the
    oracle, in three ways:

    1. strict, the bar the metric defines: the device's y against the oracle's
       down and rank-order combine applied to the device's own h (read back
       from the scratch), within 1e-5 of the per-row normaliser
       sum_r |w| sum_i |D[o][i] h[i]| plus the shared row's;
    2. every slot's h against the oracle's gate_up, within 1e-5 of nh, the
       first-order reach of errors of 1e-5 A_g in g and 1e-5 A_u in u;
    3. end to end against the oracle's group (the propagated normaliser).

    Returns (y, the worst strict normalised error)."""
    import oracle
    S, k = ids.shape
    if scratch is None:
        scratch = table.scratch(S, k)
    if issue:
        ticket, y, _ = dqg_expert_group_issue(table, dev_i32(ids), dev_f32(w), shared, dev_f32(x),
                                              scratch=scratch)
        dqg_expert_group_take(ticket)   # raises on an out-of-range id
    else:
        y = dqg_expert_group(table, dev_i32(ids), dev_f32(w), shared, dev_f32(x), scratch=scratch)
    y = host(y)
    hdev = scratch_h(scratch, S, k, table.I)
    yd, ad = oracle.expert_group_down(hs, ids, w, shared, hdev)
    worst = assert_close(y, yd, ad, f"{what}: down and combine on the device's h")
    if slot_h:
        for t in range(S):
            for r in range(k):
                e = int(ids[t, r])
                if 0 <= e < len(hs):
                    o = oracle.gate_up(hs[e].gate, hs[e].up, x[t:t + 1], limit)
                    assert_close(hdev[t * k + r][None], o["h"], o["nh"], f"{what} h[{t},{r}]")
            if shared is not None and shared >= 0:
                o = oracle.gate_up(hs[shared].gate, hs[shared].up, x[t:t + 1], limit)
                assert_close(hdev[S * k + t][None], o["h"], o["nh"], f"{what} h[shared {t}]")
    yr, a = oracle.expert_group(hs, ids, w, shared, x, limit)
    assert_close(y, yr, a, f"{what}: end to end (propagated normaliser)")
    log(f"  {what}: worst strict error {worst:.2e}")
    return y, worst
