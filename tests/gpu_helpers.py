"""Helpers of the GPU parity tests: upload seeded inputs, compare with the oracle."""
from __future__ import annotations

import sys
from concurrent.futures import ThreadPoolExecutor

import numpy as np
import torch

import synth
from dequant_gemv_expert_amd import Expert, ExpertTable, Matrix

TOL = 1e-5   # max |y_gpu - y_ref| / sum|w*x| per row


def log(msg: str) -> None:
    print(msg, file=sys.stderr, flush=True)


def dev_f32(a) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).cuda()


def dev_i32(a) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).cuda()


def host(t: torch.Tensor) -> np.ndarray:
    return t.detach().cpu().numpy()


def assert_close(y_gpu, y_ref, absn, what: str, tol: float = TOL) -> float:
    """Every |y_gpu - y_ref| <= tol * absn (rows with absn == 0 must be exact).

    Returns the largest normalised error seen.
    """
    y = np.asarray(y_gpu, dtype=np.float64)
    assert y.shape == y_ref.shape, (what, y.shape, y_ref.shape)
    assert np.all(np.isfinite(y)), f"{what}: non-finite output"
    err = np.abs(y - y_ref)
    bad = err > tol * absn
    with np.errstate(divide="ignore", invalid="ignore"):
        rel = np.where(absn > 0, err / absn, np.where(err > 0, np.inf, 0.0))
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
