"""The Python binding checks shapes and byte counts before any pointer reaches
the C ABI (the kernels read through raw pointers, so a short buffer would be
read or written past its end).  CPU only: every case raises before a launch."""
import pytest
import torch

from dequant_gemv_expert_amd import _lib as L


@pytest.mark.parametrize("fmt,O,K,gs,want", [
    (1, 256, 512, 512, (256 * 512, 0, 256)),
    (2, 4, 64, 64, (128, 0, 4)),
    (4, 6144, 6144, 32, (6144 * 3072, 0, 6144 * 192)),
    (5, 6144, 16384, 64, (6144 * 4096, 6144 * 2048, 6144 * 256)),
    (7, 2048, 7168, 32, (2048 * 3584, 0, 2048 * 224)),
    (10, 3, 8, 0, (96, 0, 0)),
    (11, 3, 8, 0, (48, 0, 0)),
    (14, 3, 8, 8, (48, 0, 0)),
    (12, 130, 256, 128, (130 * 256, 0, 2 * 2)),
    (13, 2, 256, 64, (512, 0, 8)),
])
def test_storage_sizes(fmt, O, K, gs, want):
    assert L.storage_sizes(fmt, O, K, gs) == want


@pytest.mark.parametrize("fmt,O,K,gs", [(3, 4, 64, 32), (4, 0, 64, 32), (4, 4, 96, 64), (5, 4, 96, 64),
                                        (12, 4, 64, 128)])
def test_storage_sizes_rejects(fmt, O, K, gs):
    with pytest.raises(ValueError):
        L.storage_sizes(fmt, O, K, gs)


def _cpu(n, dtype=torch.uint8):
    return torch.zeros(n, dtype=dtype)


@pytest.mark.parametrize("kw,match", [
    (dict(fmt=4, O=8, K=64, gs=32, q=_cpu(255), scales=_cpu(16, torch.float32)), "q holds"),
    (dict(fmt=4, O=8, K=64, gs=32, q=_cpu(256), scales=_cpu(15, torch.float32)), "scales hold"),
    (dict(fmt=4, O=8, K=64, gs=32, q=_cpu(256), scales=None), "scales hold"),
    (dict(fmt=5, O=2, K=64, gs=64, q=_cpu(32), scales=_cpu(2, torch.float32), q2=_cpu(15)), "q2 holds"),
    (dict(fmt=5, O=2, K=64, gs=64, q=_cpu(32), scales=_cpu(2, torch.float32), q2=None), "q2 holds"),
    (dict(fmt=10, O=2, K=8, gs=0, q=_cpu(64), scales=_cpu(2, torch.float32)), "no scales"),
    (dict(fmt=4, O=8, K=100, gs=32, q=_cpu(400), scales=_cpu(32, torch.float32)), "multiple of gs"),
])
def test_matrix_rejects_short_or_wrong_buffers(kw, match):
    with pytest.raises(ValueError, match=match):
        L.Matrix(**kw)
