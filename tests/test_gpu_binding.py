"""Shape checks of the binding's calls on device tensors: each mismatch raises
ValueError before the C ABI is called, so nothing is launched."""
import pytest
import torch

import synth
from gpu_helpers import log

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


def _f32(*shape):
    return torch.zeros(shape, dtype=torch.float32, device="cuda")


def test_calls_reject_mismatched_shapes():
    m = synth.matrix(4, 64, 256, 32, 9900, 0)
    W = dq.Matrix.upload(m)
    U = dq.Matrix.upload(synth.matrix(4, 64, 256, 32, 9900, 1))
    U2 = dq.Matrix.upload(synth.matrix(4, 32, 256, 32, 9900, 2))
    dq.dqg_stats_reset()
    with pytest.raises(ValueError):
        dq.dqg_matmul(W, _f32(2, 128))           # K mismatch
    with pytest.raises(ValueError):
        dq.dqg_matmul(W, _f32(256))              # not [S][K]
    with pytest.raises(ValueError):
        dq.dqg_matmul(W, _f32(2, 256), y=_f32(2, 63))
    with pytest.raises(ValueError):
        dq.dqg_gate_up(W, U2, _f32(1, 256))      # gate and up differ
    with pytest.raises(ValueError):
        dq.dqg_gate_up(W, U, _f32(3, 256), h=_f32(2, 64))
    with pytest.raises(ValueError):
        dq.dqg_dequant(W, out=_f32(64, 255))
    hs = [synth.expert(4, 256, 64, 32, 9901, i) for i in range(3)]
    table = dq.ExpertTable([dq.Expert.upload(h) for h in hs])
    ids = torch.zeros((2, 2), dtype=torch.int32, device="cuda")
    with pytest.raises(ValueError):
        dq.dqg_expert_group(table, ids, _f32(2, 3), None, _f32(2, 256))    # w not [S][k]
    with pytest.raises(ValueError):
        dq.dqg_expert_group(table, ids, _f32(2, 2), None, _f32(3, 256))    # x rows != S
    with pytest.raises(ValueError):
        dq.dqg_expert_group(table, ids, _f32(2, 2), None, _f32(2, 128))    # x width != H
    with pytest.raises(ValueError):
        dq.dqg_expert_group(table, ids, _f32(2, 2), None, _f32(2, 256), y=_f32(1, 256))
    with pytest.raises(ValueError):
        dq.dqg_expert_group(table, ids.view(-1), _f32(2, 2), None, _f32(2, 256))
    with pytest.raises(ValueError):
        dq.dqg_route(_f32(2, 16), 4, bias=_f32(15))
    with pytest.raises(ValueError):
        dq.dqg_route(_f32(2, 16), 4, w=_f32(7))
    st = dq.dqg_stats()
    assert st["launches"] == 0, "a rejected call launched a kernel"
    table.close()
