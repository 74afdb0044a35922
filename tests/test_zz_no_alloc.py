"""dqg_expert_group_noalloc, the expert group on the library's static
per-device scratch (no allocation on the call), against dqg_expert_group
with a caller scratch: two calls in a row, the second with fewer tokens,
bit for bit and within 1e-5 of the oracle's down and combine on h."""
import numpy as np
import pytest
import torch

import oracle
import synth
from gpu_helpers import assert_close, dev_f32, dev_i32, host, log, scratch_h

pytestmark = pytest.mark.gpu

if torch.cuda.is_available():
    import dequant_gemv_expert_amd as dq
    from dequant_gemv_expert_amd import _lib as L
else:   # collected on CPU-only hosts, never run there
    dq = L = None


@pytest.fixture(autouse=True)
def _announce(request):
    log(f"[gpu] start {request.node.nodeid}")
    yield
    torch.cuda.synchronize()
    log(f"[gpu] done  {request.node.nodeid}")


def test_noalloc_matches_caller_scratch_twice():
    E, k, H, I = 12, 4, 256, 128
    hs = [synth.expert(4, H, I, 32, 9700, i) for i in range(E + 1)]
    table = dq.ExpertTable([dq.Expert.upload(h) for h in hs])
    for i, S in enumerate([6, 2]):   # the second call smaller than the first
        ids, w = synth.routing(S, E, k, 9710 + i)
        x = synth.activations(S, H, 9720 + i)
        scratch = table.scratch(S, k)
        y_ref = host(dq.dqg_expert_group(table, dev_i32(ids), dev_f32(w), E, dev_f32(x), scratch=scratch))
        y = torch.full((S, H), float("nan"), dtype=torch.float32, device="cuda")
        dq.dqg_expert_group_noalloc(table, dev_i32(ids), dev_f32(w), E, dev_f32(x), y)
        y = host(y)
        assert y.tobytes() == y_ref.tobytes(), f"call {i} (S={S}): bits differ from the caller-scratch call"
        yd, ad = oracle.expert_group_down(hs, ids, w, E, scratch_h(scratch, S, k, I))
        worst = assert_close(y, yd, ad, f"noalloc call {i} S={S}")
        yr, a = oracle.expert_group(hs, ids, w, E, x)
        assert_close(y, yr, a, f"noalloc call {i} S={S} end to end")
        log(f"  call {i} S={S}: bit-exact with the caller-scratch call, worst strict error {worst:.2e}")
    table.close()


def test_noalloc_refuses_more_than_its_scratch():
    """(S*k + S) * I * 4 bytes beyond the static scratch: DQG_ENOMEM, nothing launched."""
    H, I = 256, 8192
    hs = [synth.expert(4, H, I, 32, 9730, i) for i in range(2)]
    table = dq.ExpertTable([dq.Expert.upload(h) for h in hs])
    S, k = 64, 8
    need = table.scratch_bytes(S, k)
    assert need > (16 << 20)
    ids = dev_i32(np.zeros((S, k), np.int32))
    w = dev_f32(np.zeros((S, k), np.float32))
    x = dev_f32(np.zeros((S, H), np.float32))
    y = torch.zeros((S, H), dtype=torch.float32, device="cuda")
    dq.dqg_stats_reset()
    with pytest.raises(dq.DqgError) as ei:
        dq.dqg_expert_group_noalloc(table, ids, w, None, x, y)
    assert ei.value.code == -6 and "library holds" in str(ei.value)
    assert dq.dqg_stats()["launches"] == 0
    table.close()
