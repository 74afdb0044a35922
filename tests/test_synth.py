"""The seeded generators: deterministic, the documented shapes and ranges."""
import numpy as np

import synth


def test_deterministic_and_independent():
    a = synth.matrix(4, 16, 64, 32, 1, 2, 3)
    b = synth.matrix(4, 16, 64, 32, 1, 2, 3)
    c = synth.matrix(4, 16, 64, 32, 1, 2, 4)
    assert np.array_equal(a.q, b.q) and np.array_equal(a.scales, b.scales)
    assert not np.array_equal(a.q, c.q)


def test_shapes_and_ranges():
    m = synth.matrix(1, 64, 512, None, 9)
    assert m.q.dtype == np.int8 and m.q.shape == (64, 512) and m.scales.shape == (64, 1)
    assert m.q.min() >= -127 and m.scales.min() >= 1e-3 and m.scales.max() <= 1e-2
    m = synth.matrix(4, 32, 256, 32, 9)
    assert m.q.dtype == np.uint8 and m.q.shape == (32, 128) and m.scales.shape == (32, 8)
    assert m.scales.min() >= 1e-3 and m.scales.max() <= 2e-2
    m = synth.matrix(5, 8, 256, None, 9)
    assert m.q.shape == (8, 16) and m.q2.shape == (8, 8) and m.scales.shape == (8, 4)
    m = synth.matrix(7, 8, 256, None, 9)
    e = np.log2(m.scales)
    assert np.array_equal(e, np.round(e)) and e.min() >= -10 and e.max() <= -6


def test_routing():
    ids, w = synth.routing(4, 256, 8, 5)
    assert ids.shape == (4, 8) and w.shape == (4, 8)
    for t in range(4):
        assert len(set(ids[t].tolist())) == 8
    assert np.allclose(w.sum(axis=1), 1.0, atol=1e-6) and (w > 0).all()


def test_expert_shapes():
    e = synth.expert(4, 64, 32, 32, 7, 0)
    assert (e.gate.O, e.gate.K, e.up.O, e.up.K, e.down.O, e.down.K) == (32, 64, 32, 64, 64, 32)
