"""The seeded input recipe: deterministic, the stated shapes and distributions,
and never the sentinel pattern 0xFFFF."""
import numpy as np
import pytest

import synth


def _f32(bits):
    return (bits.astype(np.uint32) << 16).view(np.float32)


@pytest.mark.parametrize("cid", [1, 2, 3, 5])
def test_shapes_determinism_no_sentinel(cid):
    w = synth.WORKLOADS[cid]
    a = synth.input_set(cid, 0)
    b = synth.input_set(cid, 0)
    assert a.shape == (w.n_ranks, w.n) and a.dtype == np.uint16
    assert (a == b).all()
    assert not (a == synth.input_set(cid, 1)).all()
    assert not (a == 0xFFFF).any()
    assert np.isfinite(_f32(a)).all()


def test_distributions():
    x = _f32(synth.input_set(2, 0))
    assert abs(x.std() - 0.5) < 0.02 and abs(x.mean()) < 0.02
    u = _f32(synth.rank_input(4, 0, 0))
    assert u.min() >= -1.0 and u.max() < 1.0 and abs(u.mean()) < 0.01
    o = _f32(synth.rank_input(3, 0, 0))
    w = synth.WORKLOADS[3]
    assert (np.abs(o) > 6.0).sum() >= 0.9 * round(w.outlier_frac * w.n)


def test_delays():
    d = synth.delays_ns(5)
    assert d.shape == (10000, 16) and d.dtype == np.uint32
    assert d.min() == 0 and d.max() == 5000
    assert (d == synth.delays_ns(5)).all()
