"""Seeded input generator: determinism, shapes and stated distributions."""
import numpy as np

import oracle as O
import pfgen


def test_deterministic_and_shapes():
    a = pfgen.make(pfgen.C0)
    b = pfgen.make(pfgen.C0)
    for k in a:
        assert np.array_equal(a[k], b[k])
    assert a["q"].shape == (256, 2, 128) and a["q"].dtype == np.uint16
    assert a["sink_k"].shape == (512, 2, 128)
    assert a["pool_k"].shape == (80, 2, 128)
    assert a["recent_v"].shape == (256, 2, 128)
    assert a["deltas"].min() >= 1 and a["deltas"].max() <= 20 and a["deltas"].shape == (4,)
    c = pfgen.make(pfgen.C0, 1234)
    assert not np.array_equal(a["q"], c["q"])


def test_distributions():
    c = pfgen.make(pfgen.C0.replace(scale=float(1 / np.sqrt(2))))
    x = O.bf16_to_f64(c["sink_k"])
    assert abs(x.mean()) < 0.01 and abs(x.std() - 1 / np.sqrt(2)) < 0.01
    cfg = pfgen.C0.replace(pool_blocks=40, pool_offset_std=0.5)
    p = O.bf16_to_f64(pfgen.make(cfg)["pool_k"]).reshape(40, 8, 2, 128)
    mu = p.mean(axis=1)                        # block-wise means carry the offset
    assert 0.45 < (mu.std() ** 2 - 1.0 / 8) ** 0.5 < 0.55


def test_step_queries_and_rollin():
    q1 = pfgen.step_queries(pfgen.C3, 0, 0)
    q2 = pfgen.step_queries(pfgen.C3, 0, 1)
    assert q1.shape == (6240, 12, 128) and not np.array_equal(q1, q2)
    r = pfgen.rollin_block(pfgen.C3, 5)
    assert r["k"].shape == (182, 12, 128)
