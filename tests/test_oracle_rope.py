"""Oracle RoPE: closed forms, the multiplicative identity and invariants.

The identity e^{i theta p} e^{i theta delta} = e^{i theta (p+delta)} is stated in
the digest (前置知识 RoPE) and in the arXiv HTML ("Incremental RoPE adjustment");
the shift rotates only the 44 temporal dims (1_h, 1_w are identities).
"""
import math

import numpy as np
import pytest

import oracle as O


def _max_identity_error(shift_fn, encode_fn, seed=0, trials=200):
    rng = np.random.default_rng(seed)
    worst = 0.0
    for _ in range(trials):
        k = rng.standard_normal((3, O.HEAD_DIM))
        p = (int(rng.integers(0, 480)), int(rng.integers(0, 60)), int(rng.integers(0, 104)))
        d = int(rng.integers(-480, 481))
        lhs = shift_fn(encode_fn(k, *p), d)
        rhs = encode_fn(k, p[0] + d, p[1], p[2])
        worst = max(worst, float(np.max(np.abs(lhs - rhs))))
    return worst


def test_incremental_shift_equals_reencode():
    err = _max_identity_error(O.rope_shift, O.rope_encode)
    assert err <= 1e-6
    assert err < 1e-10  # the actual fp64 error is ~1e-13


def test_closed_form_rotation():
    # theta_{t,0} = base^0 = 1, so p_t = 1 rotates pair 0 by one radian, and
    # p_t = pi/2 takes (1, 0) to (0, 1): the positive sense of e^{+i theta p}.
    e0 = np.zeros(O.HEAD_DIM)
    e0[0] = 1.0
    r = O.rope_encode(e0, 1.0, 0.0, 0.0)
    assert r[0] == pytest.approx(0.5403023058681398, abs=1e-15)
    assert r[1] == pytest.approx(0.8414709848078965, abs=1e-15)
    r = O.rope_encode(e0, math.pi / 2, 0.0, 0.0)
    assert abs(r[0]) < 1e-15 and r[1] == pytest.approx(1.0, abs=1e-15)
    # height and width axes start at dims 44 and 86
    for start, pos in ((44, (0, 1, 0)), (86, (0, 0, 1))):
        e = np.zeros(O.HEAD_DIM)
        e[start] = 1.0
        r = O.rope_encode(e, *map(float, pos))
        assert r[start] == pytest.approx(0.5403023058681398, abs=1e-15)
        assert r[start + 1] == pytest.approx(0.8414709848078965, abs=1e-15)
        assert np.count_nonzero(r) == 2


def _measured_freqs(axis_start, n_pairs, axis):
    """Angle per unit position of each pair of one axis, read off the encoder:
    a unit vector in pair j encoded at position 1 of that axis comes back as
    (cos a_j, sin a_j), and a_j in (0, 1] is recovered with atan2."""
    out = np.empty(n_pairs)
    for j in range(n_pairs):
        e = np.zeros(O.HEAD_DIM)
        e[axis_start + 2 * j] = 1.0
        pos = [0.0, 0.0, 0.0]
        pos[axis] = 1.0
        r = O.rope_encode(e, *pos)
        out[j] = math.atan2(r[axis_start + 2 * j + 1], r[axis_start + 2 * j])
    return out


def _check_roformer_table(th, n_dims):
    """Properties of theta_j = 10000^(-2j/n_dims) that pin every entry without
    restating the power: theta_0 = 1; theta_j * theta_{n/2 - j} = 10000^-1 for
    the pairs that exist; consecutive ratios are all equal, and the (n/2)-th
    power of that ratio is 10000^-1 (a geometric table ending one step short
    of 1e-4)."""
    half = n_dims // 2
    assert th[0] == pytest.approx(1.0, abs=1e-15)
    for j in range(1, half):
        if half - j < len(th):
            assert th[j] * th[half - j] == pytest.approx(1e-4, rel=1e-12), j
    ratios = th[1:] / th[:-1]
    assert np.max(np.abs(ratios - ratios[0])) < 1e-12
    assert ratios[0] ** half == pytest.approx(1e-4, rel=1e-12)


def test_temporal_frequency_table():
    # [digest] 前置知识 RoPE and [arXiv] "The Position Misalignment Problem":
    # theta_t spans 44 dims = 22 pairs; the RoFormer table gives theta_{t,11} =
    # 10000^(-1/2) = 0.01 exactly, so position 100 turns pair 11 by one radian
    th = _measured_freqs(0, 22, 0)
    _check_roformer_table(th, 44)
    assert th[11] == pytest.approx(0.01, rel=1e-13)
    e = np.zeros(O.HEAD_DIM)
    e[22] = 1.0
    r = O.rope_encode(e, 100.0, 0.0, 0.0)
    assert r[22] == pytest.approx(math.cos(1.0), abs=1e-13)
    assert r[23] == pytest.approx(math.sin(1.0), abs=1e-13)


def test_height_width_frequency_tables():
    # 42 dims = 21 pairs each; theta_7 = 10000^(-1/3), so its cube is 1e-4
    for start, axis in ((44, 1), (86, 2)):
        th = _measured_freqs(start, 21, axis)
        _check_roformer_table(th, 42)
        assert th[7] ** 3 == pytest.approx(1e-4, rel=1e-12)


def test_planted_frequency_exponent_fails_the_table(monkeypatch):
    # an exponent of -j/d instead of -2j/d (and one with the axis width
    # swapped) must each break a table pin, although theta_0 = 1 still holds
    import oracle.pf_oracle as impl
    mutants = [lambda d, base=O.ROPE_BASE: base ** (-np.arange(d // 2, dtype=np.float64) / d),
               lambda d, base=O.ROPE_BASE: base ** (-2.0 * np.arange(d // 2, dtype=np.float64) / 128)]
    for mut in mutants:
        with monkeypatch.context() as m:
            m.setattr(impl, "axis_freqs", mut)
            with pytest.raises(AssertionError):
                _check_roformer_table(_measured_freqs(0, 22, 0), 44)
    # the unpatched table passes the same check
    _check_roformer_table(_measured_freqs(0, 22, 0), 44)


def test_relative_position_property():
    # Textbook RoPE: <enc(q, p1), enc(k, p2)> depends only on p1 - p2 per axis.
    rng = np.random.default_rng(3)
    q, k = rng.standard_normal((2, O.HEAD_DIM))
    a = O.rope_encode(q, 17, 5, 9) @ O.rope_encode(k, 4, 2, 30)
    b = O.rope_encode(q, 117, 25, 19) @ O.rope_encode(k, 104, 22, 40)
    assert a == pytest.approx(b, abs=1e-11)
    c = O.rope_encode(q, 18, 5, 9) @ O.rope_encode(k, 4, 2, 30)
    assert abs(a - c) > 1e-6


def test_shift_touches_only_temporal_dims_and_preserves_norms():
    rng = np.random.default_rng(4)
    k = rng.standard_normal((64, O.HEAD_DIM))
    s = O.rope_shift(k, 37.0)
    assert np.array_equal(s[:, 44:], k[:, 44:])
    n0 = np.hypot(k[:, 0:44:2], k[:, 1:44:2])
    n1 = np.hypot(s[:, 0:44:2], s[:, 1:44:2])
    assert np.max(np.abs(n0 - n1)) < 1e-12
    back = O.rope_shift(s, -37.0)
    assert np.max(np.abs(back - k)) < 1e-12


def test_shift_blocks_bf16_storage():
    rng = np.random.default_rng(5)
    n_c, H = 8, 2
    pool = O.f64_to_bf16(rng.standard_normal((10 * n_c, H, O.HEAD_DIM)))
    same = O.rope_shift_blocks(pool, n_c, [1, 4], [0, 0])
    assert np.array_equal(same, pool)                    # delta = 0 is bitwise identity
    out = O.rope_shift_blocks(pool, n_c, [1, 4], [7, 20])
    assert np.array_equal(out[..., 44:], pool[..., 44:])  # dims 44..127 bitwise unchanged
    untouched = np.ones(10 * n_c, bool)
    untouched[n_c:2 * n_c] = untouched[4 * n_c:5 * n_c] = False
    assert np.array_equal(out[untouched], pool[untouched])
    # each stored value is the bf16 rounding of the exact rotation
    exact = O.rope_shift(O.bf16_to_f64(pool[n_c:2 * n_c]), 7.0)
    assert np.array_equal(out[n_c:2 * n_c], O.f64_to_bf16(exact))


def _mut_sign(k, d):
    return O.rope_shift(k, -d)


def _mut_all_dims(k, d):
    return O.rope_encode(k, d, d, d)


def _mut_freq(k, d):
    k = np.array(k, dtype=np.float64, copy=True)
    j = np.arange(22)
    th = O.ROPE_BASE ** (-2.0 * (j + 1) / 44)       # off-by-one frequency index
    z = (k[..., 0:44:2] + 1j * k[..., 1:44:2]) * np.exp(1j * th * d)
    k[..., 0:44:2], k[..., 1:44:2] = z.real, z.imag
    return k


def _mut_pairing(k, d):
    k = np.array(k, dtype=np.float64, copy=True)
    j = np.arange(22)
    th = O.ROPE_BASE ** (-2.0 * j / 44)
    z = (k[..., 0:22] + 1j * k[..., 22:44]) * np.exp(1j * th * d)   # split-half pairs
    k[..., 0:22], k[..., 22:44] = z.real, z.imag
    return k


@pytest.mark.parametrize("mutant", [_mut_sign, _mut_all_dims, _mut_freq, _mut_pairing])
def test_planted_mistakes_fail_identity(mutant):
    assert _max_identity_error(mutant, O.rope_encode, trials=20) > 1e-3


def test_evict_and_shift_sink_closes_the_gap():
    # sink keys encoded at frames 0..S_b*B_f-1 (one row per frame here); after
    # evicting D blocks they must equal keys encoded at frame + D*B_f, and the
    # sink's last frame + 1 must be the first surviving block's first frame
    Sb, Bf, M, n_c, D = 2, 4, 6, 3, 2
    rng = np.random.default_rng(8)
    raw = rng.standard_normal((Sb * Bf, 1, O.HEAD_DIM))
    enc = np.stack([O.rope_encode(raw[f], f, 3, 5) for f in range(Sb * Bf)])
    sink = O.f64_to_bf16(enc)
    pool = O.f64_to_bf16(rng.standard_normal((M * n_c, 1, O.HEAD_DIM)))
    tags = O.initial_pos_tags(M, Sb, Bf)
    r = O.evict_and_shift_sink(sink, pool, pool, tags, D, n_c, Bf)
    assert r["delta"] == D * Bf
    assert r["pool_k"].shape[0] == (M - D) * n_c and r["tags"].tolist() == tags[D:].tolist()
    assert (Sb * Bf - 1) + r["delta"] + 1 == r["tags"][0]
    want = np.stack([O.rope_encode(raw[f], f + r["delta"], 3, 5) for f in range(Sb * Bf)])
    got = O.bf16_to_f64(r["sink_k"])
    # one bf16 rounding of the stored input plus one of the result
    assert np.max(np.abs(got - want)) <= 2 * 2.0 ** -8 * np.max(np.abs(want)) + 1e-12
    assert np.array_equal(r["sink_k"][..., O.T_DIMS:], sink[..., O.T_DIMS:])
