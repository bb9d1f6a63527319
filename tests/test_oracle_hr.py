"""Pins of the oracle's HR-branch compressor (PackForcing arXiv HTML, "HR Branch:
Progressive 3D Convolution" and "Feature Fusion"; digest 前置知识 3D卷积).

Each pin checks the oracle against something other than its own formula: a
library 3D convolution, a brute-force loop, closed forms of SiLU, the token
count the pages print, and weights that turn the stage into a plain slice.
"""
import json
import os

import numpy as np
import pytest
import torch

import oracle as O
import pfgen

GOLDEN = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "pages_numbers.json")))


def _bits(rng, shape, scale=1.0):
    return pfgen.bf16_bits(rng.standard_normal(shape).astype(np.float32) * np.float32(scale))


@pytest.mark.parametrize("kernel", [(2, 1, 1), (1, 2, 2), (2, 2, 2), (1, 1, 1)])
def test_stage_matches_torch_conv3d(kernel):
    # torch's own strided conv3d on the CPU in float64, in its NCDHW layout
    rng = np.random.default_rng(11)
    x = _bits(rng, (2, 4, 6, 10, 16))
    w = _bits(rng, (24,) + kernel + (16,), 0.2)
    b = rng.standard_normal(24).astype(np.float32)
    got = O.hr_conv_stage(x, w, b, kernel, act=False, round_output=False)
    xt = torch.from_numpy(O.bf16_to_f64(x)).permute(0, 4, 1, 2, 3)
    wt = torch.from_numpy(O.bf16_to_f64(w)).permute(0, 4, 1, 2, 3)
    ref = torch.nn.functional.conv3d(xt, wt, torch.from_numpy(b.astype(np.float64)), stride=kernel)
    ref = ref.permute(0, 2, 3, 4, 1).numpy()
    assert got.shape == ref.shape
    np.testing.assert_allclose(got, ref, rtol=1e-12, atol=1e-12)
    # with SiLU: torch's silu of the same pre-activations
    got_a = O.hr_conv_stage(x, w, b, kernel, act=True, round_output=False)
    np.testing.assert_allclose(got_a, torch.nn.functional.silu(torch.from_numpy(ref)).numpy(), rtol=1e-12, atol=1e-14)


def test_stage_matches_brute_force_loops():
    # the definition of a strided convolution, summed term by term
    rng = np.random.default_rng(12)
    kt, kh, kw = 1, 2, 2
    x = _bits(rng, (1, 2, 5, 7, 16))          # odd H and W: the last row and column are dropped
    w = _bits(rng, (3, kt, kh, kw, 16), 0.3)
    b = rng.standard_normal(3).astype(np.float32)
    got = O.hr_conv_stage(x, w, b, (kt, kh, kw), act=True, round_output=False)
    xf, wf = O.bf16_to_f64(x), O.bf16_to_f64(w)
    assert got.shape == (1, 2, 2, 3, 3)
    for t in range(2):
        for h in range(2):
            for v in range(3):
                for co in range(3):
                    acc = float(b[co])
                    for dt in range(kt):
                        for dh in range(kh):
                            for dw in range(kw):
                                for ci in range(16):
                                    acc += wf[co, dt, dh, dw, ci] * xf[0, kt * t + dt, kh * h + dh, kw * v + dw, ci]
                    ref = acc / (1.0 + np.exp(-acc))
                    assert abs(got[0, t, h, v, co] - ref) <= 1e-12 * max(1.0, abs(ref))


def test_silu_closed_forms():
    x = np.array([0.0, 1.0, -1.0, 40.0, -40.0, 800.0, -800.0])
    s = O.silu(x)
    assert s[0] == 0.0
    assert abs(s[1] - 1.0 / (1.0 + np.exp(-1.0))) < 1e-15
    assert abs(s[2] + np.exp(-1.0) / (1.0 + np.exp(-1.0))) < 1e-15
    assert abs(s[3] - 40.0) < 1e-15 * 40 and abs(s[4]) < 1e-15
    assert s[5] == 800.0 and s[6] == 0.0 and np.all(np.isfinite(s))
    # silu(x) - silu(-x) = x
    y = np.linspace(-30, 30, 601)
    np.testing.assert_allclose(O.silu(y) - O.silu(-y), y, rtol=0, atol=1e-13)


def test_selection_weights_give_a_strided_slice():
    # a weight with a single 1 at (dt, dh, dw, ci) makes the stage a plain slice of the input
    rng = np.random.default_rng(13)
    x = _bits(rng, (1, 4, 6, 8, 16))
    kernel = (2, 2, 2)
    w = np.zeros((3, 2, 2, 2, 16), np.uint16)
    picks = [(0, 0, 0, 0), (1, 1, 0, 5), (1, 0, 1, 15)]
    for co, (dt, dh, dw, ci) in enumerate(picks):
        w[co, dt, dh, dw, ci] = 0x3F80    # 1.0 in bfloat16
    y = O.hr_conv_stage(x, w, None, kernel, act=False)
    for co, (dt, dh, dw, ci) in enumerate(picks):
        assert np.array_equal(y[..., co], x[:, dt::2, dh::2, dw::2, ci])


def test_default_block_gives_the_pages_token_count():
    # N_c = floor(T/2) floor(H/8) floor(W/8) = 182 tokens and a 128x volume reduction
    lat = pfgen.HR_LATENT
    z = pfgen.hr_latent(5)
    stages, proj = pfgen.hr_weights(6)
    y = O.hr_branch(z, stages, proj)
    assert y.shape == (1, GOLDEN["compressed_tokens"]["value"], pfgen.HR_HIDDEN)
    f = GOLDEN["volume_reduction"]["factors"]
    assert int(np.prod(f)) == GOLDEN["volume_reduction"]["value"] == 128
    assert (lat["frames"] // f[0]) * (lat["height"] // f[1]) * (lat["width"] // f[2]) == 182
    # the 1x2x2 patch embedding of the attention path sees the same grid: h = 60/2, w = 104/2
    assert lat["height"] // 2 == GOLDEN["compressed_tokens"]["inputs"]["h"]
    assert lat["width"] // 2 == GOLDEN["compressed_tokens"]["inputs"]["w"]


def test_dropped_rows_do_not_reach_the_output():
    # the floor: rows past the last whole patch are never read
    rng = np.random.default_rng(14)
    stages, proj = pfgen.hr_weights(7, widths=(32, 32, 32, 32), hidden=48)
    z = pfgen.hr_latent(8, frames=5, height=17, width=9)
    y0 = O.hr_branch(z, stages, proj)
    z2 = z.copy()
    z2[:, 4] = _bits(rng, z2[:, 4].shape)      # frame 4 (T=5 -> 2 outputs use frames 0..3)
    z2[:, :, 16] = _bits(rng, z2[:, :, 16].shape)   # row 16 (H=17 -> 2 outputs use rows 0..15)
    z2[:, :, :, 8] = _bits(rng, z2[:, :, :, 8].shape)  # column 8 (W=9 -> 1 output uses 0..7)
    assert y0.shape == (1, 2 * 2 * 1, 48)
    assert np.array_equal(O.hr_branch(z2, stages, proj), y0)


def test_branch_is_the_stages_in_sequence():
    # the projection is linear (no SiLU) and the token order is t-major
    stages, proj = pfgen.hr_weights(9, widths=(32, 32, 32, 32), hidden=40)
    z = pfgen.hr_latent(10, frames=4, height=16, width=24)
    y = O.hr_branch(z, stages, proj)
    x = z
    for (w, b), k in zip(stages, O.HR_STAGE_KERNELS):
        x = O.hr_conv_stage(x, w, b, k)
    pre = O.bf16_to_f64(x).reshape(-1, 32) @ O.bf16_to_f64(proj[0]).T + proj[1].astype(np.float64)
    assert np.array_equal(y.reshape(-1, 40), O.f64_to_bf16(pre))
    assert y.shape == (1, 2 * 2 * 3, 40)
