"""GPU parity of the HR-branch compressor (PackForcing arXiv HTML, "HR Branch:
Progressive 3D Convolution"; "Feature Fusion") against the oracle.

Per stage the GPU gets the oracle's own input, so the bar is the rounding of
one stage: the GPU accumulates in fp32 and rounds to bf16, the oracle rounds
the exact value. An element may therefore differ by one bf16 ulp, or, where
the sum cancels, by the fp32 summation bound K * 2^-24 * sum|w x| (any order),
plus SiLU's slope (< 1.1) times the fp32 error of the exp2/reciprocal.
The chained branch compounds those one-ulp differences over five GEMMs.
"""
import numpy as np
import pytest
import torch

import oracle as O
import pfgen
from gpu_util import dev, host, say, ulp_diff

import bounded_kv_cache_pf_amd as pf

pytestmark = pytest.mark.gpu


def _f32(a):
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).cuda()


def _stage_bound(x_bits, w_bits, bias, kernel, act):
    """Per-element error bound of one GPU stage against the oracle (see module doc)."""
    pre = O.hr_conv_stage(x_bits, w_bits, bias, kernel, act=False, round_output=False)
    # sum |w||x| per output element: the same strided convolution on absolute values
    ax = O.f64_to_bf16(np.abs(O.bf16_to_f64(x_bits)))     # |x| is exact in bf16
    aw = O.f64_to_bf16(np.abs(O.bf16_to_f64(w_bits)))
    l1 = O.hr_conv_stage(ax, aw, None, kernel, act=False, round_output=False)
    K = int(np.prod(kernel)) * x_bits.shape[-1]
    ref = O.hr_conv_stage(x_bits, w_bits, bias, kernel, act=act, round_output=False)
    mag = np.abs(ref)
    ulp = np.where(mag > 0, 2.0 ** (np.floor(np.log2(np.maximum(mag, 1e-300))) - 7), 2.0 ** -133)
    slope = 1.1 if act else 1.0
    return ulp + slope * (K * 2.0 ** -24 * (l1 + np.abs(bias if bias is not None else 0)[None]) +
                          2.0 ** -22 * np.abs(pre)) + 1e-30


def _check_stage(x_bits, w_bits, bias, kernel, act, label):
    y = pf.pf_hr_conv(dev(x_bits), dev(w_bits), None if bias is None else _f32(bias), kernel, act=act)
    torch.cuda.synchronize()
    got = host(y)
    ref_bits = O.hr_conv_stage(x_bits, w_bits, bias, kernel, act=act)
    assert got.shape == ref_bits.shape
    diff = np.abs(O.bf16_to_f64(got) - O.bf16_to_f64(ref_bits))
    bound = _stage_bound(x_bits, w_bits, bias, kernel, act)
    exact = float(np.mean(got == ref_bits))
    say(f"  {label}: shape {got.shape}, exact {exact:.5f}, max ulp {int(ulp_diff(got, ref_bits).max())}, "
        f"max diff/bound {float((diff / bound).max()):.3f}")
    assert np.all(diff <= bound)
    assert exact >= 0.98
    return got


def test_hr_stages_default_block():
    # the default latent block through the four strided stages and the projection,
    # each stage fed the oracle's previous output
    say("test_hr_stages_default_block")
    z = pfgen.hr_latent(2001)
    stages, (wp, bp) = pfgen.hr_weights(2002)
    x = z
    for s, ((w, b), k) in enumerate(zip(stages, O.HR_STAGE_KERNELS)):
        _check_stage(x, w, b, k, True, f"stage {s} kernel {k}")
        x = O.hr_conv_stage(x, w, b, k, act=True)
    _check_stage(x, wp.reshape(wp.shape[0], 1, 1, 1, -1), bp, (1, 1, 1), False, "projection")


def test_hr_conv_ragged_and_no_bias():
    # positions and channels that fill no whole tile, odd input sizes (floored), no bias, no SiLU
    say("test_hr_conv_ragged_and_no_bias")
    rng = np.random.default_rng(2003)
    x = pfgen.bf16_bits(rng.standard_normal((3, 5, 17, 27, 48)).astype(np.float32))
    for kernel, c_out, act in (((1, 2, 2), 80, False), ((2, 1, 1), 16, True), ((2, 2, 2), 112, True),
                               ((1, 1, 1), 48, False)):
        w = pfgen.bf16_bits(rng.standard_normal((c_out,) + kernel + (48,)).astype(np.float32) * 0.1)
        _check_stage(x, w, None, kernel, act, f"kernel {kernel} c_out {c_out} act {act}")


def test_hr_conv_split_k_paths():
    # deep, narrow stages take the split-K path (fp32 partials + ordered reduction)
    say("test_hr_conv_split_k_paths")
    rng = np.random.default_rng(2004)
    for (T, H, W, ci, co) in ((2, 14, 26, 1024, 2048), (2, 8, 8, 2048, 128), (1, 2, 2, 4096, 64)):
        need = pf.pf_hr_conv_workspace_bytes(1, T, H, W, ci, (1, 2, 2), co)
        x = pfgen.bf16_bits(rng.standard_normal((1, T, H, W, ci)).astype(np.float32))
        w = pfgen.bf16_bits(rng.standard_normal((co, 1, 2, 2, ci)).astype(np.float32) * np.sqrt(2.0 / (4 * ci)))
        b = rng.standard_normal(co).astype(np.float32) * 0.1
        _check_stage(x, w, b, (1, 2, 2), True, f"{T}x{H}x{W}x{ci} -> {co} (workspace {need} B)")


def test_hr_branch_chained_default_and_batched():
    say("test_hr_branch_chained_default_and_batched")
    stages, (wp, bp) = pfgen.hr_weights(2005)
    ds = [(dev(w), _f32(b)) for w, b in stages]
    dp = (dev(wp), _f32(bp))
    for batch, seed in ((1, 2006), (3, 2007)):
        z = pfgen.hr_latent(seed, batch=batch)
        out = pf.pf_hr_branch(dev(z), ds, dp)
        out2 = pf.pf_hr_branch(dev(z), ds, dp)
        torch.cuda.synchronize()
        got = host(out)
        assert np.array_equal(got, host(out2))          # bit-reproducible
        ref = O.hr_branch(z, stages, (wp, bp))
        assert got.shape == ref.shape == (batch, 182, 1536)
        g, r = O.bf16_to_f64(got), O.bf16_to_f64(ref)
        rms = float(np.sqrt(np.mean(r ** 2)))
        rel = float(np.linalg.norm(g - r) / np.linalg.norm(r))
        mx = float(np.abs(g - r).max())
        say(f"  batch {batch}: rel-L2 {rel:.2e}, max-abs {mx:.3e} (rms {rms:.3f}), exact {np.mean(got == ref):.4f}")
        assert rel <= 5e-3 and mx <= 3e-2 * rms


def test_hr_branch_small_odd_block():
    # a latent whose sizes are not multiples of the strides: the floors drop the tail
    say("test_hr_branch_small_odd_block")
    stages, (wp, bp) = pfgen.hr_weights(2008, widths=(32, 48, 64, 80), hidden=96)
    z = pfgen.hr_latent(2009, batch=2, frames=5, height=17, width=26)
    out = pf.pf_hr_branch(dev(z), [(dev(w), _f32(b)) for w, b in stages], (dev(wp), _f32(bp)))
    torch.cuda.synchronize()
    ref = O.hr_branch(z, stages, (wp, bp))
    got = host(out)
    assert got.shape == ref.shape == (2, 2 * 2 * 3, 96)
    g, r = O.bf16_to_f64(got), O.bf16_to_f64(ref)
    rel = float(np.linalg.norm(g - r) / np.linalg.norm(r))
    say(f"  rel-L2 {rel:.2e}, exact {np.mean(got == ref):.4f}")
    assert rel <= 5e-3
