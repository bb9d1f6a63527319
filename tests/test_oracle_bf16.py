"""bfloat16 rounding used by the oracle and by the input generator."""
import numpy as np
import torch

import oracle as O
import pfgen


def test_hand_values():
    x = np.array([1.0, 1 + 2**-8, 1 + 3 * 2**-8, 1 + 2**-8 + 2**-30, -2.0, 0.0, -0.0,
                  2.0**-133, 2.0**-134, 3 * 2.0**-134, 1e39])
    got = O.f64_to_bf16(x)
    want = [0x3F80, 0x3F80, 0x3F82, 0x3F81, 0xC000, 0x0000, 0x8000, 0x0001, 0x0000, 0x0002, 0x7F80]
    assert [int(v) for v in got] == want


def test_against_torch_rne():
    rng = np.random.default_rng(5)
    x = (rng.standard_normal(200000) * np.exp(rng.uniform(-20, 20, 200000))).astype(np.float32)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(O.f64_to_bf16(x.astype(np.float64)), ref)
    assert np.array_equal(pfgen.bf16_bits(x), ref)


def test_roundtrip_exact():
    bits = np.arange(0, 0x7F80, 7, dtype=np.uint16)
    assert np.array_equal(O.f64_to_bf16(O.bf16_to_f64(bits)), bits)
    neg = bits | np.uint16(0x8000)
    assert np.array_equal(O.f64_to_bf16(O.bf16_to_f64(neg)), neg)
