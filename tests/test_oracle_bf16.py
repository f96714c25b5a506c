"""Pins for the oracle's float64 -> bf16 rounding (CPU only).

torch's float32 -> bfloat16 conversion rounds to nearest, ties to even.  On
float64 inputs that are exactly representable in float32 the two conversions
must agree bit for bit (no double rounding can occur then).
"""

import numpy as np
import torch

from oracle import bf16_bits_to_f64, f64_to_bf16_bits, round_to_bf16


def _torch_bits(x32: np.ndarray) -> np.ndarray:
    t = torch.from_numpy(x32.copy()).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16)


def test_rne_matches_torch_on_float32_values():
    rng = np.random.default_rng(1)
    x = rng.standard_normal(200_000).astype(np.float32) * np.float32(3.0)
    x = np.concatenate([x, x * np.float32(1e-30), x * np.float32(1e30)])
    np.testing.assert_array_equal(f64_to_bf16_bits(x.astype(np.float64)), _torch_bits(x))


def test_rne_exact_ties_go_to_even():
    rng = np.random.default_rng(2)
    hi = rng.integers(0, 0x7F00, size=5000, dtype=np.uint32)
    bits = (hi << np.uint32(16)) | np.uint32(0x8000)  # exactly half an ulp above
    x = bits.view(np.float32)
    got = f64_to_bf16_bits(x.astype(np.float64))
    np.testing.assert_array_equal(got, _torch_bits(x))
    # ties resolve to the even neighbour
    assert np.all(got % 2 == 0)


def test_rne_special_values():
    x = np.array([0.0, -0.0, np.inf, -np.inf, 1.0, -2.0, 2.0**-126, 2.0**-133, 2.0**-134 * 1.5])
    got = round_to_bf16(x)
    assert got[0] == 0.0 and got[1] == 0.0 and np.signbit(got[1])
    assert np.isposinf(got[2]) and np.isneginf(got[3])
    assert got[4] == 1.0 and got[5] == -2.0
    assert got[6] == 2.0**-126  # smallest normal
    assert got[7] == 2.0**-133  # smallest subnormal
    assert got[8] == 2.0**-133  # 1.5 quanta of 2**-134 = 0.75 * 2**-133 -> 2**-133
    assert np.isnan(round_to_bf16(np.array([np.nan]))[0])
    big = np.array([3.3895313892515355e38, 3.40e38])  # max bf16, then above the halfway point
    out = round_to_bf16(big)
    assert out[0] == 3.3895313892515355e38 and np.isposinf(out[1])


def test_bits_roundtrip():
    u = np.arange(0, 0x7F80, 7, dtype=np.uint16)
    np.testing.assert_array_equal(f64_to_bf16_bits(bf16_bits_to_f64(u)), u)
