"""Pins for the oracle's bf16 / f32 rounding helpers.

Fixed points come from the IEEE bfloat16 format itself (hand-derived bit
patterns) and from independent library conversions (torch float32->bfloat16,
NumPy float64->float32), both of which round to nearest even.
"""

import numpy as np
import pytest
import torch

from oracle.bf16 import bf16_bits_to_f64, f64_to_bf16_bits, round_bf16, round_f32

# (value, expected bf16 bits), derived by hand from the format:
# sign | 8-bit exponent (bias 127) | 7 fraction bits.
HAND = [
    (1.0, 0x3F80),
    (-2.5, 0xC020),                           # -1.25 * 2**1
    (1.0 + 2.0 ** -8, 0x3F80),                # exact tie between 0x3F80 and 0x3F81 -> even
    (1.0 + 3 * 2.0 ** -8, 0x3F82),            # tie between 0x3F81 and 0x3F82 -> even
    (1.0 + 2.0 ** -8 + 2.0 ** -30, 0x3F81),   # just above the tie: up (no double rounding)
    (2.0 ** -133, 0x0001),                    # smallest subnormal
    (1.5 * 2.0 ** -133, 0x0002),              # tie between 1 and 2 quanta -> even
    (0.5 * 2.0 ** -133, 0x0000),              # tie between 0 and 1 quantum -> even (0)
    ((2 - 2.0 ** -7) * 2.0 ** 127, 0x7F7F),   # largest finite
    ((2 - 2.0 ** -8) * 2.0 ** 127, 0x7F80),   # tie above the largest finite -> even = inf
    (0.0, 0x0000),
    (-0.0, 0x8000),
    (2.0 ** -126, 0x0080),                    # smallest normal
]


@pytest.mark.parametrize("value,bits", HAND)
def test_hand_bit_patterns(value, bits):
    assert int(f64_to_bf16_bits(np.array([value]))[0]) == bits


def test_widen_is_exact_and_inverse():
    bits = np.arange(0, 0x10000, dtype=np.uint32).astype(np.uint16)
    vals = bf16_bits_to_f64(bits)
    finite = np.isfinite(vals)
    back = f64_to_bf16_bits(vals[finite])
    # every finite bf16 value rounds to itself (signed zeros included)
    assert np.array_equal(back, bits[finite])


def test_matches_torch_on_float32_inputs():
    rng = np.random.default_rng(0)
    x = np.concatenate([
        rng.standard_normal(200_000).astype(np.float32),
        (rng.standard_normal(50_000) * 1e-38).astype(np.float32),   # subnormal range
        (rng.standard_normal(50_000) * 1e30).astype(np.float32),
    ])
    ours = f64_to_bf16_bits(x.astype(np.float64))
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ours, ref)


def test_round_f32_matches_numpy():
    rng = np.random.default_rng(1)
    x = np.concatenate([rng.standard_normal(100_000), rng.standard_normal(10_000) * 1e-40,
                        rng.standard_normal(10_000) * 1e35])
    assert np.array_equal(round_f32(x), x.astype(np.float32).astype(np.float64))


def test_round_bf16_is_nearest():
    rng = np.random.default_rng(2)
    x = rng.standard_normal(10_000)
    r = round_bf16(x)
    # neighbours on the bf16 grid: the rounded value is no farther than either
    bits = f64_to_bf16_bits(x).astype(np.int64)
    up = bf16_bits_to_f64(((bits + 1) & 0xFFFF).astype(np.uint16))
    dn = bf16_bits_to_f64(((bits - 1) & 0xFFFF).astype(np.uint16))
    assert np.all(np.abs(r - x) <= np.abs(up - x))
    assert np.all(np.abs(r - x) <= np.abs(dn - x))
