"""Bit-pattern pins of the two bf16 conversions both sides rely on:

- oracle.numerics.bf16_bits_to_f64: the oracle's exact upcast of stored
  bf16 bit patterns;
- synth.generators.f32_to_bf16_bits: the generator's rounding of fp32 draws
  to bf16 (nearest, ties to even), which fixes every bf16 input.

A bf16 value is sign, 8 exponent bits and 7 fraction bits: the upper half of
an IEEE binary32.  The expected values below come from that definition
(hand-computed constants), from an integer-only rounding written here from
the definition of round-to-nearest-even, and from torch's own fp32 -> bf16
conversion (a library routine)."""

import math

import numpy as np
import torch

from oracle.numerics import bf16_bits_to_f64
from synth.generators import f32_to_bf16_bits


# (bits, value): hand-worked from sign / exponent / fraction
KNOWN = [
    (0x3F80, 1.0),
    (0xBF80, -1.0),
    (0x4000, 2.0),
    (0x3F00, 0.5),
    (0x4049, 3.140625),                  # 1.5703125 * 2
    (0x3FC0, 1.5),
    (0x3F81, 1.0 + 2.0 ** -7),           # one ulp above 1
    (0x7F7F, (2.0 - 2.0 ** -7) * 2.0 ** 127),   # largest finite
    (0xFF7F, -(2.0 - 2.0 ** -7) * 2.0 ** 127),
    (0x0080, 2.0 ** -126),               # smallest normal
    (0x0001, 2.0 ** -133),               # smallest subnormal
    (0x007F, 127 * 2.0 ** -133),         # largest subnormal
]


def test_upcast_known_values():
    bits = np.array([b for b, _ in KNOWN], dtype=np.uint16)
    got = bf16_bits_to_f64(bits)
    assert got.dtype == np.float64
    for (b, want), g in zip(KNOWN, got):
        assert g == want, (hex(b), g, want)


def test_upcast_signed_zero_and_infinities():
    got = bf16_bits_to_f64(np.array([0x0000, 0x8000, 0x7F80, 0xFF80], dtype=np.uint16))
    assert got[0] == 0.0 and not math.copysign(1.0, got[0]) < 0
    assert got[1] == 0.0 and math.copysign(1.0, got[1]) < 0
    assert got[2] == math.inf and got[3] == -math.inf


def test_upcast_every_finite_pattern_from_the_definition():
    """All 65,536 patterns against (-1)^s * 2^(e-127) * (1 + f/128) (normal)
    and (-1)^s * 2^-126 * f/128 (subnormal), computed with Python floats."""
    allb = np.arange(1 << 16, dtype=np.uint32)
    bits = allb[((allb >> 7) & 0xFF) != 0xFF].astype(np.uint16)   # finite patterns
    got = bf16_bits_to_f64(bits)
    for b, g in zip(bits.tolist(), got.tolist()):
        s, e, f = b >> 15, (b >> 7) & 0xFF, b & 0x7F
        mag = math.ldexp(f / 128.0, -126) if e == 0 else math.ldexp(1.0 + f / 128.0, e - 127)
        want = -mag if s else mag
        assert g == want and math.copysign(1.0, g) == math.copysign(1.0, want), hex(b)


def rne_reference(x32: np.ndarray) -> np.ndarray:
    """fp32 -> bf16 bits by the definition: keep the upper 16 bits, look at
    the 16 dropped ones; above half round up, below round down, at exactly
    half round to the even one of the two neighbours.  (Integer logic only;
    finite inputs.)"""
    u = np.ascontiguousarray(x32, dtype=np.float32).view(np.uint32).astype(np.int64)
    upper, low = u >> 16, u & 0xFFFF
    up = (low > 0x8000) | ((low == 0x8000) & ((upper & 1) == 1))
    return (upper + up).astype(np.uint16)


def f32(bits):
    return np.array([bits], dtype=np.uint32).view(np.float32)


def test_round_known_cases():
    cases = [
        (1.0, 0x3F80),
        (-0.0, 0x8000),
        (0.0, 0x0000),
        (1.0 + 2.0 ** -8, 0x3F80),               # exactly half an ulp above 1: tie, 0x3F80 is even
        (1.0 + 3 * 2.0 ** -8, 0x3F82),           # tie between 0x3F81 and 0x3F82: the even one
        (1.0 + 2.0 ** -8 + 2.0 ** -20, 0x3F81),  # just above the tie
        (1.0 + 2.0 ** -8 - 2.0 ** -20, 0x3F80),  # just below the tie
        (-(1.0 + 3 * 2.0 ** -8), 0xBF82),
        (3.14159265, 0x4049),
    ]
    for x, want in cases:
        got = int(f32_to_bf16_bits(np.array([x], dtype=np.float32))[0])
        assert got == want, (x, hex(got), hex(want))
    # the top of the range: a tie at the largest finite bf16 (odd) rounds up
    # to infinity, just below the tie rounds down to it
    assert int(f32_to_bf16_bits(f32(0x7F7F7FFF))[0]) == 0x7F7F
    assert int(f32_to_bf16_bits(f32(0x7F7F8000))[0]) == 0x7F80
    assert int(f32_to_bf16_bits(f32(0x7F7FFFFF))[0]) == 0x7F80
    # subnormals round like any other pattern
    assert int(f32_to_bf16_bits(f32(0x00018000))[0]) == 0x0002   # tie, 0x0001 odd -> 0x0002
    assert int(f32_to_bf16_bits(f32(0x00008000))[0]) == 0x0000   # tie, 0x0000 even


def test_round_matches_definition_and_torch_on_random_patterns():
    rng = np.random.default_rng(2024)
    bits = rng.integers(0, 1 << 32, size=200_000, dtype=np.uint64).astype(np.uint32)
    bits = bits[((bits >> 23) & 0xFF) != 0xFF]             # finite patterns only
    # plus every tie and its neighbours for a spread of upper halves
    uppers = rng.integers(0, 0x7F7F, size=2000, dtype=np.uint32) << 16
    ties = np.concatenate([uppers | 0x8000, uppers | 0x7FFF, uppers | 0x8001,
                           (uppers | 0x8000) | 0x80000000])
    bits = np.concatenate([bits, ties.astype(np.uint32)])
    x = bits.view(np.float32)
    got = f32_to_bf16_bits(x)
    np.testing.assert_array_equal(got, rne_reference(x))
    lib = torch.from_numpy(x.copy()).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    np.testing.assert_array_equal(got, lib)


def test_round_trip_is_identity_on_bf16_values():
    """Every finite bf16 value, widened to fp32, rounds back to itself."""
    b = np.arange(1 << 16, dtype=np.uint32)
    b = b[((b >> 7) & 0xFF) != 0xFF].astype(np.uint16)
    x32 = (b.astype(np.uint32) << 16).view(np.float32)
    np.testing.assert_array_equal(f32_to_bf16_bits(x32), b)
    np.testing.assert_array_equal(bf16_bits_to_f64(b), x32.astype(np.float64))
