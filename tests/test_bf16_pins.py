"""CPU pins of the two bf16 conversions every bf16 workload rests on:
the oracle's exact decode of stored bf16 bits (``oracle.dflash.to_f64``) and
the seeded generator's float32 -> bf16 rounding (``synth.f32_to_bf16_bits``,
nearest with ties to even).

Both are checked against hand-written bit patterns and against a decoder and
a rounder written here from the format's definition alone (sign bit, 8
exponent bits with bias 127, 7 stored mantissa bits; subnormals at exponent
field 0), with Python's exact float arithmetic (``math.ldexp``), so a shared
mistake in the shift formulas of the two modules cannot pass.
"""
import math
import struct

import numpy as np
import pytest

import synth
from oracle import dflash as O


def bf16_value(bits: int) -> float:
    """Value of a bf16 bit pattern from the format's definition."""
    sign = -1.0 if bits >> 15 else 1.0
    e = (bits >> 7) & 0xFF
    m = bits & 0x7F
    if e == 0xFF:
        return sign * math.inf if m == 0 else math.nan
    if e == 0:
        return sign * math.ldexp(m, -126 - 7)          # subnormal: 0.m * 2^-126
    return sign * math.ldexp(128 + m, e - 127 - 7)     # 1.m * 2^(e-127)


def f32_value(bits: int) -> float:
    return struct.unpack("<f", struct.pack("<I", bits))[0]


def round_to_bf16(bits32: int) -> int:
    """Nearest bf16 of a finite float32 (given by its bits), ties to the
    even mantissa, found by comparing the exact distances to the two bf16
    neighbours (no bit tricks)."""
    v = f32_value(bits32)
    sign = bits32 & 0x80000000
    lo = (bits32 >> 16) & 0x7FFF                      # truncation toward zero, magnitude bits
    a, b = bf16_value(lo), bf16_value(lo + 1)         # |v| lies in [a, b)
    dv = abs(v)
    if dv - a < b - dv:
        mag = lo
    elif dv - a > b - dv:
        mag = lo + 1
    else:
        mag = lo if lo % 2 == 0 else lo + 1
    return (sign >> 16) | mag


# (bits, value) fixed by hand
DECODE_CASES = [
    (0x3F80, 1.0),
    (0xBF80, -1.0),
    (0xC040, -3.0),
    (0x4049, 3.140625),
    (0x0001, 2.0 ** -133),                 # smallest subnormal
    (0x007F, 127 * 2.0 ** -133),           # largest subnormal
    (0x0080, 2.0 ** -126),                 # smallest normal
    (0x7F7F, (2.0 - 2.0 ** -7) * 2.0 ** 127),   # largest finite
    (0x3C23, 163 * 2.0 ** -14),            # 0.00994873046875 (weights of std 0.02)
    (0x0000, 0.0),
]

# (float32 bits, bf16 bits) fixed by hand
ROUND_CASES = [
    (0x3F800000, 0x3F80),   # exact
    (0x3F808000, 0x3F80),   # tie, even below: stays
    (0x3F818000, 0x3F82),   # tie, odd below: up to even
    (0x3F808001, 0x3F81),   # just above the tie: up
    (0x3F807FFF, 0x3F80),   # just below the tie: down
    (0x3F80FFFF, 0x3F81),
    (0xBF808000, 0xBF80),   # negative tie stays even
    (0xBF818000, 0xBF82),
    (0x3FFF8000, 0x4000),   # tie, odd: the carry moves into the exponent
    (0x00008000, 0x0000),   # subnormal tie to even (zero)
    (0x00018000, 0x0002),   # subnormal tie, odd below
    (0x7F7F7FFF, 0x7F7F),   # largest finite stays finite
    (0x80000000, 0x8000),   # -0
]


@pytest.mark.parametrize("bits,value", DECODE_CASES)
def test_decode_hand_patterns(bits, value):
    got = float(O.to_f64(np.array([bits], np.uint16), "bf16")[0])
    assert got == value
    assert bf16_value(bits) == value


def test_decode_negative_zero_sign():
    got = O.to_f64(np.array([0x8000], np.uint16), "bf16")[0]
    assert got == 0.0 and math.copysign(1.0, got) == -1.0


def test_decode_every_finite_pattern_against_definition():
    bits = np.arange(1 << 16, dtype=np.uint32)
    finite = ((bits >> 7) & 0xFF) != 0xFF
    got = O.to_f64(bits.astype(np.uint16), "bf16")
    ref = np.array([bf16_value(int(b)) for b in bits[finite]])
    assert np.array_equal(got[finite], ref)
    inf = finite == False  # noqa: E712
    assert np.all(np.isinf(got[inf & ((bits & 0x7F) == 0)]))
    assert np.all(np.isnan(got[inf & ((bits & 0x7F) != 0)]))


@pytest.mark.parametrize("f32,bf", ROUND_CASES)
def test_round_hand_patterns(f32, bf):
    got = int(synth.f32_to_bf16_bits(np.array([f32], np.uint32).view(np.float32))[0])
    assert got == bf, f"{f32:#010x} -> {got:#06x}, expected {bf:#06x}"
    assert round_to_bf16(f32) == bf


def test_round_against_definition_on_random_and_tie_patterns():
    rng = np.random.default_rng(7)
    r = rng.integers(0, 1 << 32, 20000, dtype=np.uint64).astype(np.uint32)
    ties = (rng.integers(0, 1 << 16, 4000, dtype=np.uint64).astype(np.uint32) << 16) | 0x8000
    near = (rng.integers(0, 1 << 16, 4000, dtype=np.uint64).astype(np.uint32) << 16) | \
        rng.choice(np.array([0x7FFF, 0x8001, 0x0001, 0xFFFF], np.uint32), 4000)
    allb = np.concatenate([r, ties, near])
    # finite inputs whose nearest bf16 is finite (no rounding up into inf)
    allb = allb[((allb >> 23) & 0xFF) != 0xFF]
    allb = allb[(allb & 0x7FFFFFFF) < 0x7F7F8000]
    got = synth.f32_to_bf16_bits(allb.view(np.float32))
    ref = np.array([round_to_bf16(int(b)) for b in allb], np.uint16)
    bad = np.nonzero(got != ref)[0]
    assert bad.size == 0, f"{bad.size} mismatches, first {int(allb[bad[0]]):#010x}"


def test_round_is_nearest_on_normal_draws():
    """The rounded weights of a workload are within half a bf16 ulp of the
    float32 draw: the unit roundoff of an 8-bit significand, 2^-8 relative."""
    rng = np.random.default_rng(3)
    v = (rng.standard_normal(5000) * 0.02).astype(np.float32)
    back = O.to_f64(synth.f32_to_bf16_bits(v), "bf16")
    rel = np.abs(back - v.astype(np.float64)) / np.abs(v.astype(np.float64))
    assert float(rel.max()) <= 2.0 ** -8
