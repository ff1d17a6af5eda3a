"""Pins for the oracle's decoders and its fp64 -> bf16 rounding.

Independent sources: torch's float8_e4m3fn / float8_e8m0fnu dtypes (a separate
implementation of the OCP formats), the OCP MX v1.0 E2M1 value list written
out literally here, torch's fp32 -> bf16 cast (RNE) and exact rational
rounding with fractions.Fraction.
"""

import math
import random
from fractions import Fraction

import numpy as np
import pytest
import torch

from oracle import bf16_bits_to_f64, bf16_rne_bits, e2m1_table, e4m3_table, e8m0_value


def test_e4m3_table_matches_torch_dtype():
    ours = e4m3_table()
    ref = torch.arange(256, dtype=torch.uint8).view(torch.float8_e4m3fn).double().numpy()
    assert np.isnan(ours[0x7F]) and np.isnan(ours[0xFF])
    assert np.array_equal(np.isnan(ours), np.isnan(ref))
    ok = ~np.isnan(ref)
    assert np.array_equal(ours[ok], ref[ok])


def test_e4m3_spec_points():
    t = e4m3_table()
    assert t[0x38] == 1.0
    assert t[0x7E] == 448.0 and t[0xFE] == -448.0
    assert t[0x01] == 2.0 ** -9          # smallest subnormal
    assert t[0x08] == 2.0 ** -6          # smallest normal
    assert t[0x00] == 0.0 and math.copysign(1.0, t[0x80]) == -1.0
    assert np.nanmax(np.abs(t)) == 448.0


def test_e2m1_table_matches_spec_list():
    # OCP MX v1.0, FP4 E2M1 element values for the 8 positive codes
    spec = [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]
    t = e2m1_table()
    assert list(t[:8]) == spec
    assert list(t[8:]) == [-v for v in spec]
    assert t[0x2] == 1.0 and t[0x7] == 6.0


def test_e8m0_matches_torch_dtype():
    codes = np.arange(256)
    ours = e8m0_value(codes)
    ref = torch.arange(256, dtype=torch.uint8).view(torch.float8_e8m0fnu).double().numpy()
    assert np.isnan(ours[255]) and np.isnan(ref[255])
    assert np.array_equal(ours[:255], ref[:255])
    assert ours[127] == 1.0 and ours[0] == 2.0 ** -127 and ours[254] == 2.0 ** 127


def test_bf16_matches_torch_on_fp32_inputs():
    rng = np.random.default_rng(7)
    bits = rng.integers(0, 2 ** 32, size=200_000, dtype=np.uint64).astype(np.uint32)
    x32 = bits.view(np.float32)
    x32 = x32[np.isfinite(x32)]
    # add exact ties: low 16 bits == 0x8000 with both parities of bit 16
    tie = (rng.integers(0, 2 ** 16, size=5000, dtype=np.uint64).astype(np.uint32) << 16) | 0x8000
    tie32 = tie.view(np.float32)
    x32 = np.concatenate([x32, tie32[np.isfinite(tie32)]])
    ref = torch.from_numpy(x32.copy()).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    ours = bf16_rne_bits(x32.astype(np.float64))
    assert np.array_equal(ours, ref)


def _bf16_exact(q: Fraction) -> int:
    """Independent exact RNE of a rational to bf16 bits (finite inputs)."""
    if q == 0:
        return 0
    sign = 0x8000 if q < 0 else 0
    a = abs(q)
    p = a.numerator.bit_length() - a.denominator.bit_length()
    while Fraction(2) ** p <= a:
        p += 1
    while Fraction(2) ** (p - 1) > a:
        p -= 1
    quantum = Fraction(2) ** max(p - 8, -133)
    n = a / quantum
    fl = n.numerator // n.denominator
    rem = n - fl
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and fl % 2 == 1):
        fl += 1
    v = fl * quantum
    if v > Fraction(2) ** 127 * (2 - Fraction(1, 128)):
        return sign | 0x7F80
    f32 = np.float32(float(v))
    return sign | int(np.array([f32]).view(np.uint32)[0] >> 16)


def test_bf16_matches_exact_rational_rounding_near_ties():
    rnd = random.Random(11)
    xs = []
    for _ in range(3000):
        e = rnd.randint(-140, 126)
        mant = rnd.randint(128, 255)              # 8-bit significand
        base = math.ldexp(mant + 0.5, e)          # exact midpoint
        eps = math.ldexp(1.0, e - 30)
        xs += [base, base + eps, base - eps, -base, math.ldexp(rnd.random() + 0.5, e)]
    xs = [x for x in xs if math.isfinite(x)]
    ours = bf16_rne_bits(np.array(xs))
    ref = np.array([_bf16_exact(Fraction(x)) for x in xs], dtype=np.uint16)
    assert np.array_equal(ours, ref)


def test_bf16_special_values():
    big = math.ldexp(2.0 - 2.0 ** -8, 127)   # halfway to 2^128: ties to even -> inf
    vals = np.array([0.0, -0.0, np.inf, -np.inf, np.nan, big, -big, 1e300, 2.0 ** -134, 2.0 ** -133])
    b = bf16_rne_bits(vals)
    assert b[0] == 0x0000 and b[1] == 0x8000
    assert b[2] == 0x7F80 and b[3] == 0xFF80
    assert (b[4] & 0x7F80) == 0x7F80 and (b[4] & 0x7F) != 0
    assert b[5] == 0x7F80 and b[6] == 0xFF80 and b[7] == 0x7F80
    assert b[8] == 0x0000       # half the smallest subnormal: tie to even (0)
    assert b[9] == 0x0001       # smallest bf16 subnormal
    back = bf16_bits_to_f64(np.array([0x3F80, 0xC000, 0x0001], dtype=np.uint16))
    assert list(back) == [1.0, -2.0, 2.0 ** -133]


@pytest.mark.parametrize("x", [1.0, 3.0, -7.5, 2.0 ** -130])
def test_bf16_exact_values_roundtrip(x):
    assert bf16_bits_to_f64(bf16_rne_bits(np.array([x])))[0] == x
