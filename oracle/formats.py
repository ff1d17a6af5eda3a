"""Exact decoders for the path's number formats, and fp64 -> bf16 rounding.

Formats (the pages name them only: humming PR #129, benchmark command
``--a_dtype float8e4m3 --b_dtype float4e2m1 --bs_dtype float8e8m0
--c_dtype bfloat16``).  Their bit layouts are the OCP 8-bit floating point
and OCP Microscaling (MX) v1.0 definitions:

  E4M3 (the "FN" variant): 1 sign, 4 exponent (bias 7), 3 mantissa bits;
      exponent field 0 is subnormal, m/8 * 2^-6; S.1111.111 is NaN; no inf;
      largest finite 448.
  E2M1: 1 sign, 2 exponent (bias 1), 1 mantissa bit; exponent field 0 is
      subnormal, m * 0.5; largest 6; no inf or NaN.
  E8M0: 8-bit unsigned exponent, value 2^(code - 127); 0xFF is NaN.
  bf16: top 16 bits of an IEEE binary32 (8 significant bits).

All decodes are exact in fp64.  Test infrastructure only.
"""

from __future__ import annotations

import math

import numpy as np

# E2M1 magnitudes for codes 0..7, as listed in the OCP MX v1.0 element table.
E2M1_VALUES = (0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0)


def _e4m3_decode(code: int) -> float:
    s = -1.0 if code & 0x80 else 1.0
    e = (code >> 3) & 0xF
    m = code & 0x7
    if e == 0xF and m == 0x7:
        return math.nan
    if e == 0:
        return s * math.ldexp(m / 8.0, -6)
    return s * math.ldexp(1.0 + m / 8.0, e - 7)


def _e2m1_decode(code: int) -> float:
    s = -1.0 if code & 0x8 else 1.0
    e = (code >> 1) & 0x3
    m = code & 0x1
    if e == 0:
        return s * 0.5 * m
    return s * math.ldexp(1.0 + 0.5 * m, e - 1)


def e4m3_table() -> np.ndarray:
    """float64[256]: value of every E4M3FN code (NaN at 0x7F and 0xFF)."""
    return np.array([_e4m3_decode(c) for c in range(256)], dtype=np.float64)


def e2m1_table() -> np.ndarray:
    """float64[16]: value of every E2M1 code (codes 8..15 are the negatives)."""
    return np.array([_e2m1_decode(c) for c in range(16)], dtype=np.float64)


def e8m0_value(codes) -> np.ndarray:
    """float64 array: 2^(code-127), NaN for code 255."""
    c = np.asarray(codes, dtype=np.int64)
    v = np.ldexp(1.0, (c - 127).astype(np.int64))
    return np.where(c == 255, np.nan, v)


_BF16_MAX = math.ldexp(2.0 - 2.0 ** -7, 127)


def bf16_rne_bits(x) -> np.ndarray:
    """Round fp64 values to bf16 (round to nearest, ties to even) in ONE step.

    For |x| in [2^(p-1), 2^p) the bf16 quantum is 2^(p-8); below the smallest
    normal 2^-126 it is the subnormal quantum 2^-133.  Results whose magnitude
    exceeds the largest finite bf16 after rounding become +-inf; NaN stays
    NaN (quiet, 0x7FC0).  Returns uint16 bit patterns.
    """
    x = np.asarray(x, dtype=np.float64)
    _, p = np.frexp(x)                      # |x| = m * 2^p, m in [0.5, 1)
    qexp = np.maximum(p.astype(np.int64) - 8, -133)
    with np.errstate(invalid="ignore", over="ignore"):
        q = np.ldexp(np.rint(np.ldexp(x, -qexp)), qexp)   # exact scaling, RNE
        q = np.where(np.abs(q) > _BF16_MAX, np.copysign(np.inf, x), q)
        q32 = q.astype(np.float32)           # exact: <= 8 significant bits
    bits = (q32.view(np.uint32) >> np.uint32(16)).astype(np.uint16)
    bits = np.where(np.isnan(x), np.uint16(0x7FC0), bits)
    return bits.astype(np.uint16)


def bf16_bits_to_f64(bits) -> np.ndarray:
    """uint16 bf16 patterns -> float64 values (exact)."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return b.view(np.float32).astype(np.float64)
