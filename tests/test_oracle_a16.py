"""Pins for the oracle's A16 grouped GEMM (bf16 activations x FP4 weights,
MXFP4 or NVFP4 scales; oracle/a16.py).

* exact rational brute force on tiny shapes, both formats, with decoders of
  its own (bf16 bits through struct, the literal OCP E2M1 value list, E8M0 as
  a power of two, E4M3 through torch's float8_e4m3fn) -- bit-for-bit;
* the W4A8 oracle: bf16 activations equal to E4M3 values times power-of-two
  scales (exact in bf16) and MXFP4 weights give exactly grouped_gemm_f64's
  values -- two independent decodings of the same products;
* MXFP4 scales rewritten as the E4M3 codes of the same powers of two give
  the same NVFP4 result;
* closed forms (all ones; the per-expert scale), sign and scale linearity;
* NaN scale codes poison exactly their columns;
* the magnitude sums match the brute force and bound the results;
* planted mistakes in copies of the decoder (NVFP4 blocks of 32, swapped
  nibbles, the per-expert scale of the wrong expert, MXFP4 blocks of 16)
  each break the brute-force pin.
"""

import struct
from fractions import Fraction

import numpy as np
import pytest
import torch

from oracle import a16 as oa
from oracle import bf16_rne_bits, grouped_gemm_f64
from oracle.a16 import FMT_MX, FMT_NV, grouped_gemm_a16_bf16, grouped_gemm_a16_f64

from test_oracle_formats import _bf16_exact

SPEC_E2M1 = [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]
_DEC8 = torch.arange(256, dtype=torch.uint8).view(torch.float8_e4m3fn).double().numpy()


def _bf16(bits):
    return struct.unpack("<f", struct.pack("<I", int(bits) << 16))[0]


def _dec4(c):
    v = SPEC_E2M1[c & 7]
    return -v if c & 8 else v


def _scale(code, fmt):
    if fmt == FMT_MX:
        return Fraction(2) ** (int(code) - 127)
    return Fraction(float(_DEC8[int(code)]))


def brute_force_bits(A, B, SB, fmt, gs, offsets, blk=None):
    """Exact rational grouped A16 GEMM rounded once to bf16, pure Python."""
    E, N, Kh = B.shape
    K = 2 * Kh
    blk = blk or (32 if fmt == FMT_MX else 16)
    R = int(offsets[E])
    out = np.zeros((R, N), dtype=np.uint16)
    for e in range(E):
        g = Fraction(float(np.float32(gs[e]))) if gs is not None else Fraction(1)
        for r in range(int(offsets[e]), int(offsets[e + 1])):
            for n in range(N):
                acc = Fraction(0)
                for k in range(K):
                    a = _bf16(A[r, k])
                    if a == 0:
                        continue
                    w = _dec4((int(B[e, n, k // 2]) >> (4 * (k % 2))) & 0xF)
                    if w == 0:
                        continue
                    acc += Fraction(a) * Fraction(w) * _scale(SB[e, n, k // blk], fmt)
                out[r, n] = _bf16_exact(acc * g)
    return out


def _problem(counts, N, K, fmt, seed, sb_range=None):
    rng = np.random.default_rng(seed)
    E = len(counts)
    R = int(sum(counts))
    off = np.zeros(E + 1, dtype=np.int64)
    off[1:] = np.cumsum(counts)
    x = rng.standard_normal((R, K)).astype(np.float32)
    A = (x.view(np.uint32) >> 16).astype(np.uint16)          # truncated to bf16 bits
    B = rng.integers(0, 256, size=(E, N, K // 2), dtype=np.uint8)
    blk = 32 if fmt == FMT_MX else 16
    if fmt == FMT_MX:
        lo, hi = sb_range or (118, 136)
        SB = rng.integers(lo, hi, size=(E, N, K // blk), dtype=np.uint8)
        gs = None
    else:
        # finite E4M3 codes of moderate size, both signs (sign bit 0x80)
        mags = rng.integers(0x20, 0x58, size=(E, N, K // blk))
        SB = (mags | (rng.integers(0, 2, size=mags.shape) << 7)).astype(np.uint8)
        gs = rng.uniform(0.25, 4.0, size=E).astype(np.float32)
    return A, B, SB, gs, off


@pytest.mark.parametrize("fmt", [FMT_MX, FMT_NV])
@pytest.mark.parametrize("counts,N,K", [([2, 0, 3], 4, 64), ([1, 2], 3, 96), ([4], 2, 128)])
def test_brute_force_bit_exact(fmt, counts, N, K):
    A, B, SB, gs, off = _problem(counts, N, K, fmt, seed=sum(counts) + N + K + 7 * fmt)
    want = brute_force_bits(A, B, SB, fmt, gs, off)
    got = grouped_gemm_a16_bf16(A, B, SB, fmt, gs, off)
    assert np.array_equal(got, want)


def test_equals_w4a8_oracle_on_fp8_representable_activations():
    """bf16 activations equal to e4m3(code) * 2^p (p per row and 128-K group)
    with the same MXFP4 weights: the A16 oracle must equal the W4A8 oracle
    exactly (every product is exact in both)."""
    rng = np.random.default_rng(3)
    counts, N, K = [5, 0, 7, 2], 16, 256
    E, R = len(counts), sum(counts)
    off = np.zeros(E + 1, dtype=np.int64)
    off[1:] = np.cumsum(counts)
    codes = rng.integers(0, 256, size=(R, K), dtype=np.uint8)
    codes[(codes & 0x7F) == 0x7F] = 0x01          # no NaN codes
    p = rng.integers(-6, 7, size=(R, K // 128))
    SA = np.ldexp(1.0, p).astype(np.float32)
    vals = _DEC8[codes] * np.repeat(SA.astype(np.float64), 128, axis=1)
    A_bits = bf16_rne_bits(vals)
    assert np.array_equal(np.asarray(torch.from_numpy(A_bits.view(np.int16)).view(torch.bfloat16).double()), vals)
    B = rng.integers(0, 256, size=(E, N, K // 2), dtype=np.uint8)
    SB = rng.integers(115, 140, size=(E, N, K // 32), dtype=np.uint8)
    ref = grouped_gemm_f64(codes, SA.reshape(-1), 0, B, SB, off)
    got = grouped_gemm_a16_f64(A_bits, B, SB, FMT_MX, None, off)
    assert np.array_equal(got, ref)


def test_mx_scales_as_e4m3_powers_of_two_give_the_same_result():
    A, B, SB, _, off = _problem([3, 4], 8, 128, FMT_MX, seed=9, sb_range=(121, 135))
    # E4M3 code of 2^(c-127) for c-127 in [-6, 7]: exponent field c-127+7, mantissa 0
    pow2 = np.repeat(SB.astype(np.int64), 2, axis=2)          # each 32-block -> two 16-blocks
    nv = ((pow2 - 127 + 7) << 3).astype(np.uint8)
    assert np.array_equal(_DEC8[nv], np.ldexp(1.0, pow2 - 127))
    mx = grouped_gemm_a16_f64(A, B, SB, FMT_MX, None, off)
    nvr = grouped_gemm_a16_f64(A, B, nv, FMT_NV, np.ones(2, np.float32), off)
    assert np.array_equal(mx, nvr)


def test_closed_forms_and_linearity():
    K, N = 256, 4
    off = np.array([0, 2, 3])
    A = np.full((3, K), 0x3F80, dtype=np.uint16)               # bf16 1.0
    B = np.full((2, N, K // 2), 0x22, dtype=np.uint8)          # E2M1 1.0 in both nibbles
    SBmx = np.full((2, N, K // 32), 127, dtype=np.uint8)
    assert np.all(grouped_gemm_a16_f64(A, B, SBmx, FMT_MX, None, off) == K)
    SBnv = np.full((2, N, K // 16), 0x40, dtype=np.uint8)      # E4M3 2.0
    gs = np.array([0.5, 3.0], np.float32)
    got = grouped_gemm_a16_f64(A, B, SBnv, FMT_NV, gs, off)
    assert np.all(got[:2] == K) and np.all(got[2] == 6 * K)
    A2, B2, SB2, gs2, off2 = _problem([3, 2], 8, 128, FMT_NV, seed=4)
    base = grouped_gemm_a16_f64(A2, B2, SB2, FMT_NV, gs2, off2)
    neg = grouped_gemm_a16_f64(A2 ^ np.uint16(0x8000), B2, SB2, FMT_NV, gs2, off2)
    assert np.array_equal(neg, -base)
    dbl = grouped_gemm_a16_f64(A2, B2, SB2, FMT_NV, gs2 * 2, off2)
    assert np.array_equal(dbl, 2 * base)


@pytest.mark.parametrize("fmt,nan_code", [(FMT_MX, 0xFF), (FMT_NV, 0x7F), (FMT_NV, 0xFF)])
def test_nan_scale_poisons_its_column(fmt, nan_code):
    A, B, SB, gs, off = _problem([2, 3], 6, 128, fmt, seed=12)
    B = B | 0x22                                                # no zero weights (0 * NaN = NaN anyway)
    SB = SB.copy()
    SB[1, 4, 2] = nan_code
    got = grouped_gemm_a16_f64(A, B, SB, fmt, gs, off)
    nan = np.isnan(got)
    assert np.all(nan[2:5, 4]) and nan.sum() == 3


def test_magnitude_sums():
    A, B, SB, gs, off = _problem([2, 2], 3, 64, FMT_NV, seed=21)
    mag = grouped_gemm_a16_f64(A, B, SB, FMT_NV, gs, off, absolute=True)
    val = grouped_gemm_a16_f64(A, B, SB, FMT_NV, gs, off)
    assert np.all(np.abs(val) <= mag * (1 + 1e-15))
    for r, e in ((0, 0), (3, 1)):
        for n in range(3):
            s = sum(abs(Fraction(_bf16(A[r, k])) * Fraction(_dec4((int(B[e, n, k // 2]) >> (4 * (k % 2))) & 0xF))
                        * _scale(SB[e, n, k // 16], FMT_NV)) for k in range(64))
            assert abs(float(s * Fraction(float(gs[e]))) - mag[r, n]) <= 1e-13 * mag[r, n]


def _planted(mistake):
    """A copy of the decoder with one mistake, as grouped_gemm_a16_bf16."""
    def f(A, B, SB, fmt, gs, off):
        orig_block, orig_dec = oa.block_of, oa.decode_weights_a16
        try:
            if mistake == "nv_block_32":
                oa.block_of = lambda fm: 32 if fm == FMT_NV else orig_block(fm)
                SBx = SB[:, :, ::2]
                return bf16_rne_bits(oa.grouped_gemm_a16_f64(A, B, SBx, fmt, gs, off))
            if mistake == "mx_block_16":
                oa.block_of = lambda fm: 16 if fm == FMT_MX else orig_block(fm)
                SBx = np.repeat(SB, 2, axis=2)[:, :, : SB.shape[2] * 2]
                SBx = SBx.copy()
                SBx[:, :, 1::2] = np.roll(SB, 1, axis=2)            # the second half-block reads its neighbour's code
                return bf16_rne_bits(oa.grouped_gemm_a16_f64(A, B, SBx, fmt, gs, off))
            if mistake == "nibbles":
                Bx = ((B & 0x0F) << 4) | (B >> 4)
                return bf16_rne_bits(oa.grouped_gemm_a16_f64(A, Bx, SB, fmt, gs, off))
            if mistake == "gs_expert":
                gx = None if gs is None else np.roll(gs, 1)
                return bf16_rne_bits(oa.grouped_gemm_a16_f64(A, B, SB, fmt, gx, off))
        finally:
            oa.block_of, oa.decode_weights_a16 = orig_block, orig_dec
    return f


@pytest.mark.parametrize("mistake,fmt", [("nv_block_32", FMT_NV), ("mx_block_16", FMT_MX),
                                         ("nibbles", FMT_MX), ("nibbles", FMT_NV), ("gs_expert", FMT_NV)])
def test_planted_mistakes_break_the_brute_force_pin(mistake, fmt):
    A, B, SB, gs, off = _problem([2, 3], 4, 64, fmt, seed=33)
    want = brute_force_bits(A, B, SB, fmt, gs, off)
    assert np.array_equal(grouped_gemm_a16_bf16(A, B, SB, fmt, gs, off), want)
    assert not np.array_equal(_planted(mistake)(A, B, SB, fmt, gs, off), want)
