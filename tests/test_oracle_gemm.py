"""Pins for the oracle's grouped GEMM.

* exact rational brute force on tiny shapes (independent decoders: torch's
  float8 dtypes for E4M3 and E8M0, the literal OCP E2M1 value list, our own
  nibble unpacking and exact bf16 rounding) -- bit-for-bit equality;
* closed forms: all-ones inputs give K * scale products, one-hot rows give a
  single product (both exactly representable, so exact bits);
* linearity and sign symmetry, layout independence, expert relabelling,
  grouped == concatenation of independent per-expert dense GEMMs, empty
  experts contribute nothing;
* planted mistakes in copies of the oracle must each break a pin.
"""

from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle
from oracle import gemm as og
from oracle import bf16_rne_bits, grouped_gemm_bf16, grouped_gemm_f64

from test_oracle_formats import _bf16_exact

SPEC_E2M1 = [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]
_DEC8 = torch.arange(256, dtype=torch.uint8).view(torch.float8_e4m3fn).double().numpy()


def _dec4(c):
    v = SPEC_E2M1[c & 7]
    return -v if c & 8 else v


def brute_force_bits(A, SA, layout, B, SB, offsets):
    """Exact rational grouped GEMM rounded once to bf16, pure Python."""
    E, N, Kh = B.shape
    K = 2 * Kh
    R = int(offsets[E])
    G = K // 128
    out = np.zeros((R, N), dtype=np.uint16)
    for e in range(E):
        for r in range(int(offsets[e]), int(offsets[e + 1])):
            for n in range(N):
                acc = Fraction(0)
                for k in range(K):
                    a = _DEC8[A[r, k]]
                    if a == 0:
                        continue
                    byte = int(B[e, n, k // 2])
                    w = _dec4((byte >> (4 * (k % 2))) & 0xF)
                    if w == 0:
                        continue
                    s = SA[r * G + k // 128] if layout == 0 else SA[(k // 128) * R + r]
                    acc += (Fraction(a) * Fraction(float(s)) * Fraction(w)
                            * Fraction(2) ** (int(SB[e, n, k // 32]) - 127))
                out[r, n] = _bf16_exact(acc)
    return out


def random_case(rng, E, N, K, rows_per_expert, sb_lo=110, sb_hi=135):
    offsets = np.concatenate([[0], np.cumsum(rows_per_expert)]).astype(np.int32)
    R = int(offsets[-1])
    A = rng.integers(0, 256, size=(R, K), dtype=np.uint8)
    A[(A & 0x7F) == 0x7F] = 0x38          # no NaN codes
    SA = (rng.random(R * (K // 128)) * 4 + 0.01).astype(np.float32)
    B = rng.integers(0, 256, size=(E, N, K // 2), dtype=np.uint8)
    SB = rng.integers(sb_lo, sb_hi, size=(E, N, K // 32), dtype=np.uint8)
    return A, SA, B, SB, offsets


@pytest.mark.parametrize("layout", [0, 1])
def test_bruteforce_bitexact(layout):
    rng = np.random.default_rng(100 + layout)
    A, SA, B, SB, off = random_case(rng, E=3, N=5, K=256, rows_per_expert=[2, 0, 3])
    R = int(off[-1])
    if layout == 1:
        SA = SA.reshape(R, -1).T.copy().reshape(-1)
    ours = grouped_gemm_bf16(A, SA, layout, B, SB, off)
    assert np.array_equal(ours, brute_force_bits(A, SA, layout, B, SB, off))


def test_bruteforce_single_row_k512():
    rng = np.random.default_rng(5)
    A, SA, B, SB, off = random_case(rng, E=1, N=16, K=512, rows_per_expert=[1])
    ours = grouped_gemm_bf16(A, SA, 0, B, SB, off)
    assert np.array_equal(ours, brute_force_bits(A, SA, 0, B, SB, off))


def test_all_ones_closed_form():
    E, N, K = 2, 8, 512
    off = np.array([0, 3, 7], dtype=np.int32)
    R = 7
    A = np.full((R, K), 0x38, dtype=np.uint8)          # E4M3 1.0
    B = np.full((E, N, K // 2), 0x22, dtype=np.uint8)  # E2M1 1.0 in both nibbles
    SB = np.full((E, N, K // 32), 120, dtype=np.uint8)
    SA = np.full(R * (K // 128), 0.125, dtype=np.float32)
    f = grouped_gemm_f64(A, SA, 0, B, SB, off)
    assert np.all(f == K * 0.125 * 2.0 ** -7)
    # per-block scales: C = sum_b 32 * SA(r, b//4) * 2^(SB[n,b]-127)
    rng = np.random.default_rng(1)
    SB2 = rng.integers(115, 125, size=SB.shape).astype(np.uint8)
    SA2 = (2.0 ** rng.integers(-4, 3, size=SA.shape)).astype(np.float32)
    got = grouped_gemm_bf16(A, SA2, 0, B, SB2, off)
    for r in range(R):
        e = 0 if r < 3 else 1
        for n in range(N):
            exact = sum(Fraction(32) * Fraction(float(SA2[r * 4 + b // 4]))
                        * Fraction(2) ** (int(SB2[e, n, b]) - 127) for b in range(K // 32))
            assert got[r, n] == _bf16_exact(exact)


def test_one_hot_closed_form_every_position():
    rng = np.random.default_rng(3)
    E, N, K = 1, 4, 256
    B = rng.integers(0, 256, size=(E, N, K // 2), dtype=np.uint8)
    SB = rng.integers(118, 130, size=(E, N, K // 32), dtype=np.uint8)
    for k0 in range(K):
        A = np.zeros((1, K), dtype=np.uint8)
        A[0, k0] = 0x4C  # E4M3: exponent 9, mantissa 4 -> 6.0
        SA = np.array([0.5, 0.25], dtype=np.float32)
        got = grouped_gemm_f64(A, SA, 0, B, SB, np.array([0, 1]))
        for n in range(N):
            byte = int(B[0, n, k0 // 2])
            w = _dec4((byte >> (4 * (k0 % 2))) & 0xF)
            want = 6.0 * float(SA[k0 // 128]) * w * 2.0 ** (int(SB[0, n, k0 // 32]) - 127)
            assert got[0, n] == want


def test_linearity_and_sign():
    rng = np.random.default_rng(9)
    A, SA, B, SB, off = random_case(rng, E=4, N=32, K=384, rows_per_expert=[5, 1, 0, 9])
    base = grouped_gemm_f64(A, SA, 0, B, SB, off)
    assert np.array_equal(grouped_gemm_f64(A, SA * np.float32(2), 0, B, SB, off), 2 * base)
    Bneg = B ^ np.uint8(0x88)                       # flip both E2M1 sign bits
    assert np.array_equal(grouped_gemm_f64(A, SA, 0, Bneg, SB, off), -base)
    SBp = SB + np.uint8(1)
    assert np.array_equal(grouped_gemm_f64(A, SA, 0, B, SBp, off), 2 * base)


def test_layouts_agree():
    rng = np.random.default_rng(12)
    A, SA, B, SB, off = random_case(rng, E=3, N=16, K=512, rows_per_expert=[7, 0, 4])
    R = int(off[-1])
    mm = SA.reshape(R, -1).T.copy().reshape(-1)
    assert np.array_equal(grouped_gemm_bf16(A, SA, 0, B, SB, off),
                          grouped_gemm_bf16(A, mm, 1, B, SB, off))


def test_grouped_equals_concat_of_dense_and_relabel():
    rng = np.random.default_rng(21)
    rows = [6, 0, 3, 11]
    A, SA, B, SB, off = random_case(rng, E=4, N=24, K=256, rows_per_expert=rows)
    G = 2
    full = grouped_gemm_f64(A, SA, 0, B, SB, off)
    parts = []
    for e in range(4):
        lo, hi = int(off[e]), int(off[e + 1])
        parts.append(grouped_gemm_f64(A[lo:hi], SA[lo * G:hi * G], 0, B[e:e + 1], SB[e:e + 1],
                                      np.array([0, hi - lo])))
    assert np.array_equal(full, np.concatenate(parts, axis=0))
    # relabel experts: reversed order permutes the output row blocks
    perm = [3, 2, 1, 0]
    blocks = [np.arange(off[e], off[e + 1]) for e in perm]
    ridx = np.concatenate(blocks)
    off2 = np.concatenate([[0], np.cumsum([rows[e] for e in perm])])
    sa2 = SA.reshape(-1, G)[ridx].reshape(-1)
    got = grouped_gemm_f64(A[ridx], sa2, 0, B[perm], SB[perm], off2)
    assert np.array_equal(got, full[ridx])


def test_empty_experts_weights_unused():
    rng = np.random.default_rng(31)
    A, SA, B, SB, off = random_case(rng, E=4, N=8, K=128, rows_per_expert=[0, 4, 0, 2])
    base = grouped_gemm_f64(A, SA, 0, B, SB, off)
    B2, SB2 = B.copy(), SB.copy()
    B2[[0, 2]] = 0x77
    SB2[[0, 2]] = 255  # NaN scales on experts with no rows
    assert np.array_equal(grouped_gemm_f64(A, SA, 0, B2, SB2, off), base)
    z = grouped_gemm_f64(A[:0], SA[:0], 0, B, SB, np.zeros(5, dtype=np.int32))
    assert z.shape == (0, 8)


def test_rows_gemm_matches_grouped():
    rng = np.random.default_rng(41)
    A, SA, B, SB, off = random_case(rng, E=3, N=40, K=256, rows_per_expert=[4, 5, 3])
    full = grouped_gemm_f64(A, SA, 0, B, SB, off)
    rows = np.array([0, 3, 4, 8, 11])
    ex = np.searchsorted(off, rows, side="right") - 1
    cols = np.array([1, 7, 39])
    got = og.rows_gemm_f64(A[rows], SA.reshape(-1, 2)[rows], ex, B, SB, cols)
    # same exact products; only the fp64 summation order inside BLAS differs
    np.testing.assert_allclose(got, full[rows][:, cols], rtol=1e-12, atol=0)


def test_bad_offsets_rejected():
    rng = np.random.default_rng(2)
    A, SA, B, SB, off = random_case(rng, E=2, N=4, K=128, rows_per_expert=[1, 2])
    with pytest.raises(ValueError):
        grouped_gemm_f64(A, SA, 0, B, SB, np.array([0, 2, 1]))
    with pytest.raises(ValueError):
        grouped_gemm_f64(A, SA, 0, B, SB, np.array([1, 2, 3]))


# --------------------------------------------------------------------------
# planted mistakes: each mutation of the oracle must break the brute-force pin
# --------------------------------------------------------------------------

def _swap_nibbles(b, sb, absolute=False):
    b = og._np(b).astype(np.uint8)
    n, kh = b.shape
    codes = np.empty((n, 2 * kh), dtype=np.intp)
    codes[:, 0::2] = b >> 4
    codes[:, 1::2] = b & 0x0F
    return og._LUT4[codes] * np.repeat(oracle.e8m0_value(og._np(sb)), 32, axis=1)


_ORIG_DECODE_WEIGHTS = og.decode_weights


def _sb_off_by_block(b, sb, absolute=False):
    w = _ORIG_DECODE_WEIGHTS(b, sb)
    sbv = np.roll(oracle.e8m0_value(og._np(sb)), 1, axis=1)
    return w / np.repeat(oracle.e8m0_value(og._np(sb)), 32, axis=1) * np.repeat(sbv, 32, axis=1)


def _drop_sa(a, s, absolute=False):
    return og._LUT8[og._np(a).astype(np.intp)]


def _sa_wrong_row(a, s, absolute=False):
    a8 = og._LUT8[og._np(a).astype(np.intp)]
    s = np.roll(og._np(s).astype(np.float64), 1, axis=0)
    return a8 * np.repeat(s, 128, axis=1)


def _sign_loss(b, sb, absolute=False):
    return np.abs(_ORIG_DECODE_WEIGHTS(b, sb))


@pytest.mark.parametrize("target,mutant", [
    ("decode_weights", _swap_nibbles),
    ("decode_weights", _sb_off_by_block),
    ("decode_weights", _sign_loss),
    ("decode_activations", _drop_sa),
    ("decode_activations", _sa_wrong_row),
])
def test_planted_mistakes_are_caught(monkeypatch, target, mutant):
    rng = np.random.default_rng(77)
    A, SA, B, SB, off = random_case(rng, E=2, N=4, K=256, rows_per_expert=[2, 1])
    want = brute_force_bits(A, SA, 0, B, SB, off)
    assert np.array_equal(grouped_gemm_bf16(A, SA, 0, B, SB, off), want)
    monkeypatch.setattr(og, target, mutant)
    got = bf16_rne_bits(og.grouped_gemm_f64(A, SA, 0, B, SB, off))
    assert not np.array_equal(got, want)


def test_planted_transpose_is_caught():
    rng = np.random.default_rng(78)
    A, SA, B, SB, off = random_case(rng, E=1, N=3, K=128, rows_per_expert=[3])
    want = brute_force_bits(A, SA, 0, B, SB, off)
    wd = og.decode_weights(B[0], SB[0])
    ad = og.decode_activations(A, SA.reshape(3, 1))
    wrong = bf16_rne_bits((ad @ wd.T).T)    # transposed result, same shape here
    assert not np.array_equal(wrong, want)


def test_absolute_sum_bruteforce_and_invariants():
    """absolute=True gives sum_k |a_k w_k| (the scale of any evaluation's
    rounding error): equal to an exact rational sum of magnitudes on a tiny
    case, >= |C| everywhere, equal to C when every product is nonnegative,
    unchanged by flipping the sign of the weights."""
    rng = np.random.default_rng(43)
    A, SA, B, SB, off = random_case(rng, E=2, N=5, K=256, rows_per_expert=[2, 3])
    got = grouped_gemm_f64(A, SA, 0, B, SB, off, absolute=True)
    G = 2
    for e in range(2):
        for r in range(int(off[e]), int(off[e + 1])):
            for n in range(5):
                acc = Fraction(0)
                for k in range(256):
                    byte = int(B[e, n, k // 2])
                    w = _dec4((byte >> (4 * (k % 2))) & 0xF)
                    acc += abs(Fraction(_DEC8[A[r, k]]) * Fraction(float(SA[r * G + k // 128])) * Fraction(w)
                               * Fraction(2) ** (int(SB[e, n, k // 32]) - 127))
                assert abs(Fraction(got[r, n]) - acc) <= acc * Fraction(1, 2 ** 50)
    C = grouped_gemm_f64(A, SA, 0, B, SB, off)
    assert np.all(got >= np.abs(C) * (1 - 1e-15))
    assert np.array_equal(grouped_gemm_f64(A, SA, 0, B ^ 0x88, SB, off, absolute=True), got)
    Apos = A & 0x7F                                   # nonnegative activations
    Bpos = B & 0x77                                   # nonnegative weights
    Cp = grouped_gemm_f64(Apos, SA, 0, Bpos, SB, off)
    np.testing.assert_allclose(grouped_gemm_f64(Apos, SA, 0, Bpos, SB, off, absolute=True), Cp, rtol=1e-14)
    rows = np.array([0, 4])
    ex = np.array([0, 1])
    np.testing.assert_allclose(og.rows_gemm_f64(A[rows], SA.reshape(-1, 2)[rows], ex, B, SB, absolute=True),
                               got[rows], rtol=1e-12)
