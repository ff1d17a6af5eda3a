"""fp64 grouped-contiguous GEMM with 16-bit activations and FP4 weights (A16).
TEST INFRASTRUCTURE ONLY (see the package docstring).

What it computes: the BF16-activation FP4 paths humming PR #58 tunes
("Summary": the small-M FP4 paths exercised by MXFP4/NVFP4 A16; "Validation":
exact MXFP4/NVFP4 kernel correctness coverage), on the grouped-contiguous
layout of the W4A8 path:

    C[r, n] = bf16_rne( gs[e] * sum_k bf16(A[r, k]) * e2m1(B[e, n, k]) * s(e, n, k) )

with e the expert of row r and the weight scale s from one of two formats:

  MXFP4 (fmt 0):  s = 2^(SB[e, n, k/32] - 127), an E8M0 code per 32 K
                  (OCP MX v1.0); gs = 1.
  NVFP4 (fmt 1):  s = e4m3(SB[e, n, k/16]), an E4M3FN code per 16 K, and one
                  fp32 scale gs[e] per expert (the per-tensor scale of the
                  format; each expert's weights are a tensor of their own).

Layouts: A bf16 bit patterns [R, K], rows grouped by expert as in gemm.py;
B uint8 [E, N, K/2] (E2M1 codes, element 2j in the low nibble); SB uint8
[E, N, K/32] (fmt 0) or [E, N, K/16] (fmt 1); gs fp32 [E]; C bf16 [R, N].

Every product bf16 * e2m1 * scale is exact in fp64 (8 + 2 + 4 significant
bits at most, exponents far inside fp64's range); the fp64 sum rounds once
per addition (about 1e-16 relative) and the result is rounded once to bf16
after the multiplication by gs (exact in fp64 too: 24 + 14 bits).
"""

from __future__ import annotations

import numpy as np

from .formats import bf16_bits_to_f64, bf16_rne_bits, e2m1_table, e4m3_table, e8m0_value

_LUT4 = e2m1_table()
_LUT8 = e4m3_table()

FMT_MX = 0
FMT_NV = 1


def _np(x):
    if hasattr(x, "detach"):
        x = x.detach().cpu().numpy()
    return np.asarray(x)


def block_of(fmt: int) -> int:
    """K elements per weight-scale code: 32 (MXFP4) or 16 (NVFP4)."""
    if fmt == FMT_MX:
        return 32
    if fmt == FMT_NV:
        return 16
    raise ValueError("fmt must be 0 (MXFP4, E8M0 per 32) or 1 (NVFP4, E4M3 per 16)")


def scale_values(sb, fmt: int) -> np.ndarray:
    """Weight-scale codes -> fp64 values (E8M0 2^(c-127) or E4M3FN)."""
    sb = _np(sb).astype(np.intp)
    if fmt == FMT_MX:
        return e8m0_value(sb)
    block_of(fmt)
    return _LUT8[sb]


def decode_weights_a16(b_packed, sb, fmt: int, absolute: bool = False) -> np.ndarray:
    """Packed E2M1 [N, K/2] and scale codes [N, K/blk] -> fp64 [N, K]
    (their magnitudes with absolute=True)."""
    b = _np(b_packed).astype(np.uint8)
    n, kh = b.shape
    codes = np.empty((n, 2 * kh), dtype=np.intp)
    codes[:, 0::2] = b & 0x0F
    codes[:, 1::2] = b >> 4
    w = _LUT4[codes] * np.repeat(scale_values(sb, fmt), block_of(fmt), axis=1)
    return np.abs(w) if absolute else w


def grouped_gemm_a16_f64(A_bits, B, SB, fmt: int, gs, offsets, absolute: bool = False) -> np.ndarray:
    """fp64 [R, N]: the definition above.  With absolute=True, the sum of the
    magnitudes of the products times |gs|, sum_k |a_k w_k| |gs|: the scale of
    the rounding error of any evaluation of the sum.  gs may be None (all
    ones)."""
    A = bf16_bits_to_f64(_np(A_bits).astype(np.uint16))
    B = _np(B)
    SB = _np(SB)
    off = _np(offsets).astype(np.int64)
    E, N = B.shape[0], B.shape[1]
    R = int(off[E])
    if off[0] != 0 or np.any(np.diff(off) < 0):
        raise ValueError("offsets must start at 0 and be nondecreasing")
    if A.shape[0] != R:
        raise ValueError("A must have offsets[E] rows")
    g = np.ones(E) if gs is None else _np(gs).astype(np.float32).astype(np.float64).reshape(E)
    out = np.zeros((R, N), dtype=np.float64)
    for e in range(E):
        lo, hi = int(off[e]), int(off[e + 1])
        if hi == lo:
            continue
        a = np.abs(A[lo:hi]) if absolute else A[lo:hi]
        w = decode_weights_a16(B[e], SB[e], fmt, absolute)
        out[lo:hi] = (a @ w.T) * (abs(g[e]) if absolute else g[e])
    return out


def grouped_gemm_a16_bf16(A_bits, B, SB, fmt: int, gs, offsets) -> np.ndarray:
    """The reference output: uint16 bf16 bit patterns [R, N]."""
    return bf16_rne_bits(grouped_gemm_a16_f64(A_bits, B, SB, fmt, gs, offsets))
