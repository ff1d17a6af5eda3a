"""fp64 grouped-contiguous W4A8 GEMM (the plain definition, one expert at a time).

Data layout (the pages fix dtypes, group sizes and the two input-scale
layouts -- humming PR #129, benchmark command and commit 2 "both layouts";
the byte layouts below are the plainest reading and are shared with the
library's documented interface):

  A   uint8 [R, K]          E4M3 codes, rows grouped contiguously by expert:
                            rows offsets[e] .. offsets[e+1]-1 belong to expert e.
  SA  fp32                  one scale per (row, 128-K group);
                            layout 0 (row-major): SA[r, g]   at r*(K/128) + g
                            layout 1 (M-major):   SA[g, r]   at g*R + r,
                            R = offsets[E].
  B   uint8 [E, N, K/2]     E2M1 codes, two per byte along K; element 2j in the
                            low nibble, 2j+1 in the high nibble.
  SB  uint8 [E, N, K/32]    E8M0 code per (expert, column, 32-K block).
  C   bf16  [R, N]          row-major.

Each product dec8 * SA * dec4 * 2^(SB-127) is exact in fp64 (at most
4 x 2 significant bits times a 24-bit fp32 scale times a power of two), so
only the fp64 summation inside BLAS rounds (about 1e-16 relative); the bf16
result is then one RNE step from that fp64 value.  Test infrastructure only.
"""

from __future__ import annotations

import numpy as np

from .formats import bf16_rne_bits, e2m1_table, e4m3_table, e8m0_value

_LUT8 = e4m3_table()
_LUT4 = e2m1_table()


def _np(x):
    """Accept numpy arrays or anything with a .numpy() (CPU torch tensors)."""
    if hasattr(x, "detach"):
        x = x.detach().cpu().numpy()
    return np.asarray(x)


def decode_activations(a_codes, sa_rows, absolute: bool = False) -> np.ndarray:
    """E4M3 codes [r, K] and fp32 scales [r, K/128] -> fp64 [r, K] (their
    magnitudes with absolute=True)."""
    a = _LUT8[_np(a_codes).astype(np.intp)]
    s = _np(sa_rows).astype(np.float64)
    out = a * np.repeat(s, 128, axis=1)
    return np.abs(out) if absolute else out


def decode_weights(b_packed, sb, absolute: bool = False) -> np.ndarray:
    """Packed E2M1 [N, K/2] and E8M0 [N, K/32] -> fp64 [N, K] (their
    magnitudes with absolute=True)."""
    b = _np(b_packed).astype(np.uint8)
    n, kh = b.shape
    codes = np.empty((n, 2 * kh), dtype=np.intp)
    codes[:, 0::2] = b & 0x0F          # even k: low nibble
    codes[:, 1::2] = b >> 4            # odd k: high nibble
    w = _LUT4[codes] * np.repeat(e8m0_value(_np(sb)), 32, axis=1)
    return np.abs(w) if absolute else w


def sa_rows(sa, layout: int, rows: np.ndarray, R: int, K: int) -> np.ndarray:
    """Gather the [len(rows), K/128] scales of the given rows from either layout."""
    G = K // 128
    sa = _np(sa).astype(np.float32).reshape(-1)
    rows = np.asarray(rows, dtype=np.int64)
    if layout == 0:
        return sa.reshape(R, G)[rows]
    if layout == 1:
        return sa.reshape(G, R)[:, rows].T
    raise ValueError("layout must be 0 (row-major) or 1 (M-major)")


def expert_gemm_f64(a_codes, sa_r, b_packed, sb) -> np.ndarray:
    """Dense C = decode(A) @ decode(B)^T for one expert, fp64 [r, N]."""
    return decode_activations(a_codes, sa_r) @ decode_weights(b_packed, sb).T


def grouped_gemm_f64(A, SA, layout, B, SB, offsets, chunk_rows: int = 8192, absolute: bool = False) -> np.ndarray:
    """Exact-product fp64 grouped GEMM, [R, N].  With absolute=True, the sum
    of the magnitudes of the same products, sum_k |a_k w_k| per output: the
    scale of the rounding error of any evaluation of the sum."""
    A = _np(A)
    B = _np(B)
    SB = _np(SB)
    off = _np(offsets).astype(np.int64)
    E = B.shape[0]
    N = B.shape[1]
    K = A.shape[1]
    R = int(off[E])
    if off[0] != 0 or np.any(np.diff(off) < 0):
        raise ValueError("offsets must start at 0 and be nondecreasing")
    if A.shape[0] != R:
        raise ValueError("A must have offsets[E] rows")
    out = np.zeros((R, N), dtype=np.float64)
    for e in range(E):
        lo, hi = int(off[e]), int(off[e + 1])
        if hi == lo:
            continue
        wd = decode_weights(B[e], SB[e], absolute)
        for c0 in range(lo, hi, chunk_rows):
            c1 = min(hi, c0 + chunk_rows)
            rows = np.arange(c0, c1)
            ad = decode_activations(A[c0:c1], sa_rows(SA, layout, rows, R, K), absolute)
            out[c0:c1] = ad @ wd.T
    return out


def grouped_gemm_bf16(A, SA, layout, B, SB, offsets) -> np.ndarray:
    """The reference output: uint16 bf16 bit patterns [R, N]."""
    return bf16_rne_bits(grouped_gemm_f64(A, SA, layout, B, SB, offsets))


def rows_gemm_f64(a_rows, sa_r, expert_of_row, B, SB, cols=None, absolute: bool = False) -> np.ndarray:
    """fp64 outputs for a sample of rows (each with its own expert), [r, len(cols)].

    ``a_rows``  E4M3 codes of the sampled rows [r, K]
    ``sa_r``    their scales [r, K/128]
    ``expert_of_row`` the expert each sampled row belongs to
    ``cols``    optional subset of output columns (default: all N)
    ``absolute`` sum the magnitudes of the products instead
    """
    a_rows = _np(a_rows)
    sa_r = _np(sa_r)
    ex = np.asarray(expert_of_row, dtype=np.int64)
    N = B.shape[1]
    cols = np.arange(N) if cols is None else np.asarray(cols, dtype=np.int64)
    out = np.empty((len(ex), len(cols)), dtype=np.float64)
    for e in np.unique(ex):
        sel = np.nonzero(ex == e)[0]
        wd = decode_weights(_np(B[int(e)])[cols], _np(SB[int(e)])[cols], absolute)
        out[sel] = decode_activations(a_rows[sel], sa_r[sel], absolute) @ wd.T
    return out
