"""SwiGLU of the gate/up projection's output and its FP8 requantization for
the down projection.  TEST INFRASTRUCTURE ONLY (see the package docstring).

What it computes: the step between the two benchmarked projections (humming
PR #129 and PR #58 time gate/up and down as a pair, "Results" / "H200
performance"): the gate/up output C [R][2I] bf16 holds the gate in columns
0 .. I-1 and the up projection in columns I .. 2I-1 (the concatenated
[w1; w3] layout), and

    h[r, i] = silu(C[r, i]) * C[r, I + i],    silu(g) = g / (1 + exp(-g)),

quantized per (row, 128) group exactly as oracle/quant.py does for tokens
(s = amax/448 in fp32, codes by round to nearest even of clip(h/s, +-448)).

Since a float decides the integer codes, both sides compute h with one
fixed fp32 sequence (IEEE single operations, no fused multiply-add):
    x = -g; clamp to [-88, 89] (at the top the scaling below overflows to
        inf, so silu is g / inf = -0; at the bottom e^x is far below 2^-24
        and 1 + e^x rounds to 1, whatever happens to its denormals)
    n = rint(x * log2(e)); r = (x - n * L_hi) - n * L_lo   (Cody and Waite's
        two-constant reduction, L_hi + L_lo = ln 2, L_hi with 12 significant
        bits so that n * L_hi is exact)
    p = Horner's rule for the Taylor polynomial of e^r to degree 7
    e = ldexp(p, n)          (exact scaling; inf above, 0 below the range)
    silu = g / (1 + e);  h = silu * up
The degree-7 Taylor remainder on |r| <= ln2/2 is below 2^-27 relative, so
the fp32 exp is within a couple of units in the last place of e^x.
"""

from __future__ import annotations

import numpy as np

from .quant import E4M3_MAX, bf16_bits_to_f32, e4m3_encode_rne

F = np.float32
LOG2E = F(1.4426950408889634)
L_HI = F(0.693359375)               # 12 significant bits: n * L_HI is exact for |n| < 2^12
L_LO = F(0.6931471805599453 - 0.693359375)
TAYLOR = [F(1.0 / np.prod(np.arange(1, k + 1, dtype=np.float64))) for k in range(8)]  # 1/k!, k = 0..7
X_MIN, X_MAX = F(-88.0), F(89.0)


def exp_f32(x: np.ndarray) -> np.ndarray:
    """e^x by the fixed fp32 sequence above (inputs float32)."""
    x = np.clip(np.asarray(x, dtype=F), X_MIN, X_MAX).astype(F)
    n = np.rint((x * LOG2E).astype(F)).astype(F)
    r = ((x - (n * L_HI).astype(F)).astype(F) - (n * L_LO).astype(F)).astype(F)
    p = np.full(x.shape, TAYLOR[7], dtype=F)
    for k in range(6, -1, -1):
        p = ((p * r).astype(F) + TAYLOR[k]).astype(F)
    with np.errstate(over="ignore", under="ignore"):
        return np.ldexp(p, n.astype(np.int32)).astype(F)


def swiglu_f32(g: np.ndarray, u: np.ndarray) -> np.ndarray:
    g = np.asarray(g, dtype=F)
    u = np.asarray(u, dtype=F)
    e = exp_f32(-g)
    with np.errstate(over="ignore"):
        d = (F(1.0) + e).astype(F)
        silu = (g / d).astype(F)
    return (silu * u).astype(F)


def swiglu_quant(C_bits: np.ndarray, layout: int):
    """C bf16 bits [R][2I] -> (codes uint8 [R][I], scales float32 flat in
    `layout`: row-major [R][I/128] or M-major [I/128][R])."""
    C = bf16_bits_to_f32(C_bits)
    R, N2 = C.shape
    I = N2 // 2
    if N2 % 2 or I % 128:
        raise ValueError("C must be [R][2I] with I a multiple of 128")
    h = swiglu_f32(C[:, :I], C[:, I:])
    G = I // 128
    hg = h.reshape(R, G, 128)
    amax = np.max(np.abs(hg), axis=2)
    s = np.where(amax > 0, amax / F(E4M3_MAX), F(1.0)).astype(F)
    v = np.clip((hg / s[:, :, None]).astype(F), F(-E4M3_MAX), F(E4M3_MAX))
    codes = e4m3_encode_rne(v).reshape(R, I)
    SA = s.reshape(-1) if layout == 0 else s.T.copy().reshape(-1)
    return codes, SA.astype(F)
