"""SwiGLU of the gate/up projection's output and its FP8 requantization for
the down projection.  TEST INFRASTRUCTURE ONLY (see the package docstring).

What it computes: the step between the two benchmarked projections (humming
PR #129 and PR #58 time gate/up and down as a pair, "Results" / "H200
performance"): the gate/up output C [R][2I] bf16 holds the gate in columns
0 .. I-1 and the up projection in columns I .. 2I-1 (the concatenated
[w1; w3] layout), and

    h[r, i] = silu(C[r, i]) * C[r, I + i],    silu(g) = g / (1 + exp(-g)),

quantized per (row, 128) group as oracle/quant.py does for tokens: the
scale s = amax|h| / 448 (1 for an all-zero group), the code the E4M3FN
round-to-nearest-even of clip(h / s, +-448).

The oracle is that definition in fp64 with the library exp (`swiglu_f64`,
`swiglu_quant_f64`).  A GPU computes h in fp32, so near an E4M3 rounding
midpoint, and in the last bits of the scale, more than one result is
correct.  `check_swiglu_quant` therefore accepts a GPU result exactly when
it is what the definition gives for values within a stated distance of the
fp64 ones:

  * h' is admissible for an element when |h' - h| <= H_REL * |h| +
    H_ABS * |u|.  H_REL = 2^-20 (8 fp32 units in the last place) covers an
    fp32 evaluation of silu(g) * u with an exp and a reciprocal accurate to
    about an ulp each; H_ABS = 2^-118 covers the range where e^-g
    overflows fp32 (g below about -88.7, where silu(g) rounds to -0 although
    its magnitude is below 2^-120, or where the reciprocal of 1 + e^-g is
    subnormal).
  * the scale s' of a group is admissible when |s' - amax/448| <=
    max(slack)/448 + 2^-23 * amax/448, the slack of an element being the
    bound on |h' - h| above (amax of admissible h' can differ from the fp64
    amax by no more than the largest slack; the division by 448 rounds), or
    when s' = 1 and every h of the group is within its slack of zero.
  * a code is admissible when its value is the E4M3 round-to-nearest-even of
    clip(v, +-448) for some v with |v - h/s'| <= (H_REL * |h| + H_ABS * |u|)
    / s' + Q_REL * |h/s'| (the quotient by s' itself rounded in fp32).
    Rounding is monotone, so the admissible values form one interval,
    [rne(lo), rne(hi)]; the code's value must lie in it (+0 and -0 are the
    same value).
"""

from __future__ import annotations

import numpy as np

from .formats import e4m3_table
from .quant import E4M3_MAX, bf16_bits_to_f32, e4m3_encode_rne

H_REL = 2.0 ** -20
H_ABS = 2.0 ** -118
Q_REL = 2.0 ** -21


def silu_f64(g: np.ndarray) -> np.ndarray:
    """silu(g) = g / (1 + e^-g) in fp64 (for g below about -709 e^-g is inf
    and the quotient -0, whose true magnitude is below 2^-1000)."""
    g = np.asarray(g, dtype=np.float64)
    with np.errstate(over="ignore"):
        return g / (1.0 + np.exp(-g))


def swiglu_f64(g: np.ndarray, u: np.ndarray) -> np.ndarray:
    """h = silu(g) * u in fp64."""
    return silu_f64(g) * np.asarray(u, dtype=np.float64)


def _split(C_bits: np.ndarray):
    C = bf16_bits_to_f32(C_bits).astype(np.float64)
    R, N2 = C.shape
    I = N2 // 2
    if N2 % 2 or I % 128:
        raise ValueError("C must be [R][2I] with I a multiple of 128")
    return C[:, :I], C[:, I:], R, I


def swiglu_quant_f64(C_bits: np.ndarray, layout: int):
    """C bf16 bits [R][2I] -> (codes uint8 [R][I], scales float64 flat in
    `layout`: row-major [R][I/128] or M-major [I/128][R]), the definition
    evaluated in fp64: s = amax/448 (1 if amax = 0), code = RNE(clip(h/s))."""
    g, u, R, I = _split(C_bits)
    return h_quant_f64(g, u, layout)


def h_quant_f64(g: np.ndarray, u: np.ndarray, layout: int):
    """The same from fp64 gate and up values g, u [R][I] (the fused GEMM's
    definition: the exact GEMM outputs, not rounded to bf16)."""
    R, I = g.shape
    h = swiglu_f64(g, u)
    G = I // 128
    hg = h.reshape(R, G, 128)
    amax = np.max(np.abs(hg), axis=2)
    s = np.where(amax > 0, amax / E4M3_MAX, 1.0)
    v = np.clip(hg / s[:, :, None], -E4M3_MAX, E4M3_MAX)
    codes = e4m3_encode_rne(v).reshape(R, I)
    SA = s.reshape(-1) if layout == 0 else s.T.copy().reshape(-1)
    return codes, SA


def check_swiglu_quant(C_bits: np.ndarray, codes: np.ndarray, scales: np.ndarray, layout: int) -> dict:
    """Admissibility of a result (codes uint8 [R][I], fp32 scales flat in
    `layout`) of the SwiGLU step applied to the bf16 gate/up output C_bits,
    against the fp64 definition, with the bounds of the module docstring."""
    g, u, R, I = _split(C_bits)
    return check_h_quant(g, u, codes, scales, layout)


def check_h_quant(g: np.ndarray, u: np.ndarray, codes: np.ndarray, scales: np.ndarray, layout: int,
                  g_slack: np.ndarray | None = None, u_slack: np.ndarray | None = None) -> dict:
    """Admissibility of E4M3 codes and fp32 scales of h = silu(g) * u for
    fp64 gate and up values g, u [R][I].  g_slack / u_slack (same shape, or
    None for 0) widen the check for inputs that are themselves computed with
    a bounded error (the fused GEMM's fp32 accumulators): any g' within
    g_slack of g and u' within u_slack of u may have been used, and since
    |silu'| <= 1.1 everywhere, |silu(g') u' - silu(g) u| <= 1.1 g_slack
    (|u| + u_slack) + |silu(g)| u_slack is added to each element's slack.
    Returns counts: bad_scales, bad_codes, nan (codes or scales that are
    NaN), ambiguous (elements for which more than one code value is
    admissible), elements, and max_scale_rel (the largest relative distance
    of an accepted scale from amax/448, over groups not within the floor of
    zero)."""
    g = np.asarray(g, dtype=np.float64)
    u = np.asarray(u, dtype=np.float64)
    R, I = g.shape
    G = I // 128
    codes = np.asarray(codes, dtype=np.uint8).reshape(R, I)
    s_in = np.asarray(scales, dtype=np.float32).reshape(-1).astype(np.float64)
    if s_in.size != R * G:
        raise ValueError("scales must hold R * I/128 values")
    sg = s_in.reshape(R, G) if layout == 0 else s_in.reshape(G, R).T
    sil = silu_f64(g)
    h = sil * u
    au = np.abs(u)
    slack = H_REL * np.abs(h) + H_ABS * au                     # per element
    if g_slack is not None or u_slack is not None:
        gs = np.zeros_like(g) if g_slack is None else np.asarray(g_slack, dtype=np.float64)
        us = np.zeros_like(u) if u_slack is None else np.asarray(u_slack, dtype=np.float64)
        slack = slack + 1.1 * gs * (au + us) + np.abs(sil) * us
    hg = np.abs(h).reshape(R, G, 128)
    amax = hg.max(axis=2)
    ref = amax / E4M3_MAX
    sl_g = slack.reshape(R, G, 128)
    tiny = np.all(hg <= sl_g, axis=2)                          # the group may read as all zero
    nan_s = ~np.isfinite(sg) | (sg <= 0)
    ok_s = (np.abs(sg - ref) <= sl_g.max(axis=2) / E4M3_MAX + 2.0 ** -23 * ref) | (tiny & (sg == 1.0))
    ok_s &= ~nan_s
    sgf = np.where(nan_s, 1.0, sg)
    s_el = np.repeat(sgf, 128, axis=1)
    c = h / s_el
    rad = slack / s_el + Q_REL * np.abs(c)
    lo = np.clip(c - rad, -E4M3_MAX, E4M3_MAX)
    hi = np.clip(c + rad, -E4M3_MAX, E4M3_MAX)
    lut = e4m3_table()
    vlo = lut[e4m3_encode_rne(lo)]
    vhi = lut[e4m3_encode_rne(hi)]
    nan_c = (codes & 0x7F) == 0x7F
    val = lut[np.where(nan_c, 0, codes)]
    ok_c = (val >= vlo) & (val <= vhi) & ~nan_c
    rel = np.where(ok_s & ~tiny, np.abs(sg - ref) / np.where(ref > 0, ref, 1.0), 0.0)
    return {"bad_scales": int((~ok_s).sum()), "bad_codes": int((~ok_c).sum()),
            "nan": int(nan_c.sum() + nan_s.sum()), "ambiguous": int((vlo != vhi).sum()),
            "elements": int(R * I), "max_scale_rel": float(rel.max()) if rel.size else 0.0}
