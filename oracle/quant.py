"""Activation quantization with the gather into grouped rows: bf16 tokens ->
FP8 E4M3 codes with one fp32 scale per (row, 128-K group), written to the
grouped row of every (token, slot).  TEST INFRASTRUCTURE ONLY (see the
package docstring).

What it computes.  The benchmark's activation recipe (humming PR #129,
"Results" command: float8e4m3 activations, input-scale group size 128) gives
each (row, 128-K group) its own fp32 scale; the amax/448 scale and the E4M3
codes follow the OCP 8-bit floating point definition of E4M3FN (largest
finite value 448).  Plain reading, the same on both sides:

    amax(t, g) = max |x[t, 128g .. 128g+127]|            (exact in fp32)
    s(t, g)    = fl32(amax / 448), or 1 when amax == 0
    v          = clip(fl32(x / s), -448, 448)             (IEEE fp32 division)
    code       = E4M3FN round-to-nearest-even of v, sign kept (-0 -> 0x80)

and for every slot (t, j) with r = row_of_slot[t * top_k + j] >= 0:
A[r, :] = codes of token t, SA(r, g) = s(t, g), in the row-major
[R][K/128] or M-major [K/128][R] layout.  Rows that no slot names are left
as they were.  NaN or infinite inputs are outside the definition.

The encoder works from the format definition in fp64 on exact fp32 values:
below 2^-6 the quantum is 2^-9 (subnormals, up to the smallest normal);
above, a value in [2^E, 2^(E+1)) has quantum 2^(E-3).  numpy's rint rounds
halves to even.
"""

from __future__ import annotations

import numpy as np

E4M3_MAX = 448.0


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    """bf16 bit patterns (uint16) -> float32, exactly (the top half of binary32)."""
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def e4m3_encode_rne(v: np.ndarray) -> np.ndarray:
    """float32 or float64 values with |v| <= 448 -> E4M3FN codes, round to
    nearest even (other dtypes are taken as float32)."""
    v = np.asarray(v)
    if v.dtype != np.float64:
        v = v.astype(np.float32)
    if np.any(~np.isfinite(v)) or np.any(np.abs(v) > E4M3_MAX):
        raise ValueError("E4M3 encoding needs finite values with |v| <= 448")
    a = np.abs(v.astype(np.float64))
    sign = np.signbit(v).astype(np.uint8) << 7
    code = np.zeros(v.shape, dtype=np.int64)
    sub = a < 2.0 ** -6
    # subnormal range: multiples of 2^-9; 8 * 2^-9 is the smallest normal (code 8)
    code[sub] = np.rint(a[sub] / 2.0 ** -9).astype(np.int64)
    nrm = ~sub
    if np.any(nrm):
        _, p = np.frexp(a[nrm])          # a = m * 2^p, m in [0.5, 1)
        E = p.astype(np.int64) - 1       # a in [2^E, 2^(E+1))
        q = np.rint(np.ldexp(a[nrm], -(E - 3))).astype(np.int64)  # 8 .. 16
        up = q == 16
        E = np.where(up, E + 1, E)
        q = np.where(up, 8, q)
        code[nrm] = ((E + 7) << 3) | (q - 8)
    return (code.astype(np.uint8) | sign).astype(np.uint8)


def quantize_tokens(x_bits: np.ndarray):
    """bf16 tokens [T][K] (uint16 bits) -> (codes uint8 [T][K], scales float32 [T][K/128])."""
    x = bf16_bits_to_f32(x_bits)
    T, K = x.shape
    if K % 128:
        raise ValueError("K must be a multiple of 128")
    G = K // 128
    xg = x.reshape(T, G, 128)
    amax = np.max(np.abs(xg), axis=2)                           # float32, exact
    s = np.where(amax > 0, amax / np.float32(E4M3_MAX), np.float32(1.0)).astype(np.float32)
    v = (xg / s[:, :, None]).astype(np.float32)                 # IEEE fp32 division
    v = np.clip(v, np.float32(-E4M3_MAX), np.float32(E4M3_MAX))
    codes = e4m3_encode_rne(v).reshape(T, K)
    return codes, s


def quantize_gather(x_bits: np.ndarray, row_of_slot: np.ndarray, top_k: int, R: int, layout: int,
                    A_init: np.ndarray | None = None, SA_init: np.ndarray | None = None):
    """Quantize every token and write its codes and scales to the row of each
    of its slots.  Returns (A uint8 [R][K], SA float32 flat in `layout`).
    A_init / SA_init give the contents of rows no slot names (zeros if None)."""
    codes, s = quantize_tokens(x_bits)
    T, K = codes.shape
    G = K // 128
    rows = np.asarray(row_of_slot, dtype=np.int64).reshape(T, top_k)
    A = np.zeros((R, K), np.uint8) if A_init is None else np.array(A_init, dtype=np.uint8).reshape(R, K)
    SA = np.zeros(R * G, np.float32) if SA_init is None else np.array(SA_init, dtype=np.float32).reshape(-1)
    for t in range(T):
        for j in range(top_k):
            r = int(rows[t, j])
            if r < 0:
                continue
            A[r] = codes[t]
            for g in range(G):
                SA[r * G + g if layout == 0 else g * R + r] = s[t, g]
    return A, SA
