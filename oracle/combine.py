"""Top-k weighted combine of grouped output rows back to tokens.  TEST
INFRASTRUCTURE ONLY (see the package docstring).

What it computes: the step after the grouped expert GEMM, the single-GPU
half of an expert-parallel combine (the routing this inverts is the MoE
planning of MoonEP PR #38, background section): every token sums the rows of
its top-k slots, each weighted by the slot's router weight,

    out[t, :] = bf16_rne( sum_{j = 0 .. top_k-1} w[t, j] * C[row_of_slot[t*top_k + j], :] )

Plain reading, the same on both sides: the sum runs in fp32 in slot order j
= 0, 1, ..., each term one fp32 product and one fp32 addition (no fused
multiply-add), starting from 0; slots whose row is outside [0, R) contribute
nothing; one rounding of the fp32 sum to bf16 at the end.  With the order and
the operations fixed the result is unique, so parity is bit for bit.
"""

from __future__ import annotations

import numpy as np

from .formats import bf16_rne_bits


def combine_ref(C_bits: np.ndarray, row_of_slot: np.ndarray, weights: np.ndarray, T: int, top_k: int) -> np.ndarray:
    """C bf16 bits [R][N] (uint16), row_of_slot int32 [T*top_k], weights fp32
    [T*top_k] -> out bf16 bits [T][N] (uint16)."""
    C_bits = np.asarray(C_bits, dtype=np.uint16)
    R, N = C_bits.shape
    C = (C_bits.astype(np.uint32) << np.uint32(16)).view(np.float32)
    rows = np.asarray(row_of_slot, dtype=np.int64).reshape(T, top_k)
    w = np.asarray(weights, dtype=np.float32).reshape(T, top_k)
    acc = np.zeros((T, N), dtype=np.float32)
    for j in range(top_k):
        r = rows[:, j]
        ok = (r >= 0) & (r < R)
        term = (w[ok, j][:, None] * C[r[ok]]).astype(np.float32)     # one fp32 product
        acc[ok] = (acc[ok] + term).astype(np.float32)                 # one fp32 addition
    return bf16_rne_bits(acc.astype(np.float64)).reshape(T, N)
