"""Pins for the oracle's top-k combine (oracle/combine.py).

Independent sources: the identity with one slot and unit weight, exact
sums (small-integer rows, power-of-two weights) against an exact fp64 sum
rounded by torch's fp32 -> bf16 cast, and the same slot-ordered fp32
arithmetic written with torch tensors on the CPU, rounded by torch's cast.
"""

import numpy as np
import torch

from oracle import combine_ref


def _bf16(x):
    return torch.from_numpy(np.asarray(x, dtype=np.float32)).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def test_one_slot_unit_weight_is_identity():
    rng = np.random.default_rng(1)
    C = _bf16(rng.standard_normal((20, 64)))
    rows = rng.permutation(20).astype(np.int32)
    out = combine_ref(C, rows, np.ones(20, np.float32), 20, 1)
    assert np.array_equal(out, C[rows])


def test_exact_sums_match_exact_reference():
    rng = np.random.default_rng(2)
    T, k, N = 30, 8, 96
    R = T * k
    C = _bf16(rng.integers(-64, 65, size=(R, N)))
    w = np.exp2(rng.integers(-6, 2, size=T * k)).astype(np.float32)
    rows = rng.permutation(R).astype(np.int32)
    rows[5] = -1                                     # a skipped slot
    out = combine_ref(C, rows, w, T, k)
    Cf = (C.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    exact = np.zeros((T, N))
    for s in range(T * k):
        if rows[s] >= 0:
            exact[s // k] += w[s] * Cf[rows[s]]
    assert np.array_equal(out, _bf16(exact.astype(np.float32)))   # exact sums fit fp32


def test_matches_torch_slot_ordered_fp32():
    rng = np.random.default_rng(3)
    T, k, N, R = 50, 8, 128, 420
    C = _bf16(rng.standard_normal((R, N)))
    w = rng.random(T * k).astype(np.float32)
    rows = rng.integers(-1, R + 2, size=T * k).astype(np.int32)   # includes rows outside [0, R)
    out = combine_ref(C, rows, w, T, k)
    Ct = torch.from_numpy(C.view(np.int16)).view(torch.bfloat16).float()
    acc = torch.zeros((T, N), dtype=torch.float32)
    for t in range(T):
        for j in range(k):
            r = int(rows[t * k + j])
            if 0 <= r < R:
                acc[t] = acc[t] + torch.tensor(w[t * k + j]) * Ct[r]
    ref = acc.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(out, ref)


def test_no_valid_slot_gives_zero():
    C = _bf16(np.ones((4, 32)))
    out = combine_ref(C, np.full(6, -1, np.int32), np.ones(6, np.float32), 3, 2)
    assert not out.any()
