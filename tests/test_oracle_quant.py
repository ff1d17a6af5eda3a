"""Pins for the oracle's activation quantizer (oracle/quant.py).

Independent sources: round trips through the oracle's own E4M3 decode table
(itself pinned against torch's float8_e4m3fn dtype), the tie rule of round-
to-nearest-even checked at every midpoint between neighbouring codes,
torch's float8_e4m3fn cast (a separate implementation) on random values
across the whole range, the torch-based quantizer of the synthetic-input
module on bf16-representable data, and closed forms of the amax/448 scale.
"""

import numpy as np
import torch

from oracle import e4m3_encode_rne, e4m3_table, quantize_gather, quantize_tokens
from synth.generate import quantize_fp8_rows


def _finite_codes():
    t = e4m3_table()
    return [c for c in range(256) if not np.isnan(t[c])], t


def test_encode_round_trips_every_finite_code():
    codes, t = _finite_codes()
    v = np.array([t[c] for c in codes], dtype=np.float32)
    assert np.array_equal(e4m3_encode_rne(v), np.array(codes, dtype=np.uint8))


def test_encode_midpoints_round_to_even_code():
    _, t = _finite_codes()
    for c in range(0x7E):                      # neighbours c, c+1 among the positive codes
        lo, hi = t[c], t[c + 1]
        mid = np.float32((lo + hi) / 2)         # exact: at most 5 significant bits
        assert float(mid) == (lo + hi) / 2
        even = c if c % 2 == 0 else c + 1
        got = e4m3_encode_rne(np.array([mid, -mid], dtype=np.float32))
        assert got[0] == even and got[1] == (even | 0x80), (c, lo, hi)
        below = np.nextafter(mid, np.float32(0))
        above = np.nextafter(mid, np.float32(np.inf))
        assert e4m3_encode_rne(np.array([below], dtype=np.float32))[0] == c
        assert e4m3_encode_rne(np.array([above], dtype=np.float32))[0] == c + 1


def test_encode_matches_torch_cast():
    rng = np.random.default_rng(11)
    mag = np.exp2(rng.uniform(-14, np.log2(448.0), size=400_000)).astype(np.float32)
    mag = np.minimum(mag, np.float32(448.0))
    v = (mag * rng.choice([-1.0, 1.0], size=mag.size)).astype(np.float32)
    v[:8] = [0.0, -0.0, 448.0, -448.0, 2.0 ** -9, 2.0 ** -10, 3 * 2.0 ** -11, 2.0 ** -6]
    ref = torch.from_numpy(v).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(e4m3_encode_rne(v), ref)


def _bf16_bits(x: np.ndarray) -> np.ndarray:
    """float32 -> bf16 bits by truncation (the test only needs bf16 values)."""
    return (np.asarray(x, dtype=np.float32).view(np.uint32) >> 16).astype(np.uint16)


def test_quantize_tokens_matches_synth_quantizer():
    rng = np.random.default_rng(12)
    x = rng.standard_normal((37, 512)).astype(np.float32)
    x[3, 128:256] = 0.0                                 # all-zero group: scale 1
    x[5, :128] *= np.float32(2.0 ** -20)                # codes in the subnormal range
    bits = _bf16_bits(x)
    xb = (bits.astype(np.uint32) << 16).view(np.float32)
    codes, s = quantize_tokens(bits)
    ref_codes, ref_s = quantize_fp8_rows(torch.from_numpy(xb.copy()))
    assert np.array_equal(s, ref_s.numpy())
    assert np.array_equal(codes, ref_codes.numpy())
    assert s[3, 1] == 1.0 and not codes[3, 128:256].any()


def test_scale_closed_forms():
    x = np.zeros((2, 256), np.float32)
    x[0, :128] = np.linspace(-3.5, 7.0, 128, dtype=np.float32)
    x[0, 128:] = np.float32(448.0 * 2.0 ** -5)          # amax = 448 * 2^-5: scale exactly 2^-5
    x[1, :128] = -np.float32(2.0)                       # negative amax
    codes, s = quantize_tokens(_bf16_bits(x))
    assert s[0, 1] == np.float32(2.0 ** -5) and np.all(codes[0, 128:] == 0x7E)
    assert s[1, 0] == np.float32(2.0 / 448.0) and np.all(codes[1, :128] == 0xFE)
    assert s[1, 1] == 1.0 and np.all(codes[1, 128:] == 0)
    # the amax element of every group is +-448 after scaling and rounding
    assert codes[0, 127] == 0x7E


def test_gather_rows_layouts_and_skipped_slots():
    rng = np.random.default_rng(13)
    T, K, k = 9, 384, 3
    bits = _bf16_bits(rng.standard_normal((T, K)).astype(np.float32))
    R = T * k - 2
    perm = rng.permutation(T * k)
    ros = np.where(perm < R, perm, -1).astype(np.int32)  # two slots name no row
    codes, s = quantize_tokens(bits)
    A0, S0 = quantize_gather(bits, ros, k, R, 0)
    A1, S1 = quantize_gather(bits, ros, k, R, 1)
    G = K // 128
    assert np.array_equal(A0, A1)
    assert np.array_equal(S0.reshape(R, G), S1.reshape(G, R).T)
    for slot, r in enumerate(ros):
        if r >= 0:
            assert np.array_equal(A0[r], codes[slot // k])
            assert np.array_equal(S0.reshape(R, G)[r], s[slot // k])
    # rows that no slot names keep their initial contents
    init = np.full((R + 1, K), 0x5A, np.uint8)
    A2, _ = quantize_gather(bits, ros, k, R + 1, 0, A_init=init)
    assert np.all(A2[R] == 0x5A)
