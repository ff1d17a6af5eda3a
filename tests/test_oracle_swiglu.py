"""Pins for the oracle's SwiGLU + requantization (oracle/swiglu.py).

Independent sources: numpy's fp64 exp and the fp64 SwiGLU (the fixed fp32
sequence must stay within a few units in the last place of them), closed
forms (exp(0) = 1, silu(0) = 0, overflow and underflow ends), the E4M3
rounding bound of the dequantized codes against the fp64 SwiGLU, and the
transposition between the two scale layouts.
"""

import numpy as np

from oracle import e4m3_table, exp_f32, swiglu_f32, swiglu_quant


def _ulps(got, ref):
    ref32 = ref.astype(np.float32)
    return np.abs(got.astype(np.float64) - ref) / np.spacing(np.abs(ref32)).astype(np.float64)


def test_exp_within_two_ulp_of_fp64():
    x = np.linspace(-87.0, 88.7, 1_000_001, dtype=np.float32)
    assert _ulps(exp_f32(x), np.exp(x.astype(np.float64))).max() <= 2.0


def test_exp_closed_forms_and_ends():
    e = exp_f32(np.array([0.0, np.log(2.0) * 10, 89.0, 1e30, -88.0, -1e30], dtype=np.float32))
    assert e[0] == 1.0
    assert abs(float(e[1]) - 1024.0) <= 1024.0 * 2 ** -22
    assert np.isinf(e[2]) and np.isinf(e[3])
    assert 0.0 <= e[4] < 2.0 ** -126 and e[5] == e[4]


def test_swiglu_within_a_few_ulp_of_fp64():
    rng = np.random.default_rng(4)
    g = (rng.standard_normal(200_000) * 4).astype(np.float32)
    u = rng.standard_normal(200_000).astype(np.float32)
    ref = g.astype(np.float64) / (1.0 + np.exp(-g.astype(np.float64))) * u.astype(np.float64)
    got = swiglu_f32(g, u)
    ok = np.abs(ref) > 1e-30
    assert _ulps(got[ok], ref[ok]).max() <= 4.0
    z = swiglu_f32(np.array([0.0, -100.0, 100.0], np.float32), np.array([5.0, 1.0, 2.0], np.float32))
    assert z[0] == 0.0 and z[1] == 0.0 and np.signbit(z[1]) and z[2] == 200.0


def _bf16_bits(x):
    return (np.asarray(x, dtype=np.float32).view(np.uint32) >> 16).astype(np.uint16)


def test_requantized_values_within_e4m3_rounding_of_fp64():
    rng = np.random.default_rng(5)
    R, I = 24, 384
    C = rng.standard_normal((R, 2 * I)).astype(np.float32) * 3
    C[0, :128] = 0.0                      # zero gate group: h = 0, scale 1
    bits = _bf16_bits(C)
    codes, SA = swiglu_quant(bits, 0)
    Cf = (bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    g, u = Cf[:, :I], Cf[:, I:]
    h = g / (1.0 + np.exp(-g)) * u
    s = SA.reshape(R, I // 128).astype(np.float64)
    deq = e4m3_table()[codes] * np.repeat(s, 128, axis=1)
    bound = np.abs(h) * 2.0 ** -4 + np.repeat(s, 128, axis=1) * 2.0 ** -10 + np.abs(h) * 1e-6
    assert np.all(np.abs(deq - h) <= bound)
    assert s[0, 0] == 1.0 and not (codes[0, :128] & 0x7F).any()   # +-0 (the sign of up)
    amax = np.abs(h).reshape(R, I // 128, 128).max(axis=2)
    assert np.allclose(s[amax > 0], amax[amax > 0] / 448.0, rtol=1e-6)


def test_layouts_are_transposes():
    rng = np.random.default_rng(6)
    bits = _bf16_bits(rng.standard_normal((10, 512)).astype(np.float32))
    c0, s0 = swiglu_quant(bits, 0)
    c1, s1 = swiglu_quant(bits, 1)
    assert np.array_equal(c0, c1)
    assert np.array_equal(s0.reshape(10, 2), s1.reshape(2, 10).T)
