"""Pins for the oracle's SwiGLU + requantization (oracle/swiglu.py).

Independent sources: textbook values of the logistic function (sigmoid(0) =
1/2, sigmoid(ln 3) = 3/4, sigmoid(1) = e/(1+e)), scipy's expit (its own
implementation of the logistic function), the large-|g| limits, closed forms
of the amax/448 quantization (constant groups, groups of exact E4M3
multiples of the scale), the E4M3 rounding bound of the dequantized codes,
and the transposition between the two scale layouts.  The admissibility
check is pinned both ways: it accepts the fp64 definition and an
independent fp32 evaluation, and it rejects planted mistakes (gate and up
swapped, the wrong sign in the exponential, a code one step off, a scale a
few units off, the layouts exchanged, NaN codes).
"""

import numpy as np
import pytest
from scipy.special import expit

from oracle import (check_h_quant, check_swiglu_quant, e4m3_table, h_quant_f64, silu_f64, swiglu_f64,
                    swiglu_quant_f64)
from oracle.quant import e4m3_encode_rne


def _bf16_bits(x):
    """float32 -> bf16 bits by truncation (tests pick bf16-exact values or
    do not care about the rounding of the input)."""
    return (np.asarray(x, dtype=np.float32).view(np.uint32) >> 16).astype(np.uint16)


def _f(bits):
    return (np.asarray(bits, np.uint16).astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def test_silu_textbook_values():
    assert silu_f64(np.array([0.0]))[0] == 0.0
    ln3 = np.log(3.0)
    assert abs(silu_f64(np.array([ln3]))[0] - 0.75 * ln3) <= 1e-15 * ln3
    assert abs(silu_f64(np.array([-ln3]))[0] + 0.25 * ln3) <= 1e-15 * ln3
    assert abs(silu_f64(np.array([1.0]))[0] - np.e / (1 + np.e)) <= 1e-15
    eps = 2.0 ** -30
    assert abs(silu_f64(np.array([eps]))[0] / eps - 0.5) <= 1e-9     # slope 1/2 at 0
    big = silu_f64(np.array([60.0, -60.0, -800.0]))
    assert big[0] == 60.0 and 0 > big[1] > -60.0 * 1e-25 and big[2] == 0.0


def test_silu_against_scipy_expit():
    x = np.linspace(-80.0, 80.0, 100_001)
    ref = x * expit(x)
    got = silu_f64(x)
    assert np.all(np.abs(got - ref) <= 1e-14 * np.maximum(np.abs(ref), 1e-300))


def test_swiglu_takes_gate_first():
    C = np.zeros((1, 256), np.float32)
    C[0, :128] = 1.09375
    C[0, 128:] = 2.0
    bits = _bf16_bits(C)
    g = _f(bits)[:, :128]
    h = swiglu_f64(g, _f(bits)[:, 128:])
    assert np.allclose(h, 2.0 * g * expit(g), rtol=1e-15)                  # silu(gate) * up
    assert not np.allclose(h, g * 2.0 * expit(np.full_like(g, 2.0)), rtol=1e-3)  # not silu(up) * gate


def test_quant_closed_forms():
    R, I = 3, 256
    C = np.zeros((R, 2 * I), np.float32)
    C[0, :I] = 20.0; C[0, I:] = -1.5           # constant h: every code is -448
    C[1, :I] = 0.0;  C[1, I:] = 3.0            # zero h: scale 1, codes +0 / -0
    C[2, :I] = 30.0                            # silu(30) = 30 (1 - 1e-13)
    k = np.arange(128)
    want = np.where(k < 127, k | np.where(k % 2 == 1, 0x80, 0), 0x7E).astype(np.uint8)
    C[2, I:I + 128] = e4m3_table()[want] / 8.0   # h / s = the E4M3 value of `want`, exactly
    C[2, I + 128:] = 1.0
    bits = _bf16_bits(C)
    assert np.array_equal(_f(bits)[2, I:I + 128], e4m3_table()[want] / 8.0)
    codes, s = swiglu_quant_f64(bits, 0)
    s = s.reshape(R, 2)
    assert np.array_equal(codes[2, :128], want)
    assert np.all(codes[0] == 0xFE)
    assert np.allclose(s[0], 20.0 * 1.5 / 448.0, rtol=1e-12)
    assert np.all(s[1] == 1.0) and not (codes[1] & 0x7F).any()
    assert np.all(codes[2, 128:] == 0x7E) and np.allclose(s[2, 1], 30.0 / 448.0, rtol=1e-10)


def test_requantized_values_within_e4m3_rounding_of_fp64():
    rng = np.random.default_rng(5)
    R, I = 24, 384
    C = rng.standard_normal((R, 2 * I)).astype(np.float32) * 3
    C[0, :128] = 0.0
    bits = _bf16_bits(C)
    codes, SA = swiglu_quant_f64(bits, 0)
    g, u = _f(bits)[:, :I], _f(bits)[:, I:]
    h = g * expit(g) * u
    s = SA.reshape(R, I // 128)
    deq = e4m3_table()[codes] * np.repeat(s, 128, axis=1)
    bound = np.abs(h) * 2.0 ** -4 + np.repeat(s, 128, axis=1) * 2.0 ** -10 + np.abs(h) * 1e-12
    assert np.all(np.abs(deq - h) <= bound)
    amax = np.abs(h).reshape(R, I // 128, 128).max(axis=2)
    assert np.allclose(s[amax > 0], amax[amax > 0] / 448.0, rtol=1e-12)


def test_layouts_are_transposes():
    rng = np.random.default_rng(6)
    bits = _bf16_bits(rng.standard_normal((10, 512)).astype(np.float32))
    c0, s0 = swiglu_quant_f64(bits, 0)
    c1, s1 = swiglu_quant_f64(bits, 1)
    assert np.array_equal(c0, c1)
    assert np.array_equal(s0.reshape(10, 2), s1.reshape(2, 10).T)


def _case(R=64, I=384, seed=7):
    rng = np.random.default_rng(seed)
    C = rng.standard_normal((R, 2 * I)).astype(np.float32)
    C[:, :I] *= 6
    C[1, :I] = np.linspace(-120, 120, I, dtype=np.float32)   # past fp32 overflow of e^-g
    C[2, I:I + 128] *= np.float32(2.0 ** -30)                  # tiny h: subnormal codes
    C[3, :128] = 0.0
    return _bf16_bits(C)


def _fp32_result(bits, layout, sign=1.0, swap=False):
    """An independent fp32 evaluation: numpy's float32 exp, IEEE divisions."""
    C = _f(bits).astype(np.float32)
    I = C.shape[1] // 2
    g, u = (C[:, I:], C[:, :I]) if swap else (C[:, :I], C[:, I:])
    with np.errstate(over="ignore"):
        h = (g / (np.float32(1) + np.exp(np.float32(-sign) * g))) * u
    R, G = h.shape[0], I // 128
    amax = np.abs(h).reshape(R, G, 128).max(axis=2)
    s = np.where(amax > 0, amax / np.float32(448), np.float32(1)).astype(np.float32)
    v = np.clip(h / np.repeat(s, 128, axis=1), np.float32(-448), np.float32(448)).astype(np.float32)
    codes = e4m3_encode_rne(v)
    return codes, (s.reshape(-1) if layout == 0 else s.T.copy().reshape(-1))


@pytest.mark.parametrize("layout", [0, 1])
def test_check_accepts_definition_and_fp32_evaluation(layout):
    bits = _case()
    codes, s = swiglu_quant_f64(bits, layout)
    r = check_swiglu_quant(bits, codes, s.astype(np.float32), layout)
    assert r["bad_codes"] == 0 and r["bad_scales"] == 0 and r["nan"] == 0
    codes32, s32 = _fp32_result(bits, layout)
    r = check_swiglu_quant(bits, codes32, s32, layout)
    assert r["bad_codes"] == 0 and r["bad_scales"] == 0
    assert r["ambiguous"] <= r["elements"] // 1000     # the window is narrow


@pytest.mark.parametrize("mistake", ["swap", "sign", "code_step", "scale_ulps", "layout", "nan"])
def test_check_rejects_planted_mistakes(mistake):
    bits = _case()
    codes, s = _fp32_result(bits, 0)
    layout = 0
    if mistake == "swap":
        codes, s = _fp32_result(bits, 0, swap=True)
    elif mistake == "sign":
        codes, s = _fp32_result(bits, 0, sign=-1.0)
    elif mistake == "code_step":
        codes = codes.copy()
        codes[5, 17] = (codes[5, 17] & 0x80) | min((codes[5, 17] & 0x7F) + 1, 0x7E) \
            if (codes[5, 17] & 0x7F) < 0x7E else codes[5, 17] - 1
    elif mistake == "scale_ulps":
        s = s.copy()
        s[9] = np.float32(s[9] * (1 + 2.0 ** -16))
    elif mistake == "layout":
        layout = 1
    elif mistake == "nan":
        codes = codes.copy()
        codes[4, 3] = 0x7F
    r = check_swiglu_quant(bits, codes, s, layout)
    assert r["bad_codes"] + r["bad_scales"] > 0, r


def test_h_quant_matches_bf16_path_and_slack_widens():
    """h_quant_f64 on the bf16 values equals swiglu_quant_f64; g_slack /
    u_slack accept results computed from perturbed inputs that are rejected
    without them."""
    bits = _case(R=16, I=256, seed=9)
    g, u = _f(bits)[:, :256], _f(bits)[:, 256:]
    c0, s0 = swiglu_quant_f64(bits, 0)
    c1, s1 = h_quant_f64(g, u, 0)
    assert np.array_equal(c0, c1) and np.array_equal(s0, s1)
    gp, up = g * (1 + 3e-4), u * (1 - 3e-4)           # inputs off by 3e-4 relative
    cp, sp = h_quant_f64(gp, up, 0)
    r = check_h_quant(g, u, cp, sp.astype(np.float32), 0)
    assert r["bad_codes"] + r["bad_scales"] > 0
    r = check_h_quant(g, u, cp, sp.astype(np.float32), 0, g_slack=3e-4 * np.abs(g) * 1.001,
                      u_slack=3e-4 * np.abs(u) * 1.001)
    assert r["bad_codes"] == 0 and r["bad_scales"] == 0, r
