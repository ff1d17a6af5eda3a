"""GPU grouped GEMM with bf16 activations and FP4 weights
(w4a8_grouped_gemm_a16), MXFP4 and NVFP4 weight scales, against the oracle
(oracle/a16.py).

The kernel sums products of exact bf16 operands on the matrix core in fp32,
one rounding per 16-K step, then multiplies by the per-expert scale and
rounds to bf16: every element must lie within that accumulation bound
(a16_group_eps(K) times the magnitude sum of its products) of the exact
value, plus the usual normalised-error and ulp checks (helpers.assert_parity).
"""

import numpy as np
import pytest
import torch

import synth
from helpers import assert_parity, bits_of
from oracle import bf16_rne_bits, route_ref
from oracle.a16 import FMT_MX, FMT_NV, grouped_gemm_a16_f64

pytestmark = pytest.mark.gpu


def a16_group_eps(K: int) -> float:
    """The part of the accumulation bound beyond helpers.fp32_sum_eps's
    per-128 term: one fp32 rounding per 16-K MFMA step (K/16 of them, of
    which fp32_sum_eps already counts K/128) and a margin for the matrix
    core's own sum of 16 exact products."""
    return (K // 16 - K // 128 + 1) * 2.0 ** -24 + 2.0 ** -20


def _check(lib, A, B, SB, fmt, GS, off, label, gs_arg=True):
    dev = [t.cuda() for t in (A, B, SB, off)]
    C = lib.grouped_gemm_a16(dev[0], dev[1], dev[2], fmt, dev[3], GS.cuda() if (gs_arg and GS is not None) else None)
    torch.cuda.synchronize()
    a = A.numpy().view(np.uint16)
    gs = GS.numpy() if (gs_arg and GS is not None) else None
    ex = grouped_gemm_a16_f64(a, B.numpy(), SB.numpy(), fmt, gs, off.numpy())
    mag = grouped_gemm_a16_f64(a, B.numpy(), SB.numpy(), fmt, gs, off.numpy(), absolute=True)
    K = A.shape[1]
    assert_parity(bits_of(C), bf16_rne_bits(ex), label, exact=ex, abs_sum=mag, K=K, group_eps=a16_group_eps(K))
    return C


def _codes_problem(counts, N, K, fmt, seed):
    """bf16 N(0,1) activations, random FP4 codes, moderate scale codes."""
    g = torch.Generator().manual_seed(seed)
    E, R = len(counts), int(sum(counts))
    A = synth.bf16_bits(torch.randn((R, K), generator=g))
    B = torch.randint(0, 256, (E, N, K // 2), generator=g, dtype=torch.int32).to(torch.uint8)
    if fmt == FMT_MX:
        SB = torch.randint(118, 136, (E, N, K // 32), generator=g, dtype=torch.int32).to(torch.uint8)
        GS = None
    else:
        mags = torch.randint(0x20, 0x58, (E, N, K // 16), generator=g, dtype=torch.int32)
        SB = (mags | (torch.randint(0, 2, mags.shape, generator=g, dtype=torch.int32) << 7)).to(torch.uint8)
        GS = torch.rand(E, generator=g) * 3 + 0.25
    off = torch.zeros(E + 1, dtype=torch.int32)
    off[1:] = torch.cumsum(torch.tensor(counts), 0).to(torch.int32)
    return A, B, SB, GS, off


@pytest.mark.parametrize("fmt", [FMT_MX, FMT_NV])
@pytest.mark.parametrize("counts,N,K", [
    ([3], 16, 128),                                   # one expert, one wave's columns
    ([0, 5, 16, 17, 0, 33, 64], 256, 384),             # row blocks 1..4, empty experts
    ([100, 0, 300, 65, 64, 1], 192, 512),              # several 64-row passes over the weights
    ([7, 20], 80, 256),                                # N = 80: the second item has one wave of columns
    ([40, 2, 0, 9], 1040, 1152),                       # nine K groups, N past 16 items
])
def test_a16_codes_shapes(gpu_lib, fmt, counts, N, K):
    A, B, SB, GS, off = _codes_problem(counts, N, K, fmt, seed=sum(counts) + N + K + fmt)
    _check(gpu_lib, A, B, SB, fmt, GS, off, f"a16 fmt={fmt} counts={counts[:4]} N={N} K={K}")


@pytest.mark.parametrize("fmt", [FMT_MX, FMT_NV])
@pytest.mark.parametrize("name", ["tiny", "decode_gateup", "e12_w2_m64"])
def test_a16_workloads_full(gpu_lib, fmt, name):
    """The decode gate/up and E=12 W2 M=64 shapes (and the tiny one) in full:
    bf16 N(0,1) activations, N(0, 0.02) weights quantized to MXFP4 or
    NVFP4 (with its per-expert tensor scale)."""
    p = synth.make_a16_problem(name, fmt)
    _, off, _ = route_ref(p.topk_ids, p.E)
    _, off_dev, _ = gpu_lib.route_prep(p.topk_ids.cuda(), p.E)
    assert np.array_equal(off_dev.cpu().numpy(), off)
    _check(gpu_lib, p.A, p.B, p.SB, fmt, p.GS, torch.from_numpy(off.astype(np.int32)),
           f"a16 {name} fmt={fmt} R={p.R}")


def test_a16_without_expert_scales_equals_ones(gpu_lib):
    A, B, SB, _, off = _codes_problem([9, 30, 0, 70], 128, 256, FMT_NV, seed=4)
    d = [t.cuda() for t in (A, B, SB, off)]
    C0 = gpu_lib.grouped_gemm_a16(d[0], d[1], d[2], FMT_NV, d[3], None)
    C1 = gpu_lib.grouped_gemm_a16(d[0], d[1], d[2], FMT_NV, d[3], torch.ones(4, device="cuda"))
    torch.cuda.synchronize()
    assert np.array_equal(bits_of(C0), bits_of(C1))


def test_a16_mx_scales_across_the_exponent_range(gpu_lib):
    """MXFP4 scale codes from 2^-107 to 2^93, mixed within every column (one
    code per 32-K block): the weight operands stay normal bf16 and every sum
    stays finite in fp32, the range the header states exact, which the
    kernel's scaled FP4 conversion covers by taking the scale's exponent."""
    counts, N, K = [17, 40, 5], 96, 512
    A, B, SB, _, off = _codes_problem(counts, N, K, FMT_MX, seed=77)
    g = torch.Generator().manual_seed(78)
    levels = torch.tensor([20, 60, 100, 127, 150, 200, 220], dtype=torch.int32)
    SB = levels[torch.randint(0, len(levels), tuple(SB.shape), generator=g)].to(torch.uint8)
    _check(gpu_lib, A, B, SB, FMT_MX, None, off, "MXFP4 scale codes 20..220")


@pytest.mark.parametrize("fmt,nan_code", [(FMT_MX, 0xFF), (FMT_NV, 0x7F), (FMT_NV, 0xFF)])
def test_a16_nan_scales_poison_their_columns(gpu_lib, fmt, nan_code):
    counts, N, K = [6, 21, 3], 64, 256
    A, B, SB, GS, off = _codes_problem(counts, N, K, fmt, seed=31)
    SB = SB.clone()
    SB[1, 37, 2] = nan_code                            # expert 1, column 37
    C = gpu_lib.grouped_gemm_a16(A.cuda(), B.cuda(), SB.cuda(), fmt, off.cuda(),
                                 GS.cuda() if GS is not None else None)
    torch.cuda.synchronize()
    c = C.float().cpu().numpy()
    ex = grouped_gemm_a16_f64(A.numpy().view(np.uint16), B.numpy(), SB.numpy(), fmt,
                              None if GS is None else GS.numpy(), off.numpy())
    assert np.array_equal(np.isnan(c), np.isnan(ex))
    assert np.isnan(c[6:27, 37]).all() and np.isnan(c).sum() == 21


def test_a16_bad_offsets_write_nothing(gpu_lib):
    A, B, SB, _, off = _codes_problem([10, 10, 10], 64, 128, FMT_MX, seed=2)
    bad = torch.tensor([0, 20, 10, 30], dtype=torch.int32)
    C = torch.full((30, 64), 7.0, dtype=torch.bfloat16, device="cuda")
    gpu_lib.grouped_gemm_a16(A.cuda(), B.cuda(), SB.cuda(), FMT_MX, bad.cuda(), None, out=C)
    torch.cuda.synchronize()
    assert torch.all(C == 7.0)
    C0 = gpu_lib.grouped_gemm_a16(torch.zeros((0, 128), dtype=torch.bfloat16, device="cuda"), B.cuda(),
                                  SB.cuda(), FMT_MX, torch.zeros(4, dtype=torch.int32, device="cuda"), None)
    assert C0.shape == (0, 64)
