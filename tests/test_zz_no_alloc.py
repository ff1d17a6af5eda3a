"""The allocation-free planned GEMM (w4a8_grouped_gemm_planned_noalloc),
called through the C ABI, against the planned GEMM with a caller-owned plan
(w4a8_plan + w4a8_grouped_gemm_planned) on the same inputs: bit for bit, on
two calls in a row, the second with fewer experts and rows than the first
(the scratch keeps the first call's plan, which must not leak into the
second), and a host-side rejection of a plan larger than the scratch."""

import ctypes

import numpy as np
import pytest
import torch

import synth
from helpers import bits_of

pytestmark = pytest.mark.gpu


def _ptr(t):
    return ctypes.c_void_p(t.data_ptr())


def _stream():
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def _noalloc(lib, A, SA, layout, B, SB, off, C, max_rows):
    E, N, Kh = B.shape
    return lib.w4a8_grouped_gemm_planned_noalloc(_ptr(A), _ptr(SA), layout, _ptr(B), _ptr(SB), _ptr(off), E, N,
                                                 2 * Kh, max_rows, _ptr(C), _stream())


def _with_plan(gpu_lib, A, SA, layout, B, SB, off):
    E, N, Kh = B.shape
    plan = gpu_lib.plan(off, E, N, 2 * Kh, max_total_rows=A.shape[0])
    return gpu_lib.grouped_gemm_planned(A, SA, layout, B, SB, off, plan)


@pytest.mark.parametrize("layout", [0, 1])
def test_noalloc_matches_planned_two_calls(gpu_lib, layout):
    lib = gpu_lib.load()
    cases = [([0, 5, 64, 65, 130, 300, 17, 0, 128, 1, 257, 40, 40], 320, 384, 31),   # larger first
             ([3, 0, 90, 20], 192, 256, 32)]                                          # then a smaller one
    for counts, N, K, seed in cases:
        A, SA, B, SB, off = synth.random_codes_problem(counts, N, K, seed)
        SA_l = (SA if layout == 0 else synth.to_m_major(SA)).cuda()
        A, B, SB, off = A.cuda(), B.cuda(), SB.cuda(), off.cuda()
        R = int(off[-1].item())
        C = torch.full((R, N), 7.0, dtype=torch.bfloat16, device="cuda")
        st = _noalloc(lib, A, SA_l, layout, B, SB, off, C, R)
        assert st == 0, lib.w4a8_last_error()
        want = _with_plan(gpu_lib, A, SA_l, layout, B, SB, off)
        torch.cuda.synchronize()
        print(f"layout={layout} E={len(counts)} R={R} N={N} K={K}: bit-identical "
              f"{np.array_equal(bits_of(C), bits_of(want))}", flush=True)
        assert np.array_equal(bits_of(C), bits_of(want))


def test_noalloc_rejects_plans_past_the_scratch(gpu_lib):
    lib = gpu_lib.load()
    A, SA, B, SB, off = synth.random_codes_problem([4, 4], 64, 128, 3)
    A, SA, B, SB, off = A.cuda(), SA.cuda(), B.cuda(), SB.cuda(), off.cuda()
    C = torch.zeros((8, 64), dtype=torch.bfloat16, device="cuda")
    assert _noalloc(lib, A, SA, 0, B, SB, off, C, 1 << 40) == 5       # W4A8_ERR_CAPACITY
    assert b"scratch" in lib.w4a8_last_error()
    assert _noalloc(lib, A, SA, 0, B, SB, off, C, 8) == 0
    torch.cuda.synchronize()
