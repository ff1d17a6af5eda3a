"""GPU SwiGLU + E4M3 requantization (w4a8_swiglu_quant): codes and scales bit
for bit equal to the oracle (oracle/swiglu.py), which computes silu(g) * u
with the same fixed fp32 sequence."""

import numpy as np
import pytest
import torch

from oracle import swiglu_quant

pytestmark = pytest.mark.gpu


def _bf16_bits(x):
    return (np.asarray(x, dtype=np.float32).view(np.uint32) >> 16).astype(np.uint16)


def _gate_up(R, I, seed):
    rng = np.random.default_rng(seed)
    C = rng.standard_normal((R, 2 * I)).astype(np.float32)
    C[:, :I] *= np.float32(6.0)
    if R > 2:
        C[0, :128] = 0.0                                     # zero gate: h = +-0, scale 1
        C[1, :I] = np.linspace(-120, 120, I, dtype=np.float32)  # past both clamps of e^-g
        C[2, I:I + 128] *= np.float32(2.0 ** -30)             # tiny h: codes in the subnormal range
    return _bf16_bits(C)


@pytest.mark.parametrize("layout", [0, 1])
@pytest.mark.parametrize("R,I,seed", [(1, 128, 1), (37, 384, 2), (512, 2048, 3), (640, 1792, 4)])
def test_swiglu_quant_bit_exact(gpu_lib, layout, R, I, seed):
    bits = _gate_up(R, I, seed)
    A, SA = gpu_lib.swiglu_quant(torch.from_numpy(bits.view(np.int16)).to("cuda"), layout)
    torch.cuda.synchronize()
    codes, s = swiglu_quant(bits, layout)
    assert np.array_equal(A.cpu().numpy(), codes)
    assert np.array_equal(SA.cpu().numpy().reshape(-1).view(np.uint32), s.view(np.uint32))


def test_swiglu_quant_prefill_size_sampled(gpu_lib):
    """131072 rows x (2 x 2048) (the large prefill gate/up output), M-major
    scales: 256 sampled rows against the oracle."""
    R, I = 131072, 2048
    g = torch.Generator(device="cuda").manual_seed(7)
    C = (torch.randn((R, 2 * I), generator=g, device="cuda") * 3).to(torch.bfloat16)
    A, SA = gpu_lib.swiglu_quant(C, 1)
    torch.cuda.synchronize()
    rows = torch.from_numpy(np.random.default_rng(8).choice(R, size=256, replace=False)).to("cuda")
    bits = C[rows].view(torch.int16).cpu().numpy().view(np.uint16)
    codes, s = swiglu_quant(bits, 0)
    assert np.array_equal(A[rows].cpu().numpy(), codes)
    got = SA.view(I // 128, R)[:, rows].T.contiguous().cpu().numpy().reshape(-1)
    assert np.array_equal(got.view(np.uint32), s.view(np.uint32))


def test_swiglu_quant_empty(gpu_lib):
    A, SA = gpu_lib.swiglu_quant(torch.zeros((0, 256), dtype=torch.bfloat16, device="cuda"), 0)
    assert A.shape == (0, 128) and SA.numel() == 0
