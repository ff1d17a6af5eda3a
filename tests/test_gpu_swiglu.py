"""GPU SwiGLU + E4M3 requantization (w4a8_swiglu_quant) against the fp64
definition (oracle/swiglu.py): every scale and every code must be admissible
-- what the definition gives for values within 2^-20 relative of the exact
ones (the bounds are stated in the oracle's docstring) -- on four shapes in
both scale layouts, with rows past both ends of the fp32 exponential and
codes in the E4M3 subnormal range, and on 256 sampled rows of the large
prefill gate/up output.  The count of elements where two codes were
admissible is printed beside the result."""

import numpy as np
import pytest
import torch

from oracle import check_swiglu_quant

pytestmark = pytest.mark.gpu


def _bf16_bits(x):
    return (np.asarray(x, dtype=np.float32).view(np.uint32) >> 16).astype(np.uint16)


def _gate_up(R, I, seed):
    rng = np.random.default_rng(seed)
    C = rng.standard_normal((R, 2 * I)).astype(np.float32)
    C[:, :I] *= np.float32(6.0)
    if R > 3:
        C[0, :128] = 0.0                                     # zero gate: h = +-0, scale 1
        C[1, :I] = np.linspace(-120, 120, I, dtype=np.float32)  # past both ends of e^-g in fp32
        C[2, I:I + 128] *= np.float32(2.0 ** -30)             # tiny h: codes in the subnormal range
        C[3, I:I + 128] = 0.0
        C[3, I + 5] = 1.0                                     # one nonzero h: the scale's element codes 448
    return _bf16_bits(C)


def _assert_admissible(bits, codes, scales, layout, label):
    r = check_swiglu_quant(bits, codes, scales, layout)
    print(f"{label}: {r}", flush=True)
    assert r["bad_codes"] == 0 and r["bad_scales"] == 0 and r["nan"] == 0, r
    assert r["ambiguous"] <= max(8, r["elements"] // 1000), r
    return r


@pytest.mark.parametrize("layout", [0, 1])
@pytest.mark.parametrize("R,I,seed", [(1, 128, 1), (37, 384, 2), (512, 2048, 3), (640, 1792, 4)])
def test_swiglu_quant_admissible(gpu_lib, layout, R, I, seed):
    bits = _gate_up(R, I, seed)
    Cd = torch.from_numpy(bits.view(np.int16)).to("cuda")
    A, SA = gpu_lib.swiglu_quant(Cd, layout)
    A2, SA2 = gpu_lib.swiglu_quant(Cd, layout)
    torch.cuda.synchronize()
    codes = A.cpu().numpy()
    _assert_admissible(bits, codes, SA.cpu().numpy().reshape(-1), layout, f"R={R} I={I} layout={layout}")
    assert np.array_equal(codes, A2.cpu().numpy())                       # deterministic
    assert np.array_equal(SA.cpu().numpy(), SA2.cpu().numpy())
    if R > 3:
        assert (codes[3, 5] & 0x7F) == 0x7E and not np.delete(codes[3, :128] & 0x7F, 5).any()


def test_swiglu_quant_prefill_size_sampled(gpu_lib):
    """131072 rows x (2 x 2048) (the large prefill gate/up output), M-major
    scales: 256 sampled rows against the definition."""
    R, I = 131072, 2048
    g = torch.Generator(device="cuda").manual_seed(7)
    C = (torch.randn((R, 2 * I), generator=g, device="cuda") * 3).to(torch.bfloat16)
    A, SA = gpu_lib.swiglu_quant(C, 1)
    torch.cuda.synchronize()
    rows = torch.from_numpy(np.random.default_rng(8).choice(R, size=256, replace=False)).to("cuda")
    bits = C[rows].view(torch.int16).cpu().numpy().view(np.uint16)
    got = SA.view(I // 128, R)[:, rows].T.contiguous().cpu().numpy().reshape(-1)
    _assert_admissible(bits, A[rows].cpu().numpy(), got, 0, "prefill sample")


def test_swiglu_quant_empty(gpu_lib):
    A, SA = gpu_lib.swiglu_quant(torch.zeros((0, 256), dtype=torch.bfloat16, device="cuda"), 0)
    assert A.shape == (0, 128) and SA.numel() == 0
