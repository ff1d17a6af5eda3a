"""GPU gate/up GEMM with the SwiGLU + E4M3 requantization epilogue
(w4a8_grouped_gemm_swiglu) against the oracle chain: the exact fp64 GEMM
(oracle grouped_gemm_f64 / rows_gemm_f64) split into gate and up, then the
fp64 SwiGLU and quantization (oracle h_quant_f64 / check_h_quant).  The
fused kernel's gate and up are fp32 accumulators, so each may differ from
the exact value by the accumulation bound of the GEMM tests
(helpers.fp32_sum_eps(K) times the magnitude sum of its products); every
code and scale must be admissible for some gate and up within that bound.
The count of codes equal to the exact fp64 chain's is printed beside."""

import numpy as np
import pytest
import torch

import synth
from helpers import fp32_sum_eps
from oracle import check_h_quant, grouped_gemm_f64, h_quant_f64, route_ref
from oracle.gemm import rows_gemm_f64, sa_rows

pytestmark = pytest.mark.gpu


def _check(label, gexact, uexact, gmag, umag, K, codes, scales, layout2):
    eps = fp32_sum_eps(K)
    r = check_h_quant(gexact, uexact, codes, scales, layout2, g_slack=eps * gmag, u_slack=eps * umag)
    ref_codes, _ = h_quant_f64(gexact, uexact, layout2)
    same = int(np.count_nonzero(ref_codes == np.asarray(codes).reshape(ref_codes.shape)))
    print(f"{label}: {r} codes equal to the fp64 chain: {same}/{ref_codes.size}", flush=True)
    assert r["bad_codes"] == 0 and r["bad_scales"] == 0 and r["nan"] == 0, r
    assert same >= 0.98 * ref_codes.size
    return r


def _run(lib, A, SA, layout, B, SB, off, layout2):
    A2, SA2 = lib.grouped_gemm_swiglu(A, SA, layout, B, SB, off, layout2)
    torch.cuda.synchronize()
    return A2.cpu().numpy(), SA2.cpu().numpy().reshape(-1)


@pytest.mark.parametrize("layout,layout2", [(0, 0), (1, 1), (0, 1), (1, 0)])
@pytest.mark.parametrize("counts,I,K", [
    ([0, 5, 64, 65, 130, 300, 17, 0, 128, 1, 257], 256, 384),   # one to three m-tiles, empty experts
    ([3], 128, 128),                                             # E = 1, half an n-tile
    ([40, 0, 200], 384, 256),                                    # a partial last n-tile (I = 1.5 tiles)
])
def test_fused_small_shapes(gpu_lib, layout, layout2, counts, I, K):
    """Quantized N(0,1) activations and N(0, 0.02) weights, rows per expert
    given, both scale layouts on input and output."""
    E = len(counts)
    g = torch.Generator().manual_seed(sum(counts) + I + K)
    R = int(sum(counts))
    A, SA = synth.quantize_fp8_rows(torch.randn((R, K), generator=g))
    ws = [synth.quantize_mxfp4(0.02 * torch.randn((2 * I, K), generator=g)) for _ in range(E)]
    B = torch.stack([b for b, _ in ws]).contiguous()
    SB = torch.stack([s for _, s in ws]).contiguous()
    off = torch.zeros(E + 1, dtype=torch.int32)
    off[1:] = torch.cumsum(torch.tensor(counts), 0).to(torch.int32)
    SA_l = SA if layout == 0 else synth.to_m_major(SA)
    codes, scales = _run(gpu_lib, A.cuda(), SA_l.cuda(), layout, B.cuda(), SB.cuda(), off.cuda(), layout2)
    ex = grouped_gemm_f64(A, SA_l.reshape(-1), layout, B, SB, off)
    mag = grouped_gemm_f64(A, SA_l.reshape(-1), layout, B, SB, off, absolute=True)
    _check(f"counts={len(counts)} experts I={I} K={K} layouts={layout},{layout2}", ex[:, :I], ex[:, I:],
           mag[:, :I], mag[:, I:], K, codes, scales, layout2)


def test_fused_prefill_gateup_sampled(gpu_lib):
    """The 16384-token gate/up workload (E=32, top-8, N = 2I = 4096,
    K = 6144, M-major scales in and out) at full size; the oracle recomputes
    sampled rows (expert and tile boundaries plus random rows)."""
    p = synth.make_problem("prefill_gateup", device="cuda")
    _, off_dev, _ = gpu_lib.route_prep(p.topk_ids.cuda(), p.E)
    _, off, _ = route_ref(p.topk_ids, p.E)
    assert np.array_equal(off_dev.cpu().numpy(), off)
    SA_mm = synth.to_m_major(p.SA)
    A2, SA2 = gpu_lib.grouped_gemm_swiglu(p.A, SA_mm, 1, p.B, p.SB, off_dev, 1)
    torch.cuda.synchronize()
    I = p.N // 2
    rng = np.random.default_rng(5)
    rows = set()
    for e in range(p.E):
        lo, hi = int(off[e]), int(off[e + 1])
        if hi > lo:
            rows.update([lo, hi - 1, min(hi - 1, lo + 127), min(hi - 1, lo + 128)])
            rows.update(int(x) for x in rng.integers(lo, hi, size=2))
    rows = np.array(sorted(rows), dtype=np.int64)
    ex_of = np.searchsorted(off, rows, side="right") - 1
    rows_t = torch.from_numpy(rows).cuda()
    a_rows = p.A[rows_t].cpu().numpy()
    sa_r = sa_rows(SA_mm.cpu().numpy(), 1, rows, p.R, p.K)
    Bc, SBc = p.B.cpu().numpy(), p.SB.cpu().numpy()
    exact = rows_gemm_f64(a_rows, sa_r, ex_of, Bc, SBc)
    mag = rows_gemm_f64(a_rows, sa_r, ex_of, Bc, SBc, absolute=True)
    codes = A2[rows_t].cpu().numpy()
    scales = SA2.view(I // 128, p.R)[:, rows_t].T.contiguous().cpu().numpy().reshape(-1)
    _check(f"prefill_gateup fused, {len(rows)} sampled rows", exact[:, :I], exact[:, I:], mag[:, :I],
           mag[:, I:], p.K, codes, scales, 0)


def test_fused_no_rows(gpu_lib):
    """Experts without rows: nothing to write (the binding returns the empty
    outputs; with real buffers and all-empty offsets the kernel writes
    nothing)."""
    A, SA, B, SB, off = synth.random_codes_problem([0, 0], 256, 128, 3)
    A2, SA2 = gpu_lib.grouped_gemm_swiglu(torch.zeros((0, 128), dtype=torch.uint8, device="cuda"),
                                          torch.zeros(0, dtype=torch.float32, device="cuda"), 0, B.cuda(),
                                          SB.cuda(), off.cuda(), 0)
    assert A2.shape == (0, 128) and SA2.numel() == 0
    A1 = torch.zeros((1, 128), dtype=torch.uint8, device="cuda")
    SA1 = torch.ones(1, dtype=torch.float32, device="cuda")
    A2 = torch.full((1, 128), 0x11, dtype=torch.uint8, device="cuda")
    SA2 = torch.full((1, 1), 5.0, dtype=torch.float32, device="cuda")
    gpu_lib.grouped_gemm_swiglu(A1, SA1, 0, B.cuda(), SB.cuda(), off.cuda(), 0, A2=A2, SA2=SA2)
    torch.cuda.synchronize()
    assert torch.all(A2 == 0x11) and torch.all(SA2 == 5.0)
