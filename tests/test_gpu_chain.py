"""The whole MoE expert layer through the library's entry points on the GPU,
against the oracles chained the same way (an integration check):

    tokens --quantize_gather--> A1, SA1 --grouped_gemm (gate/up)--> C1
      --swiglu_quant--> A2, SA2 --grouped_gemm (down)--> C2 --combine--> out

Each GPU stage matches its oracle on the same inputs (the stage tests);
here every GPU stage consumes the GPU's own previous output and the oracle
chain its own (the SwiGLU step in fp64), so the GEMMs' fp32 rounding and the
fp32 SwiGLU can move an E4M3 code of the requantization by one step.  The check
is the chained error: per element within 3e-2 of max(rms, |ref|), and 5e-3
in the mean."""

import numpy as np
import pytest
import torch

import synth
from oracle import combine_ref, grouped_gemm_bf16, quantize_gather, route_ref, swiglu_quant_f64

pytestmark = pytest.mark.gpu


def _bits(t: torch.Tensor) -> np.ndarray:
    return t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


@pytest.mark.parametrize("layout", [0, 1])
def test_moe_layer_chain(gpu_lib, layout):
    E, T, k, H, I = 8, 48, 2, 512, 256
    g = torch.Generator().manual_seed(31)
    x = torch.randn((T, H), generator=g).to(torch.bfloat16)
    ids = synth.make_routing("uniform", T, E, k, 31)
    w13 = [synth.quantize_mxfp4(torch.randn((2 * I, H), generator=g) * 0.05) for _ in range(E)]
    w2 = [synth.quantize_mxfp4(torch.randn((H, I), generator=g) * 0.05) for _ in range(E)]
    B1 = torch.stack([b for b, _ in w13]); SB1 = torch.stack([s for _, s in w13])
    B2 = torch.stack([b for b, _ in w2]); SB2 = torch.stack([s for _, s in w2])
    wts = torch.rand((T * k,), generator=g)

    # GPU chain
    dev = "cuda"
    _, off, ros = gpu_lib.route_prep(ids.to(dev), E)
    R = int(off[-1].item())
    A1, SA1 = gpu_lib.quantize_gather(x.to(dev), ros, k, R, layout)
    C1 = gpu_lib.grouped_gemm(A1, SA1, layout, B1.to(dev), SB1.to(dev), off)
    A2, SA2 = gpu_lib.swiglu_quant(C1, layout)
    C2 = gpu_lib.grouped_gemm(A2, SA2, layout, B2.to(dev), SB2.to(dev), off)
    out = gpu_lib.combine(C2, ros, wts.to(dev), k)
    torch.cuda.synchronize()

    # oracle chain
    _, off_r, ros_r = route_ref(ids, E)
    assert np.array_equal(off.cpu().numpy(), off_r) and np.array_equal(ros.cpu().numpy(), ros_r)
    a1, sa1 = quantize_gather(_bits(x), ros_r, k, R, layout)
    c1 = grouped_gemm_bf16(a1, sa1, layout, B1.numpy(), SB1.numpy(), off_r)
    a2, sa2 = swiglu_quant_f64(c1, layout)
    sa2 = sa2.astype(np.float32)            # the boundary's scale format
    c2 = grouped_gemm_bf16(a2, sa2, layout, B2.numpy(), SB2.numpy(), off_r)
    ref = combine_ref(c2, ros_r, wts.numpy(), T, k)

    # the first stage is exact; the rest carry the GEMMs' rounding forward
    assert np.array_equal(A1.cpu().numpy(), a1)
    to_f = lambda b: (b.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    got, want = to_f(_bits(out)), to_f(ref)
    scale = max(np.sqrt(np.mean(want ** 2)), 1e-30)
    err = np.abs(got - want) / np.maximum(scale, np.abs(want))
    assert err.max() <= 3e-2, err.max()
    assert err.mean() <= 5e-3, err.mean()
