"""The whole expert layer captured in one HIP graph through torch's graph
capture: every entry point is stream-ordered and allocation-free, so the
launches record as graph nodes.  Replays must equal the eager layer bit for
bit, several times, with eager work (clearing the outputs, new tokens)
between them; a replay must read the buffers' current contents."""

import numpy as np
import pytest
import torch

import synth

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("layout", [0, 1])
def test_layer_graph_replay_matches_eager(gpu_lib, layout):
    E, T, k, H, I = 8, 48, 2, 512, 256
    R = T * k
    g = torch.Generator().manual_seed(41)
    dev = "cuda"
    xs = [torch.randn((T, H), generator=g).to(torch.bfloat16).to(dev) for _ in range(2)]
    ids = synth.make_routing("uniform", T, E, k, 41).to(dev)
    w13 = [synth.quantize_mxfp4(torch.randn((2 * I, H), generator=g) * 0.05) for _ in range(E)]
    w2 = [synth.quantize_mxfp4(torch.randn((H, I), generator=g) * 0.05) for _ in range(E)]
    B1 = torch.stack([b for b, _ in w13]).to(dev); SB1 = torch.stack([s for _, s in w13]).to(dev)
    B2 = torch.stack([b for b, _ in w2]).to(dev); SB2 = torch.stack([s for _, s in w2]).to(dev)
    wts = torch.rand((T * k,), generator=g).to(dev)

    x = xs[0].clone()
    counts = torch.empty(E, dtype=torch.int32, device=dev)
    off = torch.empty(E + 1, dtype=torch.int32, device=dev)
    ros = torch.empty(R, dtype=torch.int32, device=dev)
    A1 = torch.empty((R, H), dtype=torch.uint8, device=dev)
    SA1 = torch.empty((R, H // 128) if layout == 0 else (H // 128, R), dtype=torch.float32, device=dev)
    C1 = torch.empty((R, 2 * I), dtype=torch.bfloat16, device=dev)
    A2 = torch.empty((R, I), dtype=torch.uint8, device=dev)
    SA2 = torch.empty((R, I // 128) if layout == 0 else (I // 128, R), dtype=torch.float32, device=dev)
    C2 = torch.empty((R, H), dtype=torch.bfloat16, device=dev)
    out = torch.empty((T, H), dtype=torch.bfloat16, device=dev)
    outputs = (counts, off, ros, A1, SA1, C1, A2, SA2, C2, out)

    def layer():
        gpu_lib.route_prep(ids, E, counts, off, ros)
        gpu_lib.quantize_gather(x, ros, k, R, layout, A=A1, SA=SA1)
        gpu_lib.grouped_gemm(A1, SA1, layout, B1, SB1, off, out=C1)
        gpu_lib.swiglu_quant(C1, layout, A=A2, SA=SA2)
        gpu_lib.grouped_gemm(A2, SA2, layout, B2, SB2, off, out=C2)
        gpu_lib.combine(C2, ros, wts, k, out=out)

    def snapshot():
        torch.cuda.synchronize()
        return [t.clone() for t in outputs]

    eager = []
    for xi in xs:
        x.copy_(xi)
        layer()
        eager.append(snapshot())
    assert not torch.equal(eager[0][-1], eager[1][-1])

    graph = torch.cuda.graph_pool_handle()
    gr = torch.cuda.CUDAGraph()
    x.copy_(xs[0])
    torch.cuda.synchronize()
    with torch.cuda.graph(gr, pool=graph):
        layer()
    torch.cuda.synchronize()

    for rep, which in enumerate([0, 1, 0, 1]):
        for t in outputs:
            t.zero_()                      # eager work between replays
        x.copy_(xs[which])
        gr.replay()
        got = snapshot()
        for name, a, b in zip(("counts", "offsets", "row_of_slot", "A1", "SA1", "C1", "A2", "SA2", "C2", "out"),
                              got, eager[which]):
            assert torch.equal(a, b), f"replay {rep}: {name} differs from the eager layer"
