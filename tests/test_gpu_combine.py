"""GPU top-k combine (w4a8_combine): per-token bf16 sums bit for bit equal to
the oracle (oracle/combine.py), at small sizes and at the prefill
down-projection size in full."""

import numpy as np
import pytest
import torch

import synth
from oracle import combine_ref

pytestmark = pytest.mark.gpu


def _case(lib, T, k, E, N, seed, routing="uniform", R_extra=0):
    rng = np.random.default_rng(seed)
    ids = synth.make_routing(routing, T, E, k, seed)
    if T > 0:
        ids[0, 0] = -1  # an ignored slot
    _, off, ros = lib.route_prep(ids.to("cuda"), E)
    R = int(off[-1].item()) + R_extra
    C = torch.from_numpy(rng.standard_normal((R, N), dtype=np.float32)).to(torch.bfloat16)
    w = torch.from_numpy(rng.random(T * k, dtype=np.float32))
    out = lib.combine(C.to("cuda"), ros, w.to("cuda"), k)
    torch.cuda.synchronize()
    ref = combine_ref(C.view(torch.int16).numpy().view(np.uint16), ros.cpu().numpy(), w.numpy(), T, k)
    assert np.array_equal(out.view(torch.int16).cpu().numpy().view(np.uint16), ref)


@pytest.mark.parametrize("T,k,E,N,seed", [
    (1, 1, 4, 8, 1),
    (37, 2, 8, 520, 2),      # N not a multiple of 64 columns per wave
    (64, 8, 32, 4096, 3),    # decode gate/up width
    (200, 8, 12, 3584, 4),   # E=12 W2 output width
    (5, 8, 32, 8192, 5),     # two passes of 512 lanes
])
def test_combine_bit_exact(gpu_lib, T, k, E, N, seed):
    _case(gpu_lib, T, k, E, N, seed)


def test_combine_prefill_down_size(gpu_lib):
    """1152 tokens, top-8 biased routing over 32 experts, 6144 columns (the
    prefill down-projection output) in full."""
    cfg = synth.CONFIGS["prefill_down"]
    _case(gpu_lib, cfg["T"], cfg["top_k"], cfg["E"], cfg["N"], cfg["seed"], routing=cfg["routing"])


def test_combine_rows_outside_range_and_empty(gpu_lib):
    # a row map naming rows past R: those slots contribute nothing
    C = torch.ones((4, 64), dtype=torch.bfloat16, device="cuda")
    ros = torch.tensor([0, 7, -1, 3], dtype=torch.int32, device="cuda")
    w = torch.tensor([1.0, 5.0, 5.0, 0.5], dtype=torch.float32, device="cuda")
    out = gpu_lib.combine(C, ros, w, 2)
    torch.cuda.synchronize()
    assert torch.equal(out.float().cpu(), torch.tensor([[1.0] * 64, [0.5] * 64]))
    empty = gpu_lib.combine(C, torch.zeros(0, dtype=torch.int32, device="cuda"),
                            torch.zeros(0, dtype=torch.float32, device="cuda"), 2)
    assert empty.shape == (0, 64)
