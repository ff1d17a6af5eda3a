"""GPU route prep and device plan: byte-for-byte equal to the oracle."""

import numpy as np
import pytest
import torch

import synth
from oracle import plan_ref, route_ref

pytestmark = pytest.mark.gpu


def _route_case(lib, ids_cpu, E):
    c, o, r = lib.route_prep(ids_cpu.to("cuda"), E)
    torch.cuda.synchronize()
    rc, ro, rr = route_ref(ids_cpu, E)
    assert np.array_equal(c.cpu().numpy(), rc)
    assert np.array_equal(o.cpu().numpy(), ro)
    assert np.array_equal(r.cpu().numpy(), rr)
    return ro


@pytest.mark.parametrize("name", list(synth.CONFIGS))
def test_route_configs(gpu_lib, name):
    cfg = synth.CONFIGS[name]
    ids = synth.make_routing(cfg["routing"], cfg["T"], cfg["E"], cfg["top_k"], cfg["seed"])
    _route_case(gpu_lib, ids, cfg["E"])


@pytest.mark.parametrize("case", ["one_expert", "e1", "sparse", "invalid", "empty", "e1024", "odd"])
def test_route_adversarial(gpu_lib, case):
    g = torch.Generator().manual_seed(hash(case) % 1000)
    if case == "one_expert":
        E, ids = 32, torch.full((1000, 8), 17, dtype=torch.int32)
    elif case == "e1":
        E, ids = 1, torch.zeros((333, 1), dtype=torch.int32)
    elif case == "sparse":
        E = 64
        ids = torch.where(torch.rand(700, 4, generator=g) < 0.5, 3, 61).to(torch.int32)
    elif case == "invalid":
        E = 16
        ids = torch.randint(-2, E + 2, (513, 3), generator=g, dtype=torch.int32)
    elif case == "empty":
        E, ids = 8, torch.zeros((0, 2), dtype=torch.int32)
    elif case == "e1024":
        E, ids = 1024, torch.randint(0, 1024, (4099, 6), generator=g, dtype=torch.int32)
    else:
        E, ids = 7, torch.randint(0, 7, (97, 5), generator=g, dtype=torch.int32)
    _route_case(gpu_lib, ids.contiguous(), E)


def _plan_case(lib, offsets_np, E, N, K=256, max_tiles=None):
    off = torch.from_numpy(np.asarray(offsets_np, dtype=np.int32)).cuda()
    R = int(np.asarray(offsets_np)[-1]) if len(offsets_np) else 0
    if max_tiles is None:
        out = lib.plan(off, E, N, K, max_total_rows=max(R, 0))
        max_tiles = (out.numel() - 8) // 4
    else:
        out = torch.zeros(8 + 4 * max_tiles, dtype=torch.int32, device="cuda")
        lib.plan(off, E, N, K, out=out)
    torch.cuda.synchronize()
    ref = plan_ref(offsets_np, E, N, max_tiles=max_tiles)
    got = out.cpu().numpy()[: len(ref)]
    assert np.array_equal(got, ref), (got[:16], ref[:16])


@pytest.mark.parametrize("name", list(synth.CONFIGS))
def test_plan_configs(gpu_lib, name):
    cfg = synth.CONFIGS[name]
    ids = synth.make_routing(cfg["routing"], cfg["T"], cfg["E"], cfg["top_k"], cfg["seed"])
    _, off, _ = route_ref(ids, cfg["E"])
    _plan_case(gpu_lib, off, cfg["E"], cfg["N"])


def test_plan_boundaries_and_capacity(gpu_lib):
    counts = [0, 1, 15, 16, 17, 63, 64, 65, 127, 128, 129, 255, 256, 257, 1000, 131072 - 3000]
    off = np.concatenate([[0], np.cumsum(counts)])
    _plan_case(gpu_lib, off, len(counts), 4096)
    _plan_case(gpu_lib, off, len(counts), 96)
    _plan_case(gpu_lib, off, len(counts), 4096, max_tiles=5)
    big = np.concatenate([[0], np.cumsum(np.random.default_rng(0).integers(0, 300, 1024))])
    _plan_case(gpu_lib, big, 1024, 256)


def test_plan_bad_offsets(gpu_lib):
    _plan_case(gpu_lib, np.array([0, 10, 5, 20]), 3, 256)
    _plan_case(gpu_lib, np.array([3, 10, 15]), 2, 256)
