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


# Batches below 1024 slots run with one ranking wave per 64 slots and a
# workgroup of those waves plus one per 64 experts: slot counts on both sides
# of each 64 boundary and of 1024, expert counts on both sides of 64 and
# beyond 16 * 64, and a few invalid ids among them.
@pytest.mark.parametrize("n", [1, 63, 64, 65, 127, 512, 1000, 1023, 1024, 1025])
@pytest.mark.parametrize("E", [1, 12, 64, 65, 1100, 6144])
def test_route_small_batches(gpu_lib, n, E):
    g = torch.Generator().manual_seed(n * 7919 + E)
    ids = torch.randint(0, E, (n, 1), generator=g, dtype=torch.int32)
    if n > 8:
        ids[3, 0] = -1
        ids[n // 2, 0] = E
    _route_case(gpu_lib, ids, E)


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


def _large_e_ids(T, top_k, E, seed, skew):
    return synth.make_wide_routing(T, E, top_k, seed, skew)


# The expert pools of MoonEP PR #38 (performance section: 1536 to 6144
# experts with 123 to 16384 tokens), top-8, and the one-wave edge of a 160 KB
# LDS workgroup (13648 experts).
LARGE_E = [(1536, 123, False), (2048, 16384, False), (3072, 4096, True), (6144, 16384, False),
           (6144, 123, True), (9216, 4096, True), (13648, 2048, False)]


@pytest.mark.parametrize("E,T,skew", LARGE_E)
def test_route_and_plan_large_e(gpu_lib, E, T, skew):
    ids = _large_e_ids(T, 8, E, seed=E + T, skew=skew)
    if E == 13648:
        ids[::7, 3] = -1            # ignored ids at the edge too
    off = _route_case(gpu_lib, ids, E)
    _plan_case(gpu_lib, off, E, 4096, K=512)


def test_route_large_e_capacity(gpu_lib):
    # 65536 experts need 786 KB of LDS with a single wave: reported before any launch
    ids = torch.zeros((4, 8), dtype=torch.int32, device="cuda")
    with pytest.raises(gpu_lib.W4A8Error) as ei:
        gpu_lib.route_prep(ids, 65536)
    assert ei.value.status == 5


def test_plan_largest_pool(gpu_lib):
    # the plan has no LDS bound: 65536 experts, most of them empty
    rng = np.random.default_rng(7)
    E = 65536
    counts = rng.integers(0, 300, size=E) * (rng.random(E) < 0.05)
    off = np.concatenate([[0], np.cumsum(counts)])
    _plan_case(gpu_lib, off, E, 2048)


@pytest.mark.parametrize("shift", [1, 2, 3])
@pytest.mark.parametrize("E,T,k", [(3072, 4096, 8), (32, 1, 2), (8, 3, 1), (6144, 123, 8)])
def test_route_ids_not_16_byte_aligned(gpu_lib, shift, E, T, k):
    # the histogram reads whole 16-byte units after a scalar head: ids that
    # start 4, 8 or 12 bytes past a 16-byte boundary, short lists included
    ids = _large_e_ids(T, k, E, seed=shift, skew=True)
    buf = torch.full((T * k + 8,), -1, dtype=torch.int32, device="cuda")
    buf[shift:shift + T * k] = ids.reshape(-1).cuda()
    view = buf[shift:shift + T * k].view(T, k)
    assert view.data_ptr() % 16 == 4 * shift
    c, o, r = gpu_lib.route_prep(view, E)
    torch.cuda.synchronize()
    rc, ro, rr = route_ref(ids, E)
    assert np.array_equal(c.cpu().numpy(), rc)
    assert np.array_equal(o.cpu().numpy(), ro)
    assert np.array_equal(r.cpu().numpy(), rr)
