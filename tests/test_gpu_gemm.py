"""GPU grouped GEMM against the CPU oracle.

Bar (elementwise): |gpu - ref| / max(rms(ref), |ref|) <= 8e-3 on seeded
workloads, at most one bf16 ulp on elements at least rms(ref) in size, and
no element farther from the exact fp64 value than fp32 accumulation plus one
bf16 rounding allow (tests/helpers.py); exact bits on inputs whose result is exactly representable
(all-ones and one-hot rows with power-of-two activation scales); row-major
and M-major scales bit-identical; repeated calls bit-identical.
"""

import numpy as np
import pytest
import torch

import synth
from helpers import GROUP_EPS_RANDOM_CODES, assert_parity, bits_of, sample_rows, to_device
from oracle import bf16_rne_bits, grouped_gemm_bf16, grouped_gemm_f64, plan as oplan, route_ref
from oracle.gemm import rows_gemm_f64, sa_rows

pytestmark = pytest.mark.gpu


def _run(lib, A, SA, layout, B, SB, off_dev):
    C = lib.grouped_gemm(A, SA, layout, B, SB, off_dev)
    torch.cuda.synchronize()
    return C


def _full_config(lib, name, layout):
    p = synth.make_problem(name)
    d = to_device(p)
    _, off_dev, _ = lib.route_prep(d["ids"], p.E)
    _, off, _ = route_ref(p.topk_ids, p.E)
    assert np.array_equal(off_dev.cpu().numpy(), off)
    SA_cpu = p.SA if layout == 0 else synth.to_m_major(p.SA)
    C = _run(lib, d["A"], SA_cpu.cuda(), layout, d["B"], d["SB"], off_dev)
    exact = grouped_gemm_f64(p.A, SA_cpu.reshape(-1), layout, p.B, p.SB, off)
    mag = grouped_gemm_f64(p.A, SA_cpu.reshape(-1), layout, p.B, p.SB, off, absolute=True)
    ref = bf16_rne_bits(exact)
    assert_parity(bits_of(C), ref, f"{name} layout={layout} R={p.R}", exact=exact, abs_sum=mag, K=p.K)
    return bits_of(C)


@pytest.mark.parametrize("name,layout", [
    ("tiny", 0), ("tiny", 1),
    ("decode_gateup", 0),
    ("prefill_down", 0), ("prefill_down", 1),
    ("e12_w13_m8", 0), ("e12_w13_m64", 0), ("e12_w2_m8", 0), ("e12_w2_m64", 0),
    ("e12_w2_m64", 1),
])
def test_gemm_config_full(gpu_lib, name, layout):
    _full_config(gpu_lib, name, layout)


def test_gemm_prefill_gateup_sampled(gpu_lib):
    """The 16384-token gate/up workload at full size, M-major scales; the
    oracle recomputes sampled rows (expert and tile boundaries plus random
    rows of every expert), all N columns each."""
    p = synth.make_problem("prefill_gateup", device="cuda")
    _, off_dev, _ = gpu_lib.route_prep(p.topk_ids.cuda(), p.E)
    _, off, _ = route_ref(p.topk_ids, p.E)
    assert np.array_equal(off_dev.cpu().numpy(), off)
    SA_mm = synth.to_m_major(p.SA)
    C = _run(gpu_lib, p.A, SA_mm, 1, p.B, p.SB, off_dev)
    rng = np.random.default_rng(4)

    def tile_m_of(rows):
        cls, tm, _ = oplan.tile_rule(rows)
        return tm if cls == oplan.CLASS_MFMA else 0

    rows = sample_rows(off, tile_m_of, rng, per_expert_random=2)
    ex = np.searchsorted(off, rows, side="right") - 1
    rows_t = torch.from_numpy(rows).cuda()
    a_rows = p.A[rows_t].cpu().numpy()
    sa_r = sa_rows(SA_mm.cpu().numpy(), 1, rows, p.R, p.K)
    Bc, SBc = p.B.cpu().numpy(), p.SB.cpu().numpy()
    exact = rows_gemm_f64(a_rows, sa_r, ex, Bc, SBc)
    mag = rows_gemm_f64(a_rows, sa_r, ex, Bc, SBc, absolute=True)
    got = bits_of(C[rows_t])
    assert_parity(got, bf16_rne_bits(exact), f"prefill_gateup sampled rows={len(rows)}", exact=exact,
                  abs_sum=mag, K=p.K)


def _codes_case(lib, counts, N, K, seed, layout=0, exact=False, a_fill=None, sa_pow2=False, sa_fill=None):
    A, SA, B, SB, off = synth.random_codes_problem(counts, N, K, seed)
    R = int(off[-1])
    if a_fill is not None:
        A = a_fill(A)
    if sa_pow2:
        g = torch.Generator().manual_seed(seed + 1)
        SA = torch.exp2(torch.randint(-3, 3, SA.shape, generator=g).float())
    if sa_fill is not None:
        SA = sa_fill(SA)
    SA_l = SA if layout == 0 else synth.to_m_major(SA)
    C = _run(lib, A.cuda(), SA_l.cuda(), layout, B.cuda(), SB.cuda(), off.cuda())
    ex64 = grouped_gemm_f64(A, SA_l.reshape(-1), layout, B, SB, off)
    ref = bf16_rne_bits(ex64)
    got = bits_of(C)
    if exact:
        assert np.array_equal(got, ref), int(np.sum(got != ref))
    else:
        mag = grouped_gemm_f64(A, SA_l.reshape(-1), layout, B, SB, off, absolute=True)
        assert_parity(got, ref, f"counts={len(counts)} experts N={N} K={K} layout={layout}", exact=ex64,
                      abs_sum=mag, K=K, group_eps=GROUP_EPS_RANDOM_CODES)
    return got


MIXED = [0, 5, 64, 65, 130, 300, 17, 0, 128, 1, 257]


@pytest.mark.parametrize("layout", [0, 1])
def test_all_ones_bit_exact(gpu_lib, layout):
    _A, _SA, B, SB, off = synth.random_codes_problem(MIXED, 288, 512, 7)
    B = torch.full_like(B, 0x22)
    R = int(off[-1])
    g = torch.Generator().manual_seed(8)
    SA = torch.exp2(torch.randint(-3, 3, (R, 4), generator=g).float())
    A = torch.full((R, 512), 0x38, dtype=torch.uint8)
    SA_l = SA if layout == 0 else synth.to_m_major(SA)
    C = _run(gpu_lib, A.cuda(), SA_l.cuda(), layout, B.cuda(), SB.cuda(), off.cuda())
    ref = grouped_gemm_bf16(A, SA_l.reshape(-1), layout, B, SB, off)
    assert np.array_equal(bits_of(C), ref)


@pytest.mark.parametrize("layout", [0, 1])
def test_one_hot_rows_bit_exact(gpu_lib, layout):
    def one_hot(A):
        g = torch.Generator().manual_seed(3)
        R, K = A.shape
        out = torch.zeros_like(A)
        k0 = torch.randint(0, K, (R,), generator=g)
        code = torch.randint(0, 0x7F, (R,), generator=g).to(torch.uint8) | \
            (torch.randint(0, 2, (R,), generator=g).to(torch.uint8) << 7)
        out[torch.arange(R), k0] = code
        return out
    _codes_case(gpu_lib, MIXED, 256, 384, 11, layout=layout, exact=True, a_fill=one_hot,
                sa_pow2=True)


@pytest.mark.parametrize("layout", [0, 1])
def test_bf16_rounding_ties_bit_exact(gpu_lib, layout):
    """One-hot rows of 1.0 times activation scales with at most 21 significant
    bits: every output is one product, exact in fp32 (E2M1 values have at most
    two significant bits), so the GPU's bf16 rounding must equal the oracle's
    round-to-nearest-even of the exact value bit for bit.  A third of the
    scales sit exactly halfway between two bf16 values (1 + j/256, j odd), so
    ties must go to even."""
    def one_hot(A):
        g = torch.Generator().manual_seed(5)
        R, K = A.shape
        out = torch.zeros_like(A)
        k0 = torch.randint(0, K, (R,), generator=g)
        out[torch.arange(R), k0] = torch.where(torch.rand(R, generator=g) < 0.5, 0x38, 0xB8).to(torch.uint8)
        return out

    def sa_fill(SA):
        g = torch.Generator().manual_seed(6)
        m = torch.randint(0, 1 << 20, SA.shape, generator=g)
        ties = (2 * torch.randint(0, 128, SA.shape, generator=g) + 1) << 12
        pick = torch.randint(0, 3, SA.shape, generator=g) == 0
        e = torch.randint(-4, 4, SA.shape, generator=g).float()
        return ((1.0 + torch.where(pick, ties, m).double() / (1 << 20)) * torch.exp2(e.double())).float()

    _codes_case(gpu_lib, MIXED, 256, 384, 13, layout=layout, exact=True, a_fill=one_hot, sa_fill=sa_fill)


def test_layouts_bit_identical_and_deterministic(gpu_lib):
    a = _codes_case(gpu_lib, MIXED, 256, 640, 21, layout=0)
    b = _codes_case(gpu_lib, MIXED, 256, 640, 21, layout=1)
    c = _codes_case(gpu_lib, MIXED, 256, 640, 21, layout=0)
    assert np.array_equal(a, b) and np.array_equal(a, c)


DECODE_ROWS = [0, 0, 1, 3, 5, 5, 6, 6, 7, 7, 7, 8, 9, 9, 11, 14, 15, 15, 16, 17, 19, 21, 21, 21, 25, 25, 26,
               30, 33, 36, 40, 54]


@pytest.mark.parametrize("counts,N,K", [
    ([3], 32, 128),                   # E = 1, one streaming item
    ([200], 96, 256),                 # E = 1, MFMA class, partial n-tile
    ([0, 0, 0, 70, 0], 288, 256),     # empty experts around one MFMA expert
    ([64, 65, 16, 17, 48, 49], 320, 384),
    (list(range(0, 140, 7)), 256, 128),
    ([5] * 300, 192, 128),            # more streaming tiles than CUs, all one row block
    ([40] * 3 + [0] + [33] * 2, 8192, 256),  # equal row blocks: units split per expert
    # decode-like skewed rows (1..4 row blocks): items dealt round-robin, four
    # units wide for experts of up to 32 rows and three above, with a
    # narrower last item per expert (62 units) or a half unit at N (4000)
    (DECODE_ROWS, 3968, 256),
    (DECODE_ROWS, 4000, 128),
    # longer K loops (two to seven stages per item, odd and even stage
    # counts, a kh=1 half one group short at K = 640, narrow last items of 62
    # and 33 units per expert, two and more items per workgroup)
    (DECODE_ROWS, 3968, 768),
    (DECODE_ROWS, 3968, 640),
    ([64, 1, 17, 33, 49, 0, 16, 32, 48] * 7, 2112, 1792),
    (DECODE_ROWS, 4000, 1408),
    ([5] * 300, 192, 1024),
    ([40] * 3 + [0] + [33] * 2, 8192, 640),
    (list(range(0, 140, 7)), 256, 1152),
    ([3], 32, 896),
    # about one workgroup per expert (200 experts of 1-4 row blocks): each
    # workgroup's range of 64 blocks runs as two or three items
    ([9, 33, 50, 2] * 50, 1024, 384),
    # narrow items split K between the two halves of the workgroup: 10
    # blocks per workgroup with four row blocks, 16 with two (odd group count)
    ([60] * 40, 1024, 384),
    ([20] * 16, 4096, 640),
    # either side of the register-only split (pools under 64 experts) and the
    # LDS-table split: 63 and 64 experts of mixed sizes, empty ones included
    ([17, 40, 3, 0, 64, 9, 80] * 9, 1024, 384),
    ([17, 40, 3, 0, 64, 9, 80] * 9 + [33], 1024, 384),
    # whole-K items of three blocks per wave (17-24 blocks per workgroup) on
    # the two-stage ring: with one and two row blocks (12 experts), three and
    # four (18 experts, where one- and two-row-block experts get 29-35 blocks,
    # some as two items), with one and three K groups (one- and two-stage
    # loops; fewer groups than a scale chunk)
    ([5, 9, 17, 30, 44, 64, 1, 12, 23, 50, 60, 33], 6144, 128),
    ([40, 47, 5, 9, 17, 30, 44, 64, 1, 12, 23, 50, 60, 33, 36, 41, 20, 8], 6144, 384),
])
def test_ragged_and_edge_shapes(gpu_lib, counts, N, K):
    _codes_case(gpu_lib, counts, N, K, seed=sum(counts) + N)


def test_zero_rows(gpu_lib):
    A, SA, B, SB, off = synth.random_codes_problem([0, 0, 0], 64, 256, 1)
    # no rows at all: the binding has nothing to launch
    C = gpu_lib.grouped_gemm(torch.zeros((0, 256), dtype=torch.uint8, device="cuda"),
                             torch.zeros(0, dtype=torch.float32, device="cuda"), 0, B.cuda(),
                             SB.cuda(), off.cuda())
    assert C.shape == (0, 64)
    # all experts empty on the device, with real buffers: the kernels write nothing
    A1 = torch.zeros((1, 256), dtype=torch.uint8, device="cuda")
    SA1 = torch.ones(2, dtype=torch.float32, device="cuda")
    C1 = torch.full((1, 64), 3.0, dtype=torch.bfloat16, device="cuda")
    gpu_lib.grouped_gemm(A1, SA1, 0, B.cuda(), SB.cuda(), off.cuda(), out=C1)
    torch.cuda.synchronize()
    assert torch.all(C1 == 3.0)


def test_bad_offsets_write_nothing(gpu_lib):
    A, SA, B, SB, off = synth.random_codes_problem([10, 10, 10], 64, 256, 2)
    bad = torch.tensor([0, 20, 10, 30], dtype=torch.int32)   # decreasing: rejected on device
    C = torch.full((30, 64), 7.0, dtype=torch.bfloat16, device="cuda")
    gpu_lib.grouped_gemm(A.cuda(), SA.cuda(), 0, B.cuda(), SB.cuda(), bad.cuda(), out=C)
    torch.cuda.synchronize()
    assert torch.all(C == 7.0)


@pytest.mark.parametrize("E,T,skew,N", [(1536, 123, False, 256), (2048, 4096, True, 192), (2048, 16, False, 320)])
def test_wide_expert_pool(gpu_lib, E, T, skew, N):
    """The grouped GEMM over the wide shared pools of MoonEP PR #38
    (performance section: 1536 and 2048 experts), rows from the GPU route
    prep of top-8 wide routing: hundreds of one- to few-row streaming experts
    and, skewed, MFMA-class experts beside them."""
    ids = synth.make_wide_routing(T, E, 8, seed=E + T, skew=skew)
    counts, off_ref, _ = route_ref(ids, E)
    _, off_dev, _ = gpu_lib.route_prep(ids.cuda(), E)
    assert np.array_equal(off_dev.cpu().numpy(), off_ref)
    A, SA, B, SB, off = synth.random_codes_problem(counts.tolist(), N, 256, seed=E + N)
    assert np.array_equal(off.numpy(), off_ref)
    for layout in (0, 1):
        SA_l = SA if layout == 0 else synth.to_m_major(SA)
        C = _run(gpu_lib, A.cuda(), SA_l.cuda(), layout, B.cuda(), SB.cuda(), off_dev)
        ex64 = grouped_gemm_f64(A, SA_l.reshape(-1), layout, B, SB, off)
        mag = grouped_gemm_f64(A, SA_l.reshape(-1), layout, B, SB, off, absolute=True)
        assert_parity(bits_of(C), bf16_rne_bits(ex64), f"E={E} T={T} skew={skew} N={N} layout={layout} "
                      f"R={int(off[-1])} max_rows={int(counts.max())}", exact=ex64, abs_sum=mag, K=256,
                      group_eps=GROUP_EPS_RANDOM_CODES)


def test_wide_pool_full_size_sampled(gpu_lib):
    """2048 experts at the benchmark's gate/up shape (N=4096, K=6144), 16384
    tokens at top-8, rows from the GPU route prep: every one of the 2048
    experts gets rows, most of them near the 64-row boundary between the two
    classes.  The oracle recomputes sampled rows of 16 experts of both
    classes (first, last and a random row each) on 512 sampled columns."""
    E, T, k, N, K = 2048, 16384, 8, 4096, 6144
    ids = synth.make_wide_routing(T, E, k, seed=2048)
    counts, off, _ = route_ref(ids, E)
    _, off_dev, _ = gpu_lib.route_prep(ids.cuda(), E)
    assert np.array_equal(off_dev.cpu().numpy(), off)
    A, SA, B, SB = synth.wide_pool_codes(counts.tolist(), N, K, seed=11)
    C = _run(gpu_lib, A, SA, 0, B, SB, off_dev)
    rng = np.random.default_rng(12)
    stream_e = np.nonzero((counts > 0) & (counts <= 64))[0]
    mfma_e = np.nonzero(counts > 64)[0]
    experts = np.concatenate([rng.choice(stream_e, 8, replace=False), rng.choice(mfma_e, 8, replace=False)])
    rows, ex = [], []
    for j, e in enumerate(experts):
        lo, hi = int(off[e]), int(off[e + 1])
        for r in sorted({lo, hi - 1, int(rng.integers(lo, hi))}):
            rows.append(r)
            ex.append(j)
    rows = np.array(rows, dtype=np.int64)
    cols = np.unique(np.concatenate([[0, 63, 64, 511, 512, N - 1], rng.choice(N, 506, replace=False)]))
    rows_t = torch.from_numpy(rows).cuda()
    exp_t = torch.from_numpy(experts).cuda()
    args = (A[rows_t].cpu().numpy(), SA[rows_t].cpu().numpy(), np.array(ex), B[exp_t].cpu().numpy(),
            SB[exp_t].cpu().numpy())
    exact = rows_gemm_f64(*args, cols=cols)
    mag = rows_gemm_f64(*args, cols=cols, absolute=True)
    got = bits_of(C[rows_t][:, torch.from_numpy(cols).cuda()])
    assert_parity(got, bf16_rne_bits(exact), f"wide pool E={E} rows={len(rows)} cols={len(cols)} classes 8+8",
                  exact=exact, abs_sum=mag, K=K, group_eps=GROUP_EPS_RANDOM_CODES)


@pytest.mark.parametrize("layout", [0, 1])
def test_nan_codes_propagate(gpu_lib, layout):
    """E4M3 NaN codes (S.1111.111) planted in some activation rows and E8M0
    0xFF planted in some weight columns' scales, in experts of both classes:
    the output is NaN exactly where the oracle's is (the rows holding a NaN
    code; the columns of an expert whose scale block is NaN, on that expert's
    rows), and every other element meets the parity bar."""
    A, SA, B, SB, off = synth.random_codes_problem(MIXED, 256, 384, 41)
    g = torch.Generator().manual_seed(42)
    R = int(off[-1])
    nan_rows = torch.randint(0, R, (9,), generator=g)
    A[nan_rows, torch.randint(0, 384, (9,), generator=g)] = torch.where(
        torch.arange(9) % 2 == 0, 0x7F, 0xFF).to(torch.uint8)
    E = len(MIXED)
    for e in (1, 4, 5, 9):                       # streaming (5, 1 rows) and MFMA (130, 300) experts
        cols = torch.randint(0, 256, (2,), generator=g)
        SB[e, cols, torch.randint(0, 384 // 32, (2,), generator=g)] = 0xFF
    SA_l = SA if layout == 0 else synth.to_m_major(SA)
    C = _run(gpu_lib, A.cuda(), SA_l.cuda(), layout, B.cuda(), SB.cuda(), off.cuda())
    ex64 = grouped_gemm_f64(A, SA_l.reshape(-1), layout, B, SB, off)
    ref = bf16_rne_bits(ex64)
    got = bits_of(C)
    nan_got = (got & 0x7FFF) > 0x7F80
    nan_ref = (ref & 0x7FFF) > 0x7F80
    print(f"layout={layout}: NaN elements gpu={int(nan_got.sum())} oracle={int(nan_ref.sum())}", flush=True)
    assert nan_ref.sum() > 0
    assert np.array_equal(nan_got, nan_ref)
    keep = ~nan_ref.any(axis=1)
    mag = grouped_gemm_f64(A, SA_l.reshape(-1), layout, B, SB, off, absolute=True)
    assert_parity(got[keep], ref[keep], f"rows without NaN, layout={layout}", exact=ex64[keep], abs_sum=mag[keep],
                  K=384, group_eps=GROUP_EPS_RANDOM_CODES)
