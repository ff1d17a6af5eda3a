"""GPU grouped GEMM over a tile list built beforehand
(w4a8_grouped_gemm_planned).

* With w4a8_plan's own plan it must equal w4a8_grouped_gemm bit for bit on
  the rows of MFMA-class experts (the same tile kernel), and meet the parity
  bar everywhere: streaming items are split differently by the two kernels
  (per-expert column ranges against fixed 512-column items), and a narrow
  item adds its two K halves at the end where a wide one walks K in one
  pass, so the fp32 sums of streaming rows may round differently.
* Over the wide shared expert pools of MoonEP PR #38 (performance table:
  3072 and 6144 experts), beyond the plain GEMM's 2048, rows from the GPU
  route prep: parity with the oracle.
* Plans built by other rules (every expert in the MFMA class, a lower
  streaming cutoff, smaller MFMA tiles): parity with the oracle.
* A plan whose tiles do not lie inside their experts' rows: those tiles
  are skipped (rows they name keep their contents), the rest computed; a
  plan with a nonzero status word writes nothing.
"""

import numpy as np
import pytest
import torch

import synth
from helpers import GROUP_EPS_RANDOM_CODES, assert_parity, bits_of
from oracle import bf16_rne_bits, grouped_gemm_f64, route_ref

pytestmark = pytest.mark.gpu

MIXED = [0, 5, 64, 65, 130, 300, 17, 0, 128, 1, 257]


def host_plan(off, E, N, smax, tmax, gran=16):
    """A plan in w4a8_plan's format under another rule: rows <= smax one
    streaming tile of ceil16(rows), else ceil(rows / tmax) MFMA tiles."""
    stream, mfma = [], []
    for e in range(E):
        rows = int(off[e + 1] - off[e])
        if rows == 0:
            continue
        if rows <= smax:
            stream.append((e, int(off[e]), rows, -(-rows // gran) * gran | (1 << 16)))
            continue
        n = -(-rows // tmax)
        tm = -(-(-(-rows // n)) // gran) * gran
        for i in range(n):
            mfma.append((e, int(off[e]) + i * tm, min(tm, rows - i * tm), tm | (2 << 16)))
    hdr = [0, len(stream) + len(mfma), len(stream), len(mfma), 0, 0, 0, int(off[E])]
    return torch.tensor(hdr + [x for t in stream + mfma for x in t], dtype=torch.int32)


def _case(counts, N, K, seed):
    A, SA, B, SB, off = synth.random_codes_problem(counts, N, K, seed)
    return A, SA, B, SB, off


@pytest.mark.parametrize("layout", [0, 1])
def test_planned_matches_plain(gpu_lib, layout):
    for counts, N, K in [(MIXED, 320, 384), ([5] * 300, 192, 128), ([40] * 3 + [0] + [33] * 2, 1024, 256)]:
        A, SA, B, SB, off = _case(counts, N, K, sum(counts) + N)
        SA_l = (SA if layout == 0 else synth.to_m_major(SA)).cuda()
        d = [t.cuda() for t in (A, B, SB, off)]
        C0 = gpu_lib.grouped_gemm(d[0], SA_l, layout, d[1], d[2], d[3])
        plan = gpu_lib.plan(d[3], len(counts), N, K, max_total_rows=int(off[-1]))
        C1 = gpu_lib.grouped_gemm_planned(d[0], SA_l, layout, d[1], d[2], d[3], plan)
        torch.cuda.synchronize()
        b0, b1 = bits_of(C0), bits_of(C1)
        o = np.asarray(off.cpu().numpy() if hasattr(off, "cpu") else off, dtype=np.int64)
        mfma_rows = np.concatenate([np.arange(o[e], o[e + 1]) for e in range(len(counts))
                                    if o[e + 1] - o[e] > 64] + [np.zeros(0, dtype=np.int64)])
        assert np.array_equal(b0[mfma_rows], b1[mfma_rows]), (counts[:4], N, K)
        ex = grouped_gemm_f64(A, SA_l.cpu().reshape(-1), layout, B, SB, off)
        mag = grouped_gemm_f64(A, SA_l.cpu().reshape(-1), layout, B, SB, off, absolute=True)
        for name, bits in (("plain", b0), ("planned", b1)):
            assert_parity(bits, bf16_rne_bits(ex), f"{name} {counts[:4]} N={N} K={K} layout={layout}",
                          exact=ex, abs_sum=mag, K=K, group_eps=GROUP_EPS_RANDOM_CODES)
        print(f"streaming rows equal bit for bit: {np.array_equal(b0, b1)}", flush=True)


@pytest.mark.parametrize("E,T,skew", [(3072, 16384, False), (6144, 2048, True), (6144, 16384, False)])
def test_planned_wide_pool(gpu_lib, E, T, skew):
    N, K = 256, 256
    ids = synth.make_wide_routing(T, E, 8, seed=E + T, skew=skew)
    counts, off_ref, _ = route_ref(ids, E)
    _, off_dev, _ = gpu_lib.route_prep(ids.cuda(), E)
    assert np.array_equal(off_dev.cpu().numpy(), off_ref)
    A, SA, B, SB, off = synth.random_codes_problem(counts.tolist(), N, K, seed=E + N)
    plan = gpu_lib.plan(off_dev, E, N, K, max_total_rows=int(off[-1]))
    for layout in (0, 1):
        SA_l = SA if layout == 0 else synth.to_m_major(SA)
        C = gpu_lib.grouped_gemm_planned(A.cuda(), SA_l.cuda(), layout, B.cuda(), SB.cuda(), off_dev, plan)
        torch.cuda.synchronize()
        ex = grouped_gemm_f64(A, SA_l.reshape(-1), layout, B, SB, off)
        mag = grouped_gemm_f64(A, SA_l.reshape(-1), layout, B, SB, off, absolute=True)
        assert_parity(bits_of(C), bf16_rne_bits(ex), f"planned E={E} T={T} skew={skew} layout={layout} "
                      f"R={int(off[-1])} max_rows={int(counts.max())}", exact=ex, abs_sum=mag, K=K,
                      group_eps=GROUP_EPS_RANDOM_CODES)


@pytest.mark.parametrize("smax,tmax", [(0, 128), (32, 128), (64, 64), (16, 96), (48, 80)])
def test_planned_other_rules(gpu_lib, smax, tmax):
    counts = MIXED + [33, 48, 49, 96, 97, 112, 113, 200]
    N, K = 288, 384
    A, SA, B, SB, off = _case(counts, N, K, 17)
    plan = host_plan(off.numpy(), len(counts), N, smax, tmax).cuda()
    C = gpu_lib.grouped_gemm_planned(A.cuda(), SA.cuda(), 0, B.cuda(), SB.cuda(), off.cuda(), plan)
    torch.cuda.synchronize()
    ex = grouped_gemm_f64(A, SA.reshape(-1), 0, B, SB, off)
    mag = grouped_gemm_f64(A, SA.reshape(-1), 0, B, SB, off, absolute=True)
    assert_parity(bits_of(C), bf16_rne_bits(ex), f"rule smax={smax} tmax={tmax}", exact=ex, abs_sum=mag, K=K,
                  group_eps=GROUP_EPS_RANDOM_CODES)


def test_planned_skips_tiles_outside_their_expert(gpu_lib):
    counts = [20, 70, 0, 40]
    N, K = 128, 256
    A, SA, B, SB, off = _case(counts, N, K, 5)
    R = int(off[-1])
    good = host_plan(off.numpy(), 4, N, 64, 128)
    bad = good.clone()
    body = bad[8:].view(-1, 4)
    body[0, 1] += 8            # streaming tile of expert 0 shifted past its rows (20 rows from row 8)
    body[1, 0] = 2             # expert 3's tile now claims the empty expert 2
    body[2, 3] = 128 | (1 << 16)   # an MFMA tile labelled streaming
    C = torch.full((R, N), 3.0, dtype=torch.bfloat16, device="cuda")
    gpu_lib.grouped_gemm_planned(A.cuda(), SA.cuda(), 0, B.cuda(), SB.cuda(), off.cuda(), bad.cuda(), out=C)
    torch.cuda.synchronize()
    got = bits_of(C)
    ref = bf16_rne_bits(grouped_gemm_f64(A, SA.reshape(-1), 0, B, SB, off))
    three = bits_of(torch.full((1,), 3.0, dtype=torch.bfloat16))[0]
    assert np.all(got == three)     # every tile of this plan was rejected: nothing written
    bad2 = good.clone()
    bad2.view(-1)[8 + 4 * 1 + 1] += 1   # one streaming tile off by a row; the others stay
    C.fill_(3.0)
    gpu_lib.grouped_gemm_planned(A.cuda(), SA.cuda(), 0, B.cuda(), SB.cuda(), off.cuda(), bad2.cuda(), out=C)
    Cg = gpu_lib.grouped_gemm_planned(A.cuda(), SA.cuda(), 0, B.cuda(), SB.cuda(), off.cuda(), good.cuda())
    torch.cuda.synchronize()
    got, want = bits_of(C), bits_of(Cg)
    lo3, hi3 = int(off[3]), int(off[4])
    assert np.all(got[lo3:hi3] == three)                        # expert 3's tile rejected
    assert np.array_equal(got[:lo3], want[:lo3])                # the other tiles computed as with the good plan
    assert_parity(want, ref, "good host plan", exact=grouped_gemm_f64(A, SA.reshape(-1), 0, B, SB, off),
                  abs_sum=grouped_gemm_f64(A, SA.reshape(-1), 0, B, SB, off, absolute=True), K=K,
                  group_eps=GROUP_EPS_RANDOM_CODES)
    status = good.clone()
    status[0] = 1
    C.fill_(3.0)
    gpu_lib.grouped_gemm_planned(A.cuda(), SA.cuda(), 0, B.cuda(), SB.cuda(), off.cuda(), status.cuda(), out=C)
    torch.cuda.synchronize()
    assert np.all(bits_of(C) == three)
