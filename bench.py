"""Benchmark of the grouped W4A8 MoE GEMM hot path on one MI355X.

One step = routing prep (histogram, offsets, row map) + the grouped GEMM
(whose kernels apply the per-expert tile plan in their prologue) over one
batch of seeded synthetic inputs already resident in HBM.

    python bench.py [--steps K] [--warmup W] [--config NAME|all] [--layout 0|1]

With the default `--config all` one run measures every workload of the
metric: the large prefill gate/up (16384 tokens, M-major scales), the
prefill down projection (1152 tokens, both scale layouts), the four E=12
shapes (8 and 64 tokens, W13 and W2), and last the decode gate/up (64
tokens), whose W warmup steps and K timed steps give the headline value.
Each workload reports the grouped GEMM launch's p10 / median / p90 in us
(HIP events on the launch stream), TFLOP/s, and its roofline: HBM (8 TB/s)
for the weight-streaming shapes, the FP8-rate MFMA peak (5.0 PFLOP/s) for
the prefill shapes, published figures, with both fractions and the HBM
bytes recorded by rocprofv3 counters for this kernel source.  The sustained
peaks measured by the probes go beside them (measured_peak); cpu_baseline =
the CPU oracle timed on a bounded sample of the headline workload.
Prints one JSON line.
"""

from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import re
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0      # MI355X HBM3E, published
MFMA_FP8_PEAK_TFS = 5000.0  # MI355X dense FP8 MFMA, published (FP8 x FP4 runs at this rate)
INFINITY_CACHE_BYTES = 256 << 20

METRIC = "grouped W4A8 GEMM us + TFLOP/s at M=64/1152/16384, % of MFMA/HBM roofline"
HEADLINE = ("decode_gateup", 0)
# the other workloads of the metric, measured after the headline, lightest
# first (the 3 ms prefill gate/up launches, run first, held the next
# workload's clocks down: prefill down read 171-174 us after them, 152 us
# on its own)
SUITE = (("e12_w13_m8", 0), ("e12_w13_m64", 0), ("e12_w2_m8", 0), ("e12_w2_m64", 0),
         ("prefill_down", 0), ("prefill_down", 1), ("prefill_gateup", 1))
BOUND = {"prefill_gateup": "mfma", "prefill_down": "mfma"}
SUITE_WARMUP = 10   # untimed launches before a suite workload's timed ones
SUITE_REPS = 30     # timed launches of a suite workload (at least --steps)

KERNEL_SOURCES = tuple("moe_grouped_precision_amd/csrc/" + f for f in (
    "gemm.hip", "stream_phase.h", "mfma_phase.h", "w4a8_kernel.h", "w4a8_device.h"))


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def kernel_source_hash() -> str:
    h = hashlib.sha256()
    for rel in KERNEL_SOURCES:
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def recorded_traffic(name: str, layout: int):
    """HBM bytes per launch recorded from rocprofv3 counters for this exact
    kernel source (profiles/traffic_<workload>_layout<l>.md); None if absent
    or stale."""
    path = os.path.join(ROOT, "profiles", f"traffic_{name}_layout{layout}.md")
    if not os.path.exists(path):
        return None
    text = open(path).read()
    m_hash = re.search(r"kernel_source_sha256:\s*([0-9a-f]+)", text)
    m_bytes = re.search(r"hbm_bytes_per_launch:\s*([0-9]+)", text)
    if not m_hash or not m_bytes or m_hash.group(1) != kernel_source_hash():
        return None
    return int(m_bytes.group(1))


def copy_calibration(steps: int):
    """A plain 1 GiB device copy, for scaling the memory counters."""
    import torch
    n = 1 << 30
    src = torch.empty(n, dtype=torch.uint8, device="cuda")
    src.fill_(7)
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    for _ in range(steps):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_calibration_bytes_read": n, "copy_calibration_bytes_written": n,
                      "launches": steps}), flush=True)


def algorithmic_bytes(counts, E, N, K):
    """Bytes the GEMM must move: the weights and E8M0 scales of every expert
    with rows, the activation codes and scales, the bf16 output, the offsets."""
    R = int(sum(counts))
    hit = sum(1 for c in counts if c > 0)
    return (hit * N * K * (0.5 + 1.0 / 32) + R * K + R * (K // 128) * 4 + R * N * 2 + 4 * (E + 1))


def pct(xs, q):
    import numpy as np
    return round(float(np.percentile(xs, q)) * 1e3, 2)


def time_launches(fn, reps, warmup=3):
    """Median-able list of ms per launch of fn(i), each between a pair of HIP
    events on the current (launch) stream."""
    import torch
    for i in range(warmup):
        fn(i)
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(reps)]
    torch.cuda.synchronize()
    for i, (a, b) in enumerate(ev):
        a.record()
        fn(i)
        b.record()
    torch.cuda.synchronize()
    return [a.elapsed_time(b) for a, b in ev]


# ---------------------------------------------------------------------------
# the grouped GEMM workloads
# ---------------------------------------------------------------------------
class Workload:
    """One workload's inputs resident in HBM: weights rotated over enough
    copies that timed reads do not come from the 256 MB Infinity Cache."""

    def __init__(self, name, layout, dev):
        import torch
        import synth
        self.name, self.layout = name, layout
        self.cfg = synth.CONFIGS[name]
        # drawn on the GPU (seconds, not minutes, for the large weights)
        p = synth.make_problem(name, device="cuda")
        self.p = p
        self.ids = p.topk_ids.to(dev)
        self.A = p.A.to(dev)
        self.SA = (p.SA if layout == 0 else synth.to_m_major(p.SA)).to(dev)
        weight_bytes = p.B.numel() + p.SB.numel()
        self.nrot = max(1, math.ceil(2 * INFINITY_CACHE_BYTES / weight_bytes) + 1)
        self.Bs = [p.B.to(dev)] + [p.B.to(dev).clone() for _ in range(self.nrot - 1)]
        self.SBs = [p.SB.to(dev)] + [p.SB.to(dev).clone() for _ in range(self.nrot - 1)]
        self.counts_d = torch.empty(p.E, dtype=torch.int32, device=dev)
        self.off_d = torch.empty(p.E + 1, dtype=torch.int32, device=dev)
        self.rows_d = torch.empty(p.R, dtype=torch.int32, device=dev)
        self.C = torch.empty((p.R, p.N), dtype=torch.bfloat16, device=dev)
        torch.cuda.synchronize()

    def route(self):
        import moe_grouped_precision_amd as w4a8
        w4a8.route_prep(self.ids, self.p.E, self.counts_d, self.off_d, self.rows_d)

    def gemm(self, i):
        import moe_grouped_precision_amd as w4a8
        w4a8.grouped_gemm(self.A, self.SA, self.layout, self.Bs[i % self.nrot], self.SBs[i % self.nrot],
                          self.off_d, out=self.C)

    def step(self, i):
        self.route()
        self.gemm(i)

    def describe(self):
        p, cfg = self.p, self.cfg
        lay = "M-major" if self.layout == 1 else "row-major"
        return (f"{self.name}: E={p.E} top_k={p.top_k} tokens={p.T} routed_rows={p.R} N={p.N} K={p.K} "
                f"{cfg['routing']} routing, {lay} input scales")

    def report(self, gemm_ms, probes=None):
        """Per-launch statistics and the roofline of the GEMM launch."""
        import numpy as np
        p = self.p
        counts = self.counts_d.cpu().numpy()
        med = statistics.median(gemm_ms)
        flops = 2.0 * p.R * p.N * p.K
        nbytes = algorithmic_bytes(counts, p.E, p.N, p.K)
        gbs = nbytes / (med * 1e-3) / 1e9
        tfs = flops / (med * 1e-3) / 1e12
        bound = BOUND.get(self.name, "hbm")
        if bound == "hbm":
            roof = {"bound": "hbm", "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                    "frac": round(gbs / HBM_PEAK_GBS, 4), "frac_mfma": round(tfs / MFMA_FP8_PEAK_TFS, 4)}
        else:
            roof = {"bound": "mfma", "achieved": round(tfs, 1), "peak": MFMA_FP8_PEAK_TFS, "unit": "TFLOP/s",
                    "frac": round(tfs / MFMA_FP8_PEAK_TFS, 4), "frac_hbm": round(gbs / HBM_PEAK_GBS, 4)}
        roof["traffic"] = recorded_traffic(self.name, self.layout)
        if probes:
            measured = probes["hbm_read_gbs"] if bound == "hbm" else probes["mfma_fp4xfp8_random_operands_tflops"]
            roof["measured_peak"] = measured
            roof["frac_of_measured"] = round(roof["achieved"] / measured, 4)
        return {
            "workload": self.describe(),
            "experts_with_rows": int((counts > 0).sum()),
            "max_rows_per_expert": int(counts.max()) if len(counts) else 0,
            "gemm_us": {"p10": pct(gemm_ms, 10), "median": round(med * 1e3, 2), "p90": pct(gemm_ms, 90)},
            "launches": len(gemm_ms),
            "tflops": round(tfs, 1),
            "algorithmic_bytes": int(nbytes),
            "flop": flops,
            "weight_copies_rotated": self.nrot,
            "roofline": roof,
        }

    def free(self):
        import torch
        for k in ("A", "SA", "Bs", "SBs", "C", "p"):
            setattr(self, k, None)
        torch.cuda.empty_cache()


def settle(fn, min_ms=20.0, max_launches=4000):
    """Untimed launches of fn(i) until about min_ms of work has run (clocks
    settle); returns the number of launches."""
    import torch
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    n = 0
    a.record()
    while True:
        for i in range(10):
            fn(n + i)
        n += 10
        b.record()
        torch.cuda.synchronize()
        if a.elapsed_time(b) >= min_ms or n >= max_launches:
            return n


def measure_suite_workload(name, layout, dev, reps, probes):
    log(f"{name} layout {layout}: generating")
    w = Workload(name, layout, dev)
    w.route()
    n_settle = settle(w.gemm)
    ms = time_launches(w.gemm, reps, warmup=SUITE_WARMUP)
    out = w.report(ms, probes)
    out["settling_launches"] = n_settle
    log(f"{name} layout {layout}: GEMM median {out['gemm_us']['median']} us, "
        f"{out['roofline']['bound']} frac {out['roofline']['frac']}")
    w.free()
    return out


# ---------------------------------------------------------------------------
# the CPU oracle beside it
# ---------------------------------------------------------------------------
def blas_info():
    """BLAS backend and thread count numpy's dgemm uses here."""
    try:
        from threadpoolctl import threadpool_info
        for d in threadpool_info():
            if d.get("user_api") == "blas":
                return f"{d.get('internal_api')} {d.get('version')}", int(d.get("num_threads"))
    except Exception:  # noqa: BLE001 -- the report is informational
        pass
    return "unknown", None


def cpu_baseline(p, off, layout, budget_s=20.0, min_s=10.0):
    """Time the oracle on a bounded sample of the workload: whole experts in
    order (at most 2048 rows of each) until about budget_s seconds of CPU
    work; a sample that finishes sooner (a decode-sized workload takes about
    2 s) is repeated until min_s seconds have passed.  Scaled to TFLOP/s."""
    import numpy as np
    from oracle import grouped_gemm_bf16

    A = p.A.cpu().numpy()
    SA = p.SA.cpu().numpy()
    B = p.B.cpu().numpy()
    SB = p.SB.cpu().numpy()
    flops = 0.0
    experts = 0
    rows_done = 0
    passes = 0
    t0 = time.perf_counter()
    done = False
    while not done:
        passes += 1
        for e in range(p.E):
            lo, hi = int(off[e]), int(off[e + 1])
            if hi == lo:
                continue
            hi = min(hi, lo + 2048)  # cap the rows of one expert in the sample
            sa = SA[lo:hi]
            sa_l = sa.T.copy().reshape(-1) if layout == 1 else sa.reshape(-1)
            grouped_gemm_bf16(A[lo:hi], sa_l, layout, B[e:e + 1], SB[e:e + 1],
                              np.array([0, hi - lo], dtype=np.int32))
            flops += 2.0 * (hi - lo) * p.N * p.K
            if passes == 1:
                experts += 1
                rows_done += hi - lo
            if time.perf_counter() - t0 > budget_s:
                done = True
                break
        if time.perf_counter() - t0 >= min_s:
            done = True
    dt = time.perf_counter() - t0
    try:
        cores = len(os.sched_getaffinity(0))
    except AttributeError:
        cores = os.cpu_count()
    blas, threads = blas_info()
    return {"value": flops / dt / 1e12, "unit": "TFLOP/s", "cores": cores, "kind": "oracle",
            "blas": blas, "blas_threads": threads,
            "sample": f"{experts} experts, {rows_done} rows (<=2048 per expert) of the same "
                      f"workload, {passes} pass(es), numpy fp64 oracle (dgemm per expert), {dt:.1f} s"}


# ---------------------------------------------------------------------------
# the entry points around the GEMM
# ---------------------------------------------------------------------------
def _hbm_result(workload, ms, nbytes, **extra):
    med = statistics.median(ms)
    gbs = nbytes / (med * 1e-3) / 1e9
    out = {"workload": workload, "us_median": round(med * 1e3, 2), "us_p10_p90": [pct(ms, 10), pct(ms, 90)],
           "algorithmic_bytes": int(nbytes)}
    out.update(extra)
    out["roofline"] = {"bound": "hbm", "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                       "frac": round(gbs / HBM_PEAK_GBS, 4)}
    return out


def _rotations(nbytes):
    """Copies of a working set needed so that it spans twice the Infinity Cache."""
    return max(1, math.ceil(2 * INFINITY_CACHE_BYTES / max(nbytes, 1)) + 1)


def measure_quantize_gather(reps=20):
    """The activation quantizer with gather (w4a8_quantize_gather) on the large
    prefill activations: 16384 bf16 tokens x 6144, top-8 biased routing over 32
    experts, M-major scales."""
    import torch

    import moe_grouped_precision_amd as w4a8
    import synth

    cfg = synth.CONFIGS["prefill_gateup"]
    T, K, E, k = cfg["T"], cfg["K"], cfg["E"], cfg["top_k"]
    g = torch.Generator(device="cuda").manual_seed(17)
    x = torch.randn((T, K), generator=g, device="cuda", dtype=torch.float32).to(torch.bfloat16)
    ids = synth.make_routing(cfg["routing"], T, E, k, cfg["seed"]).to("cuda")
    _, off, ros = w4a8.route_prep(ids, E)
    R = int(off[-1].item())
    G = K // 128
    A = torch.empty((R, K), dtype=torch.uint8, device="cuda")
    SA = torch.empty((G, R), dtype=torch.float32, device="cuda")
    ms = time_launches(lambda i: w4a8.quantize_gather(x, ros, k, R, 1, A=A, SA=SA), reps)
    nbytes = T * K * 2 + 4 * T * k + R * K + 4 * R * G
    return _hbm_result(f"{T} bf16 tokens x {K}, top-{k} {cfg['routing']} routing over {E} experts "
                       f"({R} rows), M-major scales", ms, nbytes)


def measure_combine(reps=20):
    """The top-k combine (w4a8_combine) on the prefill down-projection output:
    1152 tokens, top-8 biased routing over 32 experts, 6144 bf16 columns.
    Inputs and outputs rotate over enough copies to span twice the Infinity
    Cache, so the reads come from HBM."""
    import torch

    import moe_grouped_precision_amd as w4a8
    import synth

    cfg = synth.CONFIGS["prefill_down"]
    T, N, E, k = cfg["T"], cfg["N"], cfg["E"], cfg["top_k"]
    g = torch.Generator(device="cuda").manual_seed(19)
    ids = synth.make_routing(cfg["routing"], T, E, k, cfg["seed"]).to("cuda")
    _, off, ros = w4a8.route_prep(ids, E)
    R = int(off[-1].item())
    nbytes = R * N * 2 + T * N * 2 + 8 * T * k
    nrot = _rotations(nbytes)
    C0 = torch.randn((R, N), generator=g, device="cuda", dtype=torch.float32).to(torch.bfloat16)
    Cs = [C0] + [C0.clone() for _ in range(nrot - 1)]
    outs = [torch.empty((T, N), dtype=torch.bfloat16, device="cuda") for _ in range(nrot)]
    w = torch.rand((T * k,), generator=g, device="cuda", dtype=torch.float32)
    ms = time_launches(lambda i: w4a8.combine(Cs[i % nrot], ros, w, k, out=outs[i % nrot]), reps)
    return _hbm_result(f"{T} tokens x top-{k} rows of {N} bf16 columns ({R} rows), {cfg['routing']} routing "
                       f"over {E} experts", ms, nbytes, copies_rotated=nrot)


def measure_swiglu_quant(reps=20):
    """SwiGLU + E4M3 requantization (w4a8_swiglu_quant) on the large prefill
    gate/up output: 131072 rows x (2 x 2048) bf16, M-major scales."""
    import torch

    import moe_grouped_precision_amd as w4a8

    R, I = 131072, 2048
    g = torch.Generator(device="cuda").manual_seed(23)
    C = (torch.randn((R, 2 * I), generator=g, device="cuda") * 3).to(torch.bfloat16)
    A = torch.empty((R, I), dtype=torch.uint8, device="cuda")
    SA = torch.empty((I // 128, R), dtype=torch.float32, device="cuda")
    ms = time_launches(lambda i: w4a8.swiglu_quant(C, 1, A=A, SA=SA), reps)
    nbytes = R * 2 * I * 2 + R * I + 4 * R * (I // 128)
    return _hbm_result(f"{R} rows x (2 x {I}) bf16 gate/up output, M-major scales", ms, nbytes)


def measure_route_prep_wide(reps=20):
    """The routing prep (w4a8_route_prep) on a wide shared expert pool: 6144
    experts, 16384 tokens, top-8, uniform without replacement (the largest
    pool MoonEP PR #38 times).  Every workgroup reads all ids from L2, so
    the kernel is bound by that latency, not by HBM; the HBM roofline on the
    bytes it must move is reported for completeness."""
    import torch

    import moe_grouped_precision_amd as w4a8
    import synth

    E, T, k = 6144, 16384, 8
    ids = synth.make_wide_routing(T, E, k, seed=6144).to("cuda")
    c = torch.empty(E, dtype=torch.int32, device="cuda")
    o = torch.empty(E + 1, dtype=torch.int32, device="cuda")
    r = torch.empty(T * k, dtype=torch.int32, device="cuda")
    ms = time_launches(lambda i: w4a8.route_prep(ids, E, c, o, r), reps)
    lds = torch.cuda.get_device_properties(0).shared_memory_per_block
    out = _hbm_result(f"{T} tokens x top-{k} over {E} experts, uniform routing", ms, 8 * T * k + 8 * E + 4,
                      ranking_waves=w4a8.route_prep_waves(E, lds), lds_limit_bytes=int(lds))
    out["roofline"]["bound"] = "latency (every workgroup reads all ids from L2)"
    return out


def measure_gemm_wide_pool(reps=5):
    """The grouped GEMM over a 2048-expert pool (the 2048-expert shape of
    MoonEP PR #38's performance table, 16384 tokens at top-8, uniform routing)
    at the benchmark's gate/up expert shape N=4096, K=6144 (humming PR #129
    "Results"), random codes drawn on the GPU.  Every expert gets rows, so
    the 27 GB of weights are read once and the launch is HBM-bound (about
    225 flop per byte, below the MFMA ridge)."""
    import torch

    import moe_grouped_precision_amd as w4a8
    import synth

    E, T, k, N, K = 2048, 16384, 8, 4096, 6144
    ids = synth.make_wide_routing(T, E, k, seed=2048).to("cuda")
    counts, off, _ = w4a8.route_prep(ids, E)
    counts = counts.cpu().numpy()
    R = int(counts.sum())
    A, SA, B, SB = synth.wide_pool_codes(counts.tolist(), N, K, seed=11)
    C = torch.empty((R, N), dtype=torch.bfloat16, device="cuda")
    ms = time_launches(lambda i: w4a8.grouped_gemm(A, SA, 0, B, SB, off, out=C), reps, warmup=2)
    hit = int((counts > 0).sum())
    flops = 2.0 * R * N * K
    out = _hbm_result(f"{T} tokens x top-{k} over {E} experts ({hit} with rows, at most {int(counts.max())} "
                      f"rows), N={N} K={K}, uniform routing, row-major scales", ms,
                      algorithmic_bytes(counts, E, N, K), flop=flops,
                      tflops=round(flops / (statistics.median(ms) * 1e-3) / 1e12, 1))
    del A, SA, B, SB, C
    torch.cuda.empty_cache()
    return out


def measure_gemm_planned_wide_pool(reps=5, E=6144):
    """The grouped GEMM over the largest shared pool MoonEP PR #38 times (6144
    experts, 16384 tokens at top-8, uniform routing) at the benchmark's
    gate/up expert shape N=4096, K=6144, beyond the plain GEMM's per-expert
    tables: w4a8_plan once, then w4a8_grouped_gemm_planned (timed).  Random
    codes drawn on the GPU; about 82 GB of weights, read once per launch."""
    import torch

    import moe_grouped_precision_amd as w4a8
    import synth

    T, k, N, K = 16384, 8, 4096, 6144
    ids = synth.make_wide_routing(T, E, k, seed=E).to("cuda")
    counts, off, _ = w4a8.route_prep(ids, E)
    counts = counts.cpu().numpy()
    R = int(counts.sum())
    A, SA, B, SB = synth.wide_pool_codes(counts.tolist(), N, K, seed=13)
    C = torch.empty((R, N), dtype=torch.bfloat16, device="cuda")
    plan = w4a8.plan(off, E, N, K, max_total_rows=R)
    ms_plan = time_launches(lambda i: w4a8.plan(off, E, N, K, out=plan), 10)
    ms = time_launches(lambda i: w4a8.grouped_gemm_planned(A, SA, 0, B, SB, off, plan, out=C), reps, warmup=2)
    hit = int((counts > 0).sum())
    flops = 2.0 * R * N * K
    out = _hbm_result(f"{T} tokens x top-{k} over {E} experts ({hit} with rows, at most {int(counts.max())} "
                      f"rows), N={N} K={K}, uniform routing, row-major scales, plan built once", ms,
                      algorithmic_bytes(counts, E, N, K), flop=flops,
                      tflops=round(flops / (statistics.median(ms) * 1e-3) / 1e12, 1),
                      plan_us_median=round(statistics.median(ms_plan) * 1e3, 2))
    del A, SA, B, SB, C
    torch.cuda.empty_cache()
    return out


def measure_gemm_a16(fmt, name="decode_gateup", reps=30):
    """The grouped GEMM with bf16 activations and FP4 weights
    (w4a8_grouped_gemm_a16) on a workload's shapes and routing: bf16 N(0,1)
    activations, N(0, 0.02) weights quantized to MXFP4 (fmt 0) or NVFP4 (fmt
    1, with a per-expert tensor scale), weights rotated past the Infinity
    Cache.  HBM roofline on the bytes the launch must move."""
    import torch

    import moe_grouped_precision_amd as w4a8
    import synth

    p = synth.make_a16_problem(name, fmt, device="cuda")
    counts, off, _ = w4a8.route_prep(p.topk_ids.to("cuda"), p.E)
    counts = counts.cpu().numpy()
    wbytes = p.B.numel() + p.SB.numel()
    nrot = _rotations(wbytes)
    Bs = [p.B] + [p.B.clone() for _ in range(nrot - 1)]
    SBs = [p.SB] + [p.SB.clone() for _ in range(nrot - 1)]
    GS = p.GS if fmt == 1 else None
    C = torch.empty((p.R, p.N), dtype=torch.bfloat16, device="cuda")
    ms = time_launches(lambda i: w4a8.grouped_gemm_a16(p.A, Bs[i % nrot], SBs[i % nrot], fmt, off, GS, out=C),
                       reps, warmup=10)
    hit = int((counts > 0).sum())
    blk = 32 if fmt == 0 else 16
    nbytes = hit * p.N * p.K * (0.5 + 1.0 / blk) + p.R * p.K * 2 + p.R * p.N * 2 + 4 * (p.E + 1) + 4 * p.E * fmt
    flops = 2.0 * p.R * p.N * p.K
    cfg = p.name
    out = _hbm_result(f"{cfg}: E={p.E} top_k={p.top_k} tokens={p.T} routed_rows={p.R} N={p.N} K={p.K}, bf16 "
                      f"activations, {'MXFP4 (E8M0 per 32)' if fmt == 0 else 'NVFP4 (E4M3 per 16, fp32 per expert)'}"
                      f" weights", ms, nbytes, flop=flops,
                      tflops=round(flops / (statistics.median(ms) * 1e-3) / 1e12, 1), weight_copies_rotated=nrot)
    del Bs, SBs, C
    torch.cuda.empty_cache()
    return out


def measure_gemm_swiglu(reps=10):
    """The gate/up GEMM with the SwiGLU + E4M3 requantization epilogue
    (w4a8_grouped_gemm_swiglu) on the large prefill gate/up workload (16384
    tokens, top-8 biased routing over 32 experts, N = 2I = 4096, K = 6144,
    M-major scales in and out), beside the same inputs through the plain
    GEMM followed by w4a8_swiglu_quant.  MFMA roofline on 2 R N K."""
    import torch

    import moe_grouped_precision_amd as w4a8

    w = Workload("prefill_gateup", 1, torch.device("cuda:0"))
    w.route()
    p = w.p
    I = p.N // 2
    A2 = torch.empty((p.R, I), dtype=torch.uint8, device="cuda")
    SA2 = torch.empty((I // 128, p.R), dtype=torch.float32, device="cuda")

    def fused(i):
        w4a8.grouped_gemm_swiglu(w.A, w.SA, 1, w.Bs[i % w.nrot], w.SBs[i % w.nrot], w.off_d, 1, A2=A2, SA2=SA2)

    def unfused(i):
        w.gemm(i)
        w4a8.swiglu_quant(w.C, 1, A=A2, SA=SA2)

    ms = time_launches(fused, reps, warmup=3)
    ms_u = time_launches(unfused, reps, warmup=3)
    counts = w.counts_d.cpu().numpy()
    flops = 2.0 * p.R * p.N * p.K
    med = statistics.median(ms)
    tfs = flops / (med * 1e-3) / 1e12
    hit = int((counts > 0).sum())
    nbytes = hit * p.N * p.K * (0.5 + 1 / 32) + p.R * p.K * (1 + 4 / 128) + p.R * I * (1 + 4 / 128) + 4 * (p.E + 1)
    out = {"workload": w.describe() + ", SwiGLU + E4M3 requantization (M-major scales) in the epilogue",
           "us_median": round(med * 1e3, 2), "us_p10_p90": [pct(ms, 10), pct(ms, 90)],
           "unfused_gemm_plus_swiglu_quant_us_median": round(statistics.median(ms_u) * 1e3, 2),
           "algorithmic_bytes": int(nbytes), "flop": flops, "tflops": round(tfs, 1),
           "roofline": {"bound": "mfma", "achieved": round(tfs, 1), "peak": MFMA_FP8_PEAK_TFS, "unit": "TFLOP/s",
                        "frac": round(tfs / MFMA_FP8_PEAK_TFS, 4)}}
    w.free()
    return out


# ---------------------------------------------------------------------------
# dense sweep of the tile rule's constants
# ---------------------------------------------------------------------------
SWEEP_SHAPES = {"gateup": (4096, 6144), "down": (6144, 2048)}
SWEEP_TILES = (64, 80, 96, 112, 128)   # MFMA m-tile caps tried (the kernel's largest tile is 128 rows)


def sweep_plan(E, rows, cls, tmax, N):
    """A plan in w4a8_plan's format for E experts of `rows` rows each, every
    expert in class `cls` (1 streaming, 2 MFMA with m-tiles of at most tmax
    rows, sized as the tile rule sizes them)."""
    import torch
    body = []
    for e in range(E):
        r0 = e * rows
        if cls == 1:
            body += [e, r0, rows, -(-rows // 16) * 16 | (1 << 16)]
        else:
            n = -(-rows // tmax)
            tm = -(-(-(-rows // n)) // 16) * 16
            for i in range(n):
                body += [e, r0 + i * tm, min(tm, rows - i * tm), tm | (2 << 16)]
    tiles = len(body) // 4
    ns = tiles if cls == 1 else 0
    hdr = [0, tiles, ns, tiles - ns, 0, 0, 0, E * rows]
    return torch.tensor(hdr + body, dtype=torch.int32, device="cuda")


def sweep_tiles(rows_list, layouts, reps=10, E=32):
    """Rows per expert from rows_list (uniform experts, E of them), the two
    benchmark expert shapes (gate/up N=4096 K=6144, down N=6144 K=2048) and
    the given scale layouts: the grouped GEMM timed (median of `reps`
    launches, HIP events) with every expert in the streaming class (rows <=
    64, the most that class serves) and in the MFMA class with each m-tile
    cap of SWEEP_TILES, through w4a8_grouped_gemm_planned and plans built
    here.  Random codes drawn on the GPU; weights rotated past the Infinity
    Cache.  One JSON line per (shape, layout, rows)."""
    import torch

    import moe_grouped_precision_amd as w4a8

    for shape, (N, K) in SWEEP_SHAPES.items():
        Rmax = E * max(rows_list)
        g = torch.Generator(device="cuda").manual_seed(29)
        A = torch.randint(0, 256, (Rmax, K), generator=g, dtype=torch.uint8, device="cuda")
        A[(A & 0x7F) == 0x7F] = 0x38
        SA0 = torch.rand((Rmax, K // 128), generator=g, device="cuda") * 4 + 0.01
        wbytes = E * N * K * 17 // 32
        nrot = _rotations(wbytes)
        Bs = [torch.randint(0, 256, (E, N, K // 2), generator=g, dtype=torch.uint8, device="cuda")
              for _ in range(nrot)]
        SBs = [torch.randint(112, 132, (E, N, K // 32), generator=g, dtype=torch.uint8, device="cuda")
               for _ in range(nrot)]
        for layout in layouts:
            for rows in rows_list:
                R = E * rows
                off = torch.arange(0, E + 1, dtype=torch.int32, device="cuda") * rows
                SA = SA0[:R].contiguous() if layout == 0 else SA0[:R].t().contiguous()
                C = torch.empty((R, N), dtype=torch.bfloat16, device="cuda")
                cands = ([("stream", sweep_plan(E, rows, 1, 0, N))] if rows <= 64 else []) + \
                        [(f"mfma_t{t}", sweep_plan(E, rows, 2, t, N)) for t in SWEEP_TILES]
                res = {}
                for name, plan in cands:
                    ms = time_launches(lambda i: w4a8.grouped_gemm_planned(
                        A[:R], SA, layout, Bs[i % nrot], SBs[i % nrot], off, plan, out=C), reps)
                    res[name] = round(statistics.median(ms) * 1e3, 2)
                best = min(res, key=res.get)
                print(json.dumps({"shape": shape, "N": N, "K": K, "E": E, "layout": layout, "rows": rows,
                                  "us": res, "best": best}), flush=True)
        del A, SA0, Bs, SBs
        torch.cuda.empty_cache()


# ---------------------------------------------------------------------------
def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=None)
    ap.add_argument("--warmup", type=int, default=None)
    ap.add_argument("--config", default="all",
                    help="'all' (every workload of the metric, decode gate/up as the headline) or one workload")
    ap.add_argument("--layout", type=int, default=None, help="0 row-major, 1 M-major input scales")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-budget", type=float, default=20.0)
    ap.add_argument("--no-probes", action="store_true",
                    help="skip the measured-peak probes (MFMA rate, HBM read bandwidth)")
    ap.add_argument("--no-extras", "--no-quantize", dest="no_extras", action="store_true",
                    help="skip the quantizer, SwiGLU-requantization, combine and wide-pool "
                         "routing-prep and GEMM measurements")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a plain 1 GiB copy (memory-counter calibration)")
    ap.add_argument("--sweep-tiles", action="store_true",
                    help="only run the dense sweep of the tile rule (rows per expert 8..512 step 8, both "
                         "classes and every MFMA m-tile cap, gate/up and down shapes, both layouts)")
    args = ap.parse_args()

    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported "
              "(the path has no multi-GPU component)", file=sys.stderr)
        sys.exit(2)

    if args.copy_calibration:
        copy_calibration(args.steps or 5)
        return
    if args.sweep_tiles:
        import moe_grouped_precision_amd as w4a8
        w4a8.load()
        sweep_tiles(list(range(8, 513, 8)), (0, 1) if args.layout is None else (args.layout,))
        return

    import numpy as np
    import torch

    import moe_grouped_precision_amd as w4a8

    suite = args.config == "all"
    name = HEADLINE[0] if suite else args.config
    layout = args.layout if args.layout is not None else (
        HEADLINE[1] if suite else (1 if name == "prefill_gateup" else 0))
    steps = args.steps if args.steps is not None else (20 if name == "prefill_gateup" else 50)
    warmup = args.warmup if args.warmup is not None else (50 if name == "prefill_gateup" else 200)
    w4a8.load()
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)

    # the headline workload first, on a device that has run nothing else yet
    # (later workloads allocate and free tens of GB): untimed GEMM launches
    # until about 20 ms of work has run so that clocks settle (W = 5 steps are
    # 0.4 ms), then W untimed warmup steps, then exactly K timed steps
    log(f"{name} layout {layout}: generating")
    w = Workload(name, layout, dev)
    log(f"inputs resident: R={w.p.R} N={w.p.N} K={w.p.K} E={w.p.E}, {w.nrot} weight copies")
    w.route()
    n_settle = settle(w.gemm)
    for i in range(warmup):
        w.step(i)
    torch.cuda.synchronize()
    log(f"{n_settle} settling launches, warmup done ({warmup} steps)")
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0.record()
    for i in range(steps):
        w.step(i)
    t1.record()
    torch.cuda.synchronize()
    ms_per_step = t0.elapsed_time(t1) / steps
    # per-launch timing of the grouped GEMM call, on the stream it is launched
    # on, launches queued back to back (the routing prep's offsets do not
    # change between steps; with a prep before every launch the host's two
    # calls per step outlast the E=12 launches and the events would time
    # the host)
    gemm_ms = time_launches(w.gemm, max(steps, 20), warmup=0)
    log(f"timed {steps} steps: {ms_per_step * 1e3:.1f} us/step, gemm median "
        f"{statistics.median(gemm_ms) * 1e3:.2f} us")

    probes = None
    if not args.no_probes:
        from moe_grouped_precision_amd import probe
        log("measuring sustained peaks (MFMA fp4 x fp8, HBM read)")
        probes = {"mfma_fp4xfp8_tflops": round(probe.mfma_tflops(4, 0), 1),
                  "mfma_fp4xfp8_random_operands_tflops": round(probe.mfma_tflops_random(4, 0), 1),
                  "mfma_fp4xfp8_zero_acc_tflops": round(probe.mfma_promote_tflops(False), 1),
                  "mfma_fp4xfp8_zero_acc_promote_tflops": round(probe.mfma_promote_tflops(True), 1),
                  "hbm_read_gbs": round(probe.read_gbs(), 1)}
    head = w.report(gemm_ms, probes)
    head["settling_launches"] = n_settle
    p_head, off_head = w.p, w.off_d.cpu().numpy()
    w.free()

    configs = {}
    if suite:
        for sname, slayout in SUITE:
            configs[f"{sname}_layout{slayout}"] = measure_suite_workload(
                sname, slayout, dev, max(SUITE_REPS, steps), probes)

    extras = {}
    if not args.no_extras:
        log("timing the fused gate/up + SwiGLU GEMM, the A16 GEMMs, the activation quantizer, SwiGLU requantization, "
            "the top-k combine, the routing prep over 6144 experts and the GEMM over 2048 experts")
        extras = {"grouped_gemm_swiglu": measure_gemm_swiglu(),
                  "grouped_gemm_a16_mxfp4": measure_gemm_a16(0), "grouped_gemm_a16_nvfp4": measure_gemm_a16(1),
                  "grouped_gemm_a16_mxfp4_e12_w2_m8": measure_gemm_a16(0, "e12_w2_m8"),
                  "grouped_gemm_a16_nvfp4_e12_w2_m8": measure_gemm_a16(1, "e12_w2_m8"),
                  "quantize_gather": measure_quantize_gather(), "swiglu_quant": measure_swiglu_quant(),
                  "combine": measure_combine(), "route_prep_wide_pool": measure_route_prep_wide(),
                  "grouped_gemm_wide_pool": measure_gemm_wide_pool(),
                  "grouped_gemm_planned_wide_pool": measure_gemm_planned_wide_pool()}

    cpu = None
    if not args.no_cpu_baseline:
        log("timing the CPU oracle on a bounded sample")
        cpu = cpu_baseline(p_head, off_head, layout, args.cpu_budget)

    p = p_head
    flops = 2.0 * p.R * p.N * p.K
    config = {"workload": head["workload"]}
    config.update({k: v for k, v in head.items() if k not in ("workload", "roofline")})
    config["kernel_source_sha256"] = kernel_source_hash()
    out = {
        "metric": METRIC,
        "value": round(flops / (ms_per_step * 1e-3) / 1e12, 3),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": steps,
        "warmup": warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp8e4m3 x fp4e2m1 (fp32 accumulate, bf16 out)",
        "data": "synthetic",
        "config": config,
        "roofline": head["roofline"],
        "configs": configs or None,
        "probes": probes,
        "cpu_baseline": cpu,
    }
    out.update(extras)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
