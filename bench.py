"""Benchmark of the grouped W4A8 MoE GEMM hot path on one MI355X.

One step = routing prep (histogram, offsets, row map) + the grouped GEMM
(whose kernels apply the per-expert tile plan in their prologue) over one
batch of seeded synthetic inputs already resident in HBM.

    python bench.py [--steps K] [--warmup W] [--config NAME] [--layout 0|1]

Prints one JSON line.  value = whole-step TFLOP/s (2*R*N*K per step);
roofline = the grouped GEMM kernel launch against HBM (8 TB/s) or the
FP8-rate MFMA peak (5.0 PFLOP/s), published figures, with the sustained
peaks measured by the probes beside them (measured_peak); cpu_baseline = the
CPU oracle timed on a bounded sample of the same workload.
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

DEFAULT_STEPS = {"prefill_gateup": 20}
# untimed steps before the timed region: enough continuous work (about 20 ms
# on decode, 160 ms on the large prefill) for the GPU clocks to settle; with
# 10 warmup steps the first ~10 ms of timed decode steps ran 8% slower
DEFAULT_WARMUP = {"prefill_gateup": 50}
BOUND = {"prefill_gateup": "mfma", "prefill_down": "mfma"}


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
    kernel source (profiles/traffic_<workload>.md); None if absent or stale."""
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
    R = int(sum(counts))
    hit = sum(1 for c in counts if c > 0)
    return (hit * N * K * (0.5 + 1.0 / 32) + R * K + R * (K // 128) * 4 + R * N * 2 + 4 * (E + 1))


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
            if layout == 1:
                sa_l = sa.T.copy().reshape(-1)
            else:
                sa_l = sa.reshape(-1)
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
    return {"value": flops / dt / 1e12, "unit": "TFLOP/s", "cores": cores, "kind": "oracle",
            "sample": f"{experts} experts, {rows_done} rows (<=2048 per expert) of the same "
                      f"workload, {passes} pass(es), numpy fp64 oracle, {dt:.1f} s"}


def measure_quantize_gather(reps=20, warmup=3):
    """The activation quantizer with gather (w4a8_quantize_gather) on the large
    prefill activations: 16384 bf16 tokens x 6144, top-8 biased routing over 32
    experts, M-major scales.  Median of `reps` launches timed with HIP events
    on the launch stream; HBM roofline on the bytes it must move."""
    import numpy as np
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
    for _ in range(warmup):
        w4a8.quantize_gather(x, ros, k, R, 1, A=A, SA=SA)
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(reps)]
    torch.cuda.synchronize()
    for a, b in ev:
        a.record()
        w4a8.quantize_gather(x, ros, k, R, 1, A=A, SA=SA)
        b.record()
    torch.cuda.synchronize()
    ms = statistics.median([a.elapsed_time(b) for a, b in ev])
    nbytes = T * K * 2 + 4 * T * k + R * K + 4 * R * G
    gbs = nbytes / (ms * 1e-3) / 1e9
    return {"workload": f"{T} bf16 tokens x {K}, top-{k} {cfg['routing']} routing over {E} experts "
                        f"({R} rows), M-major scales",
            "us_median": round(ms * 1e3, 2), "algorithmic_bytes": int(nbytes),
            "roofline": {"bound": "hbm", "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                         "frac": round(gbs / HBM_PEAK_GBS, 4)}}


def measure_combine(reps=20, warmup=3):
    """The top-k combine (w4a8_combine) on the prefill down-projection output:
    1152 tokens, top-8 biased routing over 32 experts, 6144 bf16 columns.
    Median of `reps` launches timed with HIP events on the launch stream; HBM
    roofline on the bytes it must move."""
    import torch

    import moe_grouped_precision_amd as w4a8
    import synth

    cfg = synth.CONFIGS["prefill_down"]
    T, N, E, k = cfg["T"], cfg["N"], cfg["E"], cfg["top_k"]
    g = torch.Generator(device="cuda").manual_seed(19)
    ids = synth.make_routing(cfg["routing"], T, E, k, cfg["seed"]).to("cuda")
    _, off, ros = w4a8.route_prep(ids, E)
    R = int(off[-1].item())
    C = torch.randn((R, N), generator=g, device="cuda", dtype=torch.float32).to(torch.bfloat16)
    w = torch.rand((T * k,), generator=g, device="cuda", dtype=torch.float32)
    out = torch.empty((T, N), dtype=torch.bfloat16, device="cuda")
    for _ in range(warmup):
        w4a8.combine(C, ros, w, k, out=out)
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(reps)]
    torch.cuda.synchronize()
    for a, b in ev:
        a.record()
        w4a8.combine(C, ros, w, k, out=out)
        b.record()
    torch.cuda.synchronize()
    ms = statistics.median([a.elapsed_time(b) for a, b in ev])
    nbytes = R * N * 2 + T * N * 2 + 8 * T * k
    gbs = nbytes / (ms * 1e-3) / 1e9
    return {"workload": f"{T} tokens x top-{k} rows of {N} bf16 columns ({R} rows), {cfg['routing']} routing "
                        f"over {E} experts",
            "us_median": round(ms * 1e3, 2), "algorithmic_bytes": int(nbytes),
            "roofline": {"bound": "hbm", "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                         "frac": round(gbs / HBM_PEAK_GBS, 4)}}


def measure_route_prep_wide(reps=20, warmup=3):
    """The routing prep (w4a8_route_prep) on a wide shared expert pool: 6144
    experts, 16384 tokens, top-8, uniform without replacement (the largest
    pool MoonEP PR #38 times).  Median of `reps` launches timed with HIP
    events on the launch stream.  Every workgroup reads all ids from L2, so
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
    for _ in range(warmup):
        w4a8.route_prep(ids, E, c, o, r)
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(reps)]
    torch.cuda.synchronize()
    for a, b in ev:
        a.record()
        w4a8.route_prep(ids, E, c, o, r)
        b.record()
    torch.cuda.synchronize()
    ms = statistics.median([a.elapsed_time(b) for a, b in ev])
    lds = torch.cuda.get_device_properties(0).shared_memory_per_block
    nbytes = 8 * T * k + 8 * E + 4
    gbs = nbytes / (ms * 1e-3) / 1e9
    return {"workload": f"{T} tokens x top-{k} over {E} experts, uniform routing",
            "us_median": round(ms * 1e3, 2), "ranking_waves": w4a8.route_prep_waves(E, lds),
            "lds_limit_bytes": int(lds), "algorithmic_bytes": int(nbytes),
            "roofline": {"bound": "latency (every workgroup reads all ids from L2)", "achieved": round(gbs, 1),
                         "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": round(gbs / HBM_PEAK_GBS, 4)}}


def measure_gemm_wide_pool(reps=5, warmup=2):
    """The grouped GEMM over a 2048-expert pool (the 2048-expert shape of
    MoonEP PR #38's performance table, 16384 tokens at top-8, uniform routing)
    at the benchmark's gate/up expert shape N=4096, K=6144 (humming PR #129
    "Results"), random codes drawn on the GPU.  Every expert gets rows, so
    the 27 GB of weights are read once and the launch is HBM-bound (about
    225 flop per byte, below the MFMA ridge).  Median of `reps` launches timed
    with HIP events on the launch stream."""
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
    for _ in range(warmup):
        w4a8.grouped_gemm(A, SA, 0, B, SB, off, out=C)
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(reps)]
    torch.cuda.synchronize()
    for a, b in ev:
        a.record()
        w4a8.grouped_gemm(A, SA, 0, B, SB, off, out=C)
        b.record()
    torch.cuda.synchronize()
    ms = statistics.median([a.elapsed_time(b) for a, b in ev])
    hit = int((counts > 0).sum())
    nbytes = hit * N * K * (1 / 2 + 1 / 32) + R * K + R * (K // 128) * 4 + R * N * 2 + 4 * (E + 1)
    flops = 2.0 * R * N * K
    gbs = nbytes / (ms * 1e-3) / 1e9
    out = {"workload": f"{T} tokens x top-{k} over {E} experts ({hit} with rows, at most {int(counts.max())} rows), "
                       f"N={N} K={K}, uniform routing, row-major scales",
           "us_median": round(ms * 1e3, 1), "algorithmic_bytes": int(nbytes), "flop": flops,
           "tflops": round(flops / (ms * 1e-3) / 1e12, 1),
           "roofline": {"bound": "hbm", "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                        "frac": round(gbs / HBM_PEAK_GBS, 4)}}
    del A, SA, B, SB, C
    torch.cuda.empty_cache()
    return out


def measure_swiglu_quant(reps=20, warmup=3):
    """SwiGLU + E4M3 requantization (w4a8_swiglu_quant) on the large prefill
    gate/up output: 131072 rows x (2 x 2048) bf16, M-major scales.  Median of
    `reps` launches timed with HIP events; HBM roofline on the bytes it must
    move."""
    import torch

    import moe_grouped_precision_amd as w4a8

    R, I = 131072, 2048
    g = torch.Generator(device="cuda").manual_seed(23)
    C = (torch.randn((R, 2 * I), generator=g, device="cuda") * 3).to(torch.bfloat16)
    A = torch.empty((R, I), dtype=torch.uint8, device="cuda")
    SA = torch.empty((I // 128, R), dtype=torch.float32, device="cuda")
    for _ in range(warmup):
        w4a8.swiglu_quant(C, 1, A=A, SA=SA)
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(reps)]
    torch.cuda.synchronize()
    for a, b in ev:
        a.record()
        w4a8.swiglu_quant(C, 1, A=A, SA=SA)
        b.record()
    torch.cuda.synchronize()
    ms = statistics.median([a.elapsed_time(b) for a, b in ev])
    nbytes = R * 2 * I * 2 + R * I + 4 * R * (I // 128)
    gbs = nbytes / (ms * 1e-3) / 1e9
    return {"workload": f"{R} rows x (2 x {I}) bf16 gate/up output, M-major scales",
            "us_median": round(ms * 1e3, 2), "algorithmic_bytes": int(nbytes),
            "roofline": {"bound": "hbm", "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                         "frac": round(gbs / HBM_PEAK_GBS, 4)}}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=None)
    ap.add_argument("--warmup", type=int, default=None)
    ap.add_argument("--config", default="decode_gateup")
    ap.add_argument("--layout", type=int, default=None, help="0 row-major, 1 M-major input scales")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-budget", type=float, default=20.0)
    ap.add_argument("--no-probes", action="store_true",
                    help="skip the measured-peak probes (MFMA rate, HBM read bandwidth)")
    ap.add_argument("--no-quantize", action="store_true",
                    help="skip the quantizer, SwiGLU-requantization, combine and wide-pool "
                         "routing-prep and GEMM measurements")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a plain 1 GiB copy (memory-counter calibration)")
    args = ap.parse_args()

    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported "
              "(the path has no multi-GPU component)", file=sys.stderr)
        sys.exit(2)

    if args.copy_calibration:
        copy_calibration(args.steps or 5)
        return

    import numpy as np
    import torch

    import moe_grouped_precision_amd as w4a8
    import synth

    name = args.config
    cfg = synth.CONFIGS[name]
    steps = args.steps if args.steps is not None else DEFAULT_STEPS.get(name, 50)
    if args.warmup is None:
        args.warmup = DEFAULT_WARMUP.get(name, 200)
    layout = args.layout if args.layout is not None else (1 if name == "prefill_gateup" else 0)
    w4a8.load()
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)

    log(f"generating {name} on {'cuda' if name == 'prefill_gateup' else 'cpu'}")
    gen_dev = "cuda" if name == "prefill_gateup" else "cpu"
    p = synth.make_problem(name, device=gen_dev)
    ids = p.topk_ids.to(dev)
    A = p.A.to(dev)
    SA = (p.SA if layout == 0 else synth.to_m_major(p.SA)).to(dev)
    weight_bytes = p.B.numel() + p.SB.numel()
    # rotate weight copies so that timed reads come from HBM, not the 256 MB Infinity Cache
    nrot = max(1, math.ceil(2 * INFINITY_CACHE_BYTES / weight_bytes) + 1)
    Bs = [p.B.to(dev)] + [p.B.to(dev).clone() for _ in range(nrot - 1)]
    SBs = [p.SB.to(dev)] + [p.SB.to(dev).clone() for _ in range(nrot - 1)]
    counts_d = torch.empty(p.E, dtype=torch.int32, device=dev)
    off_d = torch.empty(p.E + 1, dtype=torch.int32, device=dev)
    rows_d = torch.empty(p.R, dtype=torch.int32, device=dev)
    C = torch.empty((p.R, p.N), dtype=torch.bfloat16, device=dev)
    torch.cuda.synchronize()
    log(f"inputs resident: R={p.R} N={p.N} K={p.K} E={p.E}, {nrot} weight copies")

    def step(i):
        w4a8.route_prep(ids, p.E, counts_d, off_d, rows_d)
        w4a8.grouped_gemm(A, SA, layout, Bs[i % nrot], SBs[i % nrot], off_d, out=C)

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    log(f"warmup done ({args.warmup} steps)")

    # whole-step timing
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0.record()
    for i in range(steps):
        step(i)
    t1.record()
    torch.cuda.synchronize()
    ms_per_step = t0.elapsed_time(t1) / steps

    # per-launch timing of the grouped GEMM call, on the stream it is launched on
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(steps)]
    for i in range(steps):
        w4a8.route_prep(ids, p.E, counts_d, off_d, rows_d)
        ev[i][0].record()
        w4a8.grouped_gemm(A, SA, layout, Bs[i % nrot], SBs[i % nrot], off_d, out=C)
        ev[i][1].record()
    torch.cuda.synchronize()
    gemm_ms = [a.elapsed_time(b) for a, b in ev]
    gemm_med = statistics.median(gemm_ms)
    log(f"timed {steps} steps: {ms_per_step * 1e3:.1f} us/step, gemm median {gemm_med * 1e3:.1f} us")

    counts = counts_d.cpu().numpy()
    off = off_d.cpu().numpy()
    flops = 2.0 * p.R * p.N * p.K
    tflops = flops / (ms_per_step * 1e-3) / 1e12
    nbytes = algorithmic_bytes(counts, p.E, p.N, p.K)
    bound = BOUND.get(name, "hbm")
    if bound == "hbm":
        achieved = nbytes / (gemm_med * 1e-3) / 1e9
        roof = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": recorded_traffic(name, layout)}
    else:
        achieved = flops / (gemm_med * 1e-3) / 1e12
        roof = {"bound": "mfma", "achieved": round(achieved, 1), "peak": MFMA_FP8_PEAK_TFS,
                "unit": "TFLOP/s", "frac": round(achieved / MFMA_FP8_PEAK_TFS, 4),
                "traffic": recorded_traffic(name, layout)}

    probes = None
    if not args.no_probes:
        from moe_grouped_precision_amd import probe
        log("measuring sustained peaks (MFMA fp4 x fp8, HBM read)")
        probes = {"mfma_fp4xfp8_tflops": round(probe.mfma_tflops(4, 0), 1),
                  "mfma_fp4xfp8_random_operands_tflops": round(probe.mfma_tflops_random(4, 0), 1),
                  "hbm_read_gbs": round(probe.read_gbs(), 1)}
        # the matrix core's rate depends on the operand bits: the random-operand
        # figure is the one real data can approach
        measured = (probes["hbm_read_gbs"] if bound == "hbm"
                    else probes["mfma_fp4xfp8_random_operands_tflops"])
        roof["measured_peak"] = measured
        roof["frac_of_measured"] = round(roof["achieved"] / measured, 4)

    quant = comb = swq = wide = wide_gemm = None
    if not args.no_quantize:
        log("timing the activation quantizer, SwiGLU requantization, the top-k combine, "
            "the routing prep over 6144 experts and the GEMM over 2048 experts")
        quant = measure_quantize_gather()
        swq = measure_swiglu_quant()
        comb = measure_combine()
        wide = measure_route_prep_wide()
        wide_gemm = measure_gemm_wide_pool()

    cpu = None
    if not args.no_cpu_baseline:
        log("timing the CPU oracle on a bounded sample")
        cpu = cpu_baseline(p, off, layout, args.cpu_budget)

    layout_name = "M-major" if layout == 1 else "row-major"
    out = {
        "metric": "grouped W4A8 GEMM TFLOP/s (routing prep + grouped GEMM per step)",
        "value": round(tflops, 3),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp8e4m3 x fp4e2m1 (fp32 accumulate, bf16 out)",
        "data": "synthetic",
        "config": {
            "workload": f"{name}: E={p.E} top_k={p.top_k} tokens={p.T} routed_rows={p.R} "
                        f"N={p.N} K={p.K} {cfg['routing']} routing, {layout_name} input scales",
            "experts_with_rows": int((counts > 0).sum()),
            "max_rows_per_expert": int(counts.max()) if len(counts) else 0,
            "gemm_us_median": round(gemm_med * 1e3, 2),
            "gemm_us_p10_p90": [round(float(np.percentile(gemm_ms, 10)) * 1e3, 2),
                                round(float(np.percentile(gemm_ms, 90)) * 1e3, 2)],
            "algorithmic_bytes": int(nbytes),
            "flop": flops,
            "weight_copies_rotated": nrot,
            "kernel_source_sha256": kernel_source_hash(),
        },
        "roofline": roof,
        "probes": probes,
        "quantize_gather": quant,
        "swiglu_quant": swq,
        "combine": comb,
        "route_prep_wide_pool": wide,
        "grouped_gemm_wide_pool": wide_gemm,
        "cpu_baseline": cpu,
    }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
