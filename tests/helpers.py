"""Shared test helpers: parity metric, device transfer, row sampling."""

from __future__ import annotations

import numpy as np
import torch

from oracle import bf16_bits_to_f64

TOL = 8e-3   # max |gpu - ref| / max(rms(ref), |ref|), elementwise


def bits_of(c: torch.Tensor) -> np.ndarray:
    """bf16 tensor (any device) -> uint16 numpy bit patterns."""
    return c.detach().contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def parity_error(gpu_bits: np.ndarray, ref_bits: np.ndarray, rms_ref: float | None = None) -> float:
    """Largest elementwise |g - r| / max(rms(ref), |r|); inf if any NaN/inf disagrees."""
    return parity_report(gpu_bits, ref_bits, rms_ref)["err"]


MAX_ULP_LARGE = 1          # bf16 ulps, on elements with |ref| >= rms(ref)


# Error of the matrix core's sum of one 128-K group, as a fraction of the
# group's magnitude sum.  The products are exact, but the instruction adds
# them with a finite internal width after aligning them, so the error grows
# with the spread of the products' magnitudes inside a group.  Measured on
# MI355X (largest error over all outputs, the bf16 rounding taken off, as a
# fraction of the output's magnitude sum): quantized N(0,1) activations
# times N(0, 0.02) MXFP4 weights, whose products span about a dozen
# binades, 1.1e-6 at most over every workload (2^-19.8); random E4M3 x E2M1
# codes with E8M0 scales over 20 binades, whose products span about 40
# binades, 2.1e-4 (2^-12.2) at most over the edge-case shapes.  The bounds
# keep a margin of 16x and 4.7x over them.
GROUP_EPS_QUANTIZED = 2.0 ** -16
GROUP_EPS_RANDOM_CODES = 2.0 ** -10


def fp32_sum_eps(K: int, group_eps: float = GROUP_EPS_QUANTIZED) -> float:
    """Relative bound on the accumulation error of one output, as a fraction
    of sum_k |a_k w_k|: the matrix core's sum of each 128-K group (group_eps
    of that group's magnitude sum), then one fp32 rounding per promotion into
    the accumulator (G = K / 128 groups) and one for the addition of the two
    K halves of the streaming phase."""
    return group_eps + ((K // 128) + 2) * 2.0 ** -24


def _bf16_ulp(x: np.ndarray) -> np.ndarray:
    _, p = np.frexp(np.abs(x))
    return np.ldexp(1.0, np.maximum(p - 8, -133))


def parity_report(gpu_bits: np.ndarray, ref_bits: np.ndarray, rms_ref: float | None = None,
                  exact: np.ndarray | None = None, abs_sum: np.ndarray | None = None, K: int | None = None,
                  group_eps: float = GROUP_EPS_QUANTIZED) -> dict:
    """err: the normalised maximum above; mismatches: elements whose bits
    differ; max_ulp: largest |g - r| in bf16 ulps of r (over all elements, and
    over those with |r| >= rms as max_ulp_large).  With the fp64 exact values
    and the magnitude sums of their products (oracle grouped_gemm_f64 with
    absolute=False / True) and K: beyond_fp32 = elements farther from the
    exact value than an fp32 accumulation (fp32_sum_eps(K) * abs_sum) followed
    by one bf16 rounding can be."""
    g = bf16_bits_to_f64(gpu_bits)
    r = bf16_bits_to_f64(ref_bits)
    if g.shape != r.shape:
        raise AssertionError(f"shape {g.shape} vs {r.shape}")
    n = int(g.size)
    rep = {"err": 0.0, "mismatches": 0, "n": n, "max_ulp": 0.0, "max_ulp_large": 0.0, "beyond_fp32": 0,
           "acc_err": 0.0}
    if n == 0:
        return rep
    if not np.all(np.isfinite(g)) or not np.all(np.isfinite(r)):
        rep.update(err=float("inf"), mismatches=n, max_ulp=float("inf"), max_ulp_large=float("inf"), beyond_fp32=n)
        return rep
    rms = float(np.sqrt(np.mean(r * r))) if rms_ref is None else rms_ref
    den = np.maximum(rms, np.abs(r))
    den = np.where(den == 0, 1.0, den)
    diff = np.abs(g - r)
    ulps = diff / _bf16_ulp(r)
    large = np.abs(r) >= rms
    rep.update(err=float(np.max(diff / den)),
               mismatches=int(np.count_nonzero(np.asarray(gpu_bits) != np.asarray(ref_bits))),
               max_ulp=float(ulps.max()), max_ulp_large=float(ulps[large].max()) if large.any() else 0.0)
    if exact is not None:
        acc_err = fp32_sum_eps(K, group_eps) * np.asarray(abs_sum, dtype=np.float64)
        bound = acc_err + 0.5 * _bf16_ulp(np.abs(exact) + acc_err)
        rep["beyond_fp32"] = int(np.count_nonzero(np.abs(g - exact) > bound))
        # the largest accumulation error the outputs show, as a fraction of
        # their magnitude sums (the bf16 rounding's half ulp taken off)
        mag = np.asarray(abs_sum, dtype=np.float64)
        excess = np.maximum(np.abs(g - exact) - 0.5 * _bf16_ulp(g), 0.0)
        rep["acc_err"] = float(np.max(np.where(mag > 0, excess / np.where(mag > 0, mag, 1.0), 0.0)))
    return rep


def assert_parity(gpu_bits: np.ndarray, ref_bits: np.ndarray, label: str, rms_ref: float | None = None,
                  exact: np.ndarray | None = None, abs_sum: np.ndarray | None = None, K: int | None = None,
                  group_eps: float = GROUP_EPS_QUANTIZED) -> dict:
    """Print the parity report and assert the bar: normalised error <= TOL,
    at most MAX_ULP_LARGE bf16 ulps on elements at least rms in size, and --
    given the exact values -- no element beyond what fp32 accumulation and
    one bf16 rounding allow (so a drift from rare one-ulp flips to
    widespread ones shows)."""
    rep = parity_report(gpu_bits, ref_bits, rms_ref, exact, abs_sum, K, group_eps)
    frac = rep["mismatches"] / max(rep["n"], 1)
    print(f"{label}: parity_error={rep['err']:.3e} mismatches={rep['mismatches']}/{rep['n']} "
          f"({frac:.2e}) max_ulp={rep['max_ulp']:.3g} max_ulp_large={rep['max_ulp_large']:.3g} "
          f"beyond_fp32={rep['beyond_fp32'] if exact is not None else '-'} acc_err={rep['acc_err']:.2e}", flush=True)
    assert rep["err"] <= TOL, rep
    assert rep["max_ulp_large"] <= MAX_ULP_LARGE, rep
    assert rep["beyond_fp32"] == 0, rep
    return rep


def to_device(p, device="cuda"):
    """Copy a synth.Problem's tensors to the GPU (returns a dict)."""
    return dict(
        ids=p.topk_ids.to(device),
        A=p.A.to(device),
        SA=p.SA.to(device),
        B=p.B.to(device),
        SB=p.SB.to(device),
    )


def sample_rows(offsets: np.ndarray, tile_m_of, rng, per_expert_random=4):
    """Rows at expert and tile boundaries plus random rows of every expert."""
    rows = set()
    E = len(offsets) - 1
    for e in range(E):
        lo, hi = int(offsets[e]), int(offsets[e + 1])
        if hi == lo:
            continue
        rows.update([lo, hi - 1])
        tm = tile_m_of(hi - lo)
        if tm:
            for b in range(lo, hi, tm):
                rows.update([b, min(hi - 1, b + tm - 1)])
        rows.update(int(x) for x in rng.integers(lo, hi, size=per_expert_random))
    return np.array(sorted(rows), dtype=np.int64)
