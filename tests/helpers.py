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
    g = bf16_bits_to_f64(gpu_bits)
    r = bf16_bits_to_f64(ref_bits)
    if g.shape != r.shape:
        raise AssertionError(f"shape {g.shape} vs {r.shape}")
    if g.size == 0:
        return 0.0
    if not np.all(np.isfinite(g)) or not np.all(np.isfinite(r)):
        return float("inf")
    rms = float(np.sqrt(np.mean(r * r))) if rms_ref is None else rms_ref
    den = np.maximum(rms, np.abs(r))
    den = np.where(den == 0, 1.0, den)
    return float(np.max(np.abs(g - r) / den))


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
