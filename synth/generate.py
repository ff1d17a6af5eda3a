"""Seeded synthetic workloads for the grouped-contiguous W4A8 MoE GEMM.

Workload shapes follow the pages' benchmark axes (humming PR #129, "Results"
section: FP8 E4M3 activations with fp32 scales per 128 along K, MXFP4 E2M1
weights with E8M0 scales per 32 along K, bf16 output, grouped-contiguous rows,
E experts, top-k routing) and the E=12 / top-8 shapes of humming PR #58
("H200 performance" table).

Recipe (also stated in the design notes):
  * routing ids are always drawn on the CPU with ``torch.Generator`` so that
    they are identical everywhere;
      - "uniform": each token's k experts uniformly without replacement
        (first k of a stable argsort of U(0,1) keys);
      - "biased":  logits = N(0,1) per (token, expert) + a fixed per-expert
        bias N(0,1) drawn from seed 1234; top-k by a stable descending sort.
  * A is drawn directly in grouped row order, R = T*k rows of N(0,1) fp32,
    quantised per (row, 128-K group) to E4M3 with scale amax/448
    (amax == 0 -> scale 1).
  * B is drawn per expert, [N, K] of N(0, 0.02) fp32, quantised per
    (column n, 32-K block) to E2M1 with an E8M0 scale 2^(floor(log2 amax)-2)
    (amax == 0 -> code 127), elements rounded to nearest-even on the E2M1
    grid and saturated at +-6; two codes per byte, even k in the low nibble.
  * Values may be drawn on a CUDA device (``device=``) for the largest
    workload; the bytes then differ from a CPU draw, and parity tests copy
    the device bytes to the host for the oracle.
"""

from __future__ import annotations

import dataclasses
from typing import Optional

import torch

# name -> shape/routing description.  R = T * top_k routed rows.
CONFIGS = {
    # tiny case, oracle finishes in well under a second
    "tiny": dict(E=8, T=32, top_k=2, N=256, K=512, routing="uniform", seed=0),
    # decode gate/up, E=32 top-8, 64 tokens
    "decode_gateup": dict(E=32, T=64, top_k=8, N=4096, K=6144, routing="biased", seed=1),
    # prefill down-proj, 1152 tokens
    "prefill_down": dict(E=32, T=1152, top_k=8, N=6144, K=2048, routing="biased", seed=2),
    # small-expert regime, E=12 top-8 balanced
    "e12_w13_m8": dict(E=12, T=8, top_k=8, N=6144, K=3584, routing="uniform", seed=3),
    "e12_w13_m64": dict(E=12, T=64, top_k=8, N=6144, K=3584, routing="uniform", seed=3),
    "e12_w2_m8": dict(E=12, T=8, top_k=8, N=3584, K=3072, routing="uniform", seed=3),
    "e12_w2_m64": dict(E=12, T=64, top_k=8, N=3584, K=3072, routing="uniform", seed=3),
    # large prefill gate/up, 16384 tokens
    "prefill_gateup": dict(E=32, T=16384, top_k=8, N=4096, K=6144, routing="biased", seed=4),
}

_BIAS_SEED = 1234
# sub-stream ids mixed into the seed
_S_ROUTE, _S_A, _S_B = 0, 2, 3

E4M3_MAX = 448.0


def _gen(seed: int, stream: int, device: str = "cpu") -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(seed * 1000003 + stream * 7919 + 17)
    return g


def make_routing(kind: str, T: int, E: int, top_k: int, seed: int) -> torch.Tensor:
    """Top-k expert ids per token, int32 [T, top_k], drawn on the CPU."""
    if not (1 <= top_k <= E):
        raise ValueError("need 1 <= top_k <= E")
    g = _gen(seed, _S_ROUTE)
    if kind == "uniform":
        keys = torch.rand((T, E), generator=g, dtype=torch.float32)
        order = torch.sort(keys, dim=1, stable=True).indices
    elif kind == "biased":
        gb = torch.Generator().manual_seed(_BIAS_SEED)
        bias = torch.randn((E,), generator=gb, dtype=torch.float32)
        logits = torch.randn((T, E), generator=g, dtype=torch.float32) + bias
        order = torch.sort(logits, dim=1, descending=True, stable=True).indices
    else:
        raise ValueError(f"unknown routing kind {kind!r}")
    return order[:, :top_k].to(torch.int32).contiguous()


def make_wide_routing(T: int, E: int, top_k: int, seed: int, skew: bool = False) -> torch.Tensor:
    """Top-k expert ids, int32 [T, top_k], for a wide expert pool (thousands
    of experts, as in MoonEP PR #38's shared expert pools).  Distinct within a
    token.  Uniform: the top-k of uniform random keys.  Skewed: expert weights
    exp(9 u) (u uniform, so sizes span about four orders) sampled without
    replacement by the Gumbel top-k rule.  Drawn in slices of 256 tokens to
    keep the key matrix small."""
    if not (1 <= top_k <= E):
        raise ValueError("need 1 <= top_k <= E")
    g = _gen(seed, _S_ROUTE)
    logw = None
    if skew:
        logw = 9.0 * torch.rand((E,), generator=g, dtype=torch.float64)
    out = []
    for t0 in range(0, T, 256):
        rows = min(256, T - t0)
        keys = torch.rand((rows, E), generator=g, dtype=torch.float64)
        if skew:
            keys = logw - torch.log(-torch.log(keys.clamp_min(1e-300)))
        out.append(torch.topk(keys, top_k, dim=1).indices.to(torch.int32))
    if not out:
        return torch.zeros((0, top_k), dtype=torch.int32)
    return torch.cat(out).contiguous()


def wide_pool_codes(counts, N: int, K: int, seed: int, device: str = "cuda"):
    """Raw random codes for a wide expert pool, drawn directly on `device`
    as uint8 (a pool of tens of GB never passes through a wider type).  ``counts`` rows per expert, laid out
    contiguously in expert order.  A avoids the two E4M3 NaN codes, SA is
    U(0.01, 4) fp32 row-major, B any byte, SB uniform in [112, 132).
    Returns (A, SA, B, SB) on `device`."""
    E = len(counts)
    R = int(sum(int(c) for c in counts))
    g = torch.Generator(device=device)
    g.manual_seed(seed * 1000003 + 101)
    A = torch.randint(0, 256, (R, K), generator=g, dtype=torch.uint8, device=device)
    A[(A & 0x7F) == 0x7F] = 0x38
    SA = torch.rand((R, K // 128), generator=g, dtype=torch.float32, device=device) * 4 + 0.01
    B = torch.randint(0, 256, (E, N, K // 2), generator=g, dtype=torch.uint8, device=device)
    SB = torch.randint(112, 132, (E, N, K // 32), generator=g, dtype=torch.uint8, device=device)
    return A, SA, B, SB


def quantize_fp8_rows(x: torch.Tensor):
    """fp32 [R, K] -> (E4M3 codes uint8 [R, K], fp32 scales [R, K/128]).

    Scale per (row, 128-group) is amax/448 (1.0 for an all-zero group); the
    scaled values are clamped to +-448 before the cast because the torch cast
    does not saturate.
    """
    R, K = x.shape
    if K % 128:
        raise ValueError("K must be a multiple of 128")
    xg = x.reshape(R, K // 128, 128)
    amax = xg.abs().amax(dim=2)
    s = torch.where(amax > 0, amax / E4M3_MAX, torch.ones_like(amax))
    q = (xg / s.unsqueeze(2)).clamp(-E4M3_MAX, E4M3_MAX)
    codes = q.to(torch.float8_e4m3fn).view(torch.uint8).reshape(R, K)
    return codes.contiguous(), s.to(torch.float32).contiguous()


# E2M1 magnitude decision points, with the tie direction that keeps the
# even code: a tie at a point whose lower neighbour code is even rounds
# down (strict '>'), otherwise up ('>=').
_E2M1_POINTS = ((0.25, False), (0.75, True), (1.25, False), (1.75, True),
                (2.5, False), (3.5, True), (5.0, False))


def _e2m1_codes(y: torch.Tensor) -> torch.Tensor:
    """RNE of fp32 y onto the E2M1 grid, saturating at +-6 -> codes uint8."""
    a = y.abs()
    code = torch.zeros_like(a, dtype=torch.int32)
    for p, up in _E2M1_POINTS:
        code += (a >= p if up else a > p).to(torch.int32)
    sign = ((y < 0) & (code > 0)).to(torch.int32) << 3
    return (code | sign).to(torch.uint8)


def quantize_mxfp4(w: torch.Tensor):
    """fp32 [N, K] -> (packed E2M1 uint8 [N, K/2], E8M0 scales uint8 [N, K/32])."""
    N, K = w.shape
    if K % 32:
        raise ValueError("K must be a multiple of 32")
    wb = w.reshape(N, K // 32, 32)
    amax = wb.abs().amax(dim=2)
    # floor(log2(amax)) exactly: frexp gives amax = m * 2^p with m in [0.5, 1)
    _, p = torch.frexp(amax)
    ex = (p.to(torch.int32) - 1 - 2).clamp(-127, 127)
    ex = torch.where(amax > 0, ex, torch.zeros_like(ex))
    sb = (ex + 127).to(torch.uint8)
    y = torch.ldexp(wb, (-ex).to(torch.float32).unsqueeze(2))
    codes = _e2m1_codes(y).reshape(N, K)
    packed = (codes[:, 0::2] | (codes[:, 1::2] << 4)).contiguous()
    return packed, sb.contiguous()


def to_m_major(sa_row_major: torch.Tensor) -> torch.Tensor:
    """[R, K/128] -> [K/128, R] contiguous (the M-major input-scale layout)."""
    return sa_row_major.t().contiguous()


@dataclasses.dataclass
class Problem:
    name: str
    E: int
    T: int
    top_k: int
    N: int
    K: int
    topk_ids: torch.Tensor      # int32 [T, top_k] (CPU)
    A: torch.Tensor             # uint8 [R, K] E4M3 codes, grouped row order
    SA: torch.Tensor            # fp32 [R, K/128] row-major scales
    B: torch.Tensor             # uint8 [E, N, K/2] packed E2M1
    SB: torch.Tensor            # uint8 [E, N, K/32] E8M0

    @property
    def R(self) -> int:
        return self.T * self.top_k


def make_problem(name: str, device: str = "cpu", *, T: Optional[int] = None,
                 E: Optional[int] = None, N: Optional[int] = None,
                 K: Optional[int] = None, top_k: Optional[int] = None,
                 routing: Optional[str] = None, seed: Optional[int] = None) -> Problem:
    """Build one workload.  Keyword overrides make ragged / edge variants."""
    cfg = dict(CONFIGS[name]) if name in CONFIGS else {}
    for k_, v in dict(T=T, E=E, N=N, K=K, top_k=top_k, routing=routing, seed=seed).items():
        if v is not None:
            cfg[k_] = v
    E_, T_, k_, N_, K_ = cfg["E"], cfg["T"], cfg["top_k"], cfg["N"], cfg["K"]
    seed_ = cfg["seed"]
    ids = make_routing(cfg["routing"], T_, E_, k_, seed_)
    R = T_ * k_
    ga = _gen(seed_, _S_A, device)
    x = torch.randn((R, K_), generator=ga, dtype=torch.float32, device=device)
    A, SA = quantize_fp8_rows(x)
    del x
    gb = _gen(seed_, _S_B, device)
    B = torch.empty((E_, N_, K_ // 2), dtype=torch.uint8, device=device)
    SB = torch.empty((E_, N_, K_ // 32), dtype=torch.uint8, device=device)
    for e in range(E_):
        w = 0.02 * torch.randn((N_, K_), generator=gb, dtype=torch.float32, device=device)
        B[e], SB[e] = quantize_mxfp4(w)
    return Problem(name, E_, T_, k_, N_, K_, ids, A, SA, B, SB)


def random_codes_problem(counts, N: int, K: int, seed: int, sb_lo: int = 112, sb_hi: int = 132,
                         device: str = "cpu"):
    """Raw random codes for edge-case tests (not a quantised workload).

    ``counts`` rows per expert (rows are laid out contiguously in expert
    order); A codes avoid the two E4M3 NaN codes, SA is U(0.01, 4) fp32,
    B is any byte, SB is uniform in [sb_lo, sb_hi).  Returns
    (A, SA_row_major, B, SB, offsets) as CPU tensors (offsets int32 [E+1]).
    """
    E = len(counts)
    g = torch.Generator().manual_seed(seed)
    R = int(sum(counts))
    A = torch.randint(0, 256, (R, K), generator=g, dtype=torch.int32).to(torch.uint8)
    A[(A & 0x7F) == 0x7F] = 0x38
    SA = torch.rand((R, K // 128), generator=g, dtype=torch.float32) * 4 + 0.01
    B = torch.randint(0, 256, (E, N, K // 2), generator=g, dtype=torch.int32).to(torch.uint8)
    SB = torch.randint(sb_lo, sb_hi, (E, N, K // 32), generator=g, dtype=torch.int32).to(torch.uint8)
    offsets = torch.zeros(E + 1, dtype=torch.int32)
    offsets[1:] = torch.cumsum(torch.tensor(list(counts), dtype=torch.int64), 0).to(torch.int32)
    return A, SA, B, SB, offsets


def quantize_nvfp4(w: torch.Tensor):
    """fp32 [N, K] -> (packed E2M1 uint8 [N, K/2], E4M3 codes uint8 [N, K/16],
    fp32 tensor scale gs): gs = amax|w| / (448 * 6), each 16-block's E4M3
    code the RNE of amax_block / (6 gs), then the E2M1 RNE of w / (scale gs)."""
    N, K = w.shape
    if K % 16:
        raise ValueError("K must be a multiple of 16")
    amax = float(w.abs().max())
    gs = torch.tensor(amax / (448.0 * 6.0) if amax > 0 else 1.0, dtype=torch.float32)
    wb = w.reshape(N, K // 16, 16)
    bamax = wb.abs().amax(dim=2)
    sc = (bamax / (6.0 * gs)).clamp(max=448.0).to(torch.float8_e4m3fn)
    dec = sc.to(torch.float32)
    dec = torch.where(dec > 0, dec, torch.ones_like(dec))
    y = wb / (dec * gs).unsqueeze(2)
    codes = _e2m1_codes(y).reshape(N, K)
    packed = (codes[:, 0::2] | (codes[:, 1::2] << 4)).contiguous()
    return packed, sc.view(torch.uint8).contiguous(), float(gs)


def bf16_bits(x: torch.Tensor) -> torch.Tensor:
    """fp32 -> bf16 (torch's round to nearest even), as uint16-viewable int16."""
    return x.to(torch.bfloat16).view(torch.int16).contiguous()


@dataclasses.dataclass
class ProblemA16:
    name: str
    fmt: int                    # 0 MXFP4 (E8M0 per 32), 1 NVFP4 (E4M3 per 16 + fp32 per expert)
    E: int
    T: int
    top_k: int
    N: int
    K: int
    topk_ids: torch.Tensor      # int32 [T, top_k] (CPU)
    A: torch.Tensor             # int16 [R, K] bf16 bits, grouped row order
    B: torch.Tensor             # uint8 [E, N, K/2] packed E2M1
    SB: torch.Tensor            # uint8 [E, N, K/32] E8M0 or [E, N, K/16] E4M3
    GS: torch.Tensor            # fp32 [E] (ones for MXFP4)

    @property
    def R(self) -> int:
        return self.T * self.top_k


def make_a16_problem(name: str, fmt: int, device: str = "cpu", **overrides) -> ProblemA16:
    """A workload of CONFIGS (shapes and routing) with bf16 activations
    (N(0,1) rounded to bf16) and N(0, 0.02) weights quantized to MXFP4 or
    NVFP4."""
    cfg = dict(CONFIGS[name]) if name in CONFIGS else {}
    cfg.update({k: v for k, v in overrides.items() if v is not None})
    E_, T_, k_, N_, K_ = cfg["E"], cfg["T"], cfg["top_k"], cfg["N"], cfg["K"]
    seed_ = cfg["seed"] + 101 + fmt
    ids = make_routing(cfg["routing"], T_, E_, k_, cfg["seed"])
    R = T_ * k_
    ga = _gen(seed_, _S_A, device)
    A = bf16_bits(torch.randn((R, K_), generator=ga, dtype=torch.float32, device=device))
    gb = _gen(seed_, _S_B, device)
    B = torch.empty((E_, N_, K_ // 2), dtype=torch.uint8, device=device)
    SB = torch.empty((E_, N_, K_ // (32 if fmt == 0 else 16)), dtype=torch.uint8, device=device)
    GS = torch.ones(E_, dtype=torch.float32, device=device)
    for e in range(E_):
        w = 0.02 * torch.randn((N_, K_), generator=gb, dtype=torch.float32, device=device)
        if fmt == 0:
            B[e], SB[e] = quantize_mxfp4(w)
        else:
            B[e], SB[e], GS[e] = quantize_nvfp4(w)
    return ProblemA16(name, fmt, E_, T_, k_, N_, K_, ids, A, B, SB, GS)
