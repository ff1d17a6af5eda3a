"""Grouped-contiguous W4A8 MoE expert GEMM for MI355X (gfx950).

Thin ctypes binding over libw4a8.so (declared in include/w4a8.h).  Functions
take torch CUDA tensors, check dtype/shape/device, and pass raw device
pointers and the current HIP stream to the C ABI; every step of the
computation runs in the library's HIP kernels.  Outputs are allocated with
torch when the caller does not pass them.

    route_prep(topk_ids, E)          -> counts, expert_offsets, row_of_slot
    route_prep_waves(E, lds_bytes)   -> waves per workgroup of the route prep (host only)
    plan(expert_offsets, E, N, K)    -> int32 plan (header + tiles)
    grouped_gemm(A, SA, layout, B, SB, expert_offsets, out=None) -> C (bf16)
    quantize_gather(x, row_of_slot, top_k, R, layout) -> A (E4M3 codes), SA
    combine(C, row_of_slot, weights, top_k, out=None) -> per-token bf16 sums
    swiglu_quant(C, layout) -> A (E4M3 codes of silu(gate) * up), SA
    grouped_gemm_planned(A, SA, layout, B, SB, expert_offsets, plan, out=None) -> C (bf16)
    grouped_gemm_planned_noalloc(A, SA, layout, B, SB, expert_offsets, out) -> out (plan in library scratch)
    grouped_gemm_swiglu(A, SA, layout, B13, SB13, expert_offsets, layout2)
                                     -> A2 (E4M3 codes of silu(gate) * up), SA2
    grouped_gemm_a16(A_bf16, B, SB, fmt, expert_offsets, expert_scales=None, out=None)
                                     -> C (bf16), MXFP4 (fmt 0) or NVFP4 (fmt 1) weights
"""

from ._lib import (  # noqa: F401
    SCALE_M_MAJOR,
    SCALE_ROW_MAJOR,
    WSCALE_MX,
    WSCALE_NV,
    W4A8Error,
    combine,
    grouped_gemm,
    grouped_gemm_a16,
    grouped_gemm_planned,
    grouped_gemm_planned_noalloc,
    grouped_gemm_swiglu,
    lib_path,
    load,
    plan,
    plan_bytes,
    plan_params,
    quantize_gather,
    route_prep,
    route_prep_waves,
    swiglu_quant,
)
