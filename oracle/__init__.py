"""CPU oracle for the grouped-contiguous W4A8 MoE expert GEMM.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path may import, call or
link anything here: only the test suite, the smoke check of the entry module
and the CPU-baseline leg of the benchmark use it.  It shares no code with the
HIP library (no kernels, headers, tables or constant generators) and imports
nothing from it, nor from the synthetic-input module.

What it computes (grouped-contiguous W4A8 GEMM as described by humming PR #129,
"Results" section and its benchmark command: FP8 E4M3 activations with one
fp32 scale per 128 K, MXFP4 E2M1 weights with one E8M0 scale per 32 K, bf16
output, rows grouped contiguously by expert):

    C[r, n] = bf16_rne( sum_k dec8(A[r,k]) * SA(r, k//128)
                              * dec4(B[e(r), n, k]) * 2^(SB[e(r), n, k//32] - 127) )

with every product exact in fp64, an fp64 sum, and one rounding to bf16.

Modules:
  formats -- exact decoders (E4M3FN, E2M1, E8M0) and fp64 -> bf16 RNE.
  gemm    -- the grouped GEMM above (fp64 BLAS per expert).
  route   -- routing histogram, exclusive-scan offsets, stable row map.
  plan    -- the per-expert tile rule and the tile list built from it.
  quant   -- bf16 tokens -> E4M3 codes with per-(row, 128) amax/448 scales,
             gathered to the grouped row of every slot.
  combine -- top-k weighted sum of grouped output rows back to tokens.
  swiglu  -- silu(gate) * up of the gate/up output, requantized to E4M3, in
             fp64, and the admissibility check of an fp32 result against it.
  a16     -- the grouped GEMM with bf16 activations and FP4 weights, MXFP4
             (E8M0 per 32) or NVFP4 (E4M3 per 16 and one fp32 scale per
             expert) scales.

Parity status: no page prints a worked example or output value for any of
these, so every function is pinned by closed forms, invariants, exact
brute force and independent library decoders in the CPU tests, not by
values from the pages.
"""

from .formats import (  # noqa: F401
    E2M1_VALUES,
    bf16_bits_to_f64,
    bf16_rne_bits,
    e2m1_table,
    e4m3_table,
    e8m0_value,
)
from .gemm import expert_gemm_f64, grouped_gemm_bf16, grouped_gemm_f64, rows_gemm_f64  # noqa: F401
from .plan import PLAN_PARAMS, plan_ref, tile_rule  # noqa: F401
from .route import route_ref  # noqa: F401
from .quant import bf16_bits_to_f32, e4m3_encode_rne, quantize_gather, quantize_tokens  # noqa: F401
from .combine import combine_ref  # noqa: F401
from .swiglu import check_h_quant, check_swiglu_quant, h_quant_f64, silu_f64, swiglu_f64, swiglu_quant_f64  # noqa: F401
from .a16 import FMT_MX, FMT_NV, grouped_gemm_a16_bf16, grouped_gemm_a16_f64  # noqa: F401
