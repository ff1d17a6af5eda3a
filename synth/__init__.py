"""Seeded synthetic inputs for the grouped W4A8 expert GEMM.

This module is the one piece shared by the oracle-side tests and the HIP-side
tests and benchmark.  It produces *codes* (bytes) and routing ids; it holds
none of the GEMM's arithmetic (no decoding, no contraction, no grouping, no
tile planning).  Its quantisers only turn random fp32 draws into valid
E4M3 / E2M1 / E8M0 code bytes and bf16 bit patterns; whatever rounding they
use, both sides of a parity test consume the very same bytes.
"""

from .generate import (  # noqa: F401
    CONFIGS,
    Problem,
    ProblemA16,
    bf16_bits,
    make_a16_problem,
    make_problem,
    make_routing,
    make_wide_routing,
    quantize_fp8_rows,
    quantize_mxfp4,
    quantize_nvfp4,
    random_codes_problem,
    to_m_major,
    wide_pool_codes,
)
