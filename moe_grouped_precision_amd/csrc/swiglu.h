// SwiGLU and the E4M3 requantization of its output, shared by the standalone
// SwiGLU kernel (quant.hip) and the fused gate/up epilogue (mfma_phase.h).
// gfx950 only.
//
// The step between the two projections that the pages benchmark as a pair
// (humming PR #129 "Results" and PR #58 "H200 performance": gate/up and
// down shapes side by side): h = silu(g) * u with silu(g) = g / (1 + e^-g),
// then one fp32 scale per (row, 128 columns), s = amax|h| / 448 (1 for an
// all-zero group), and the E4M3FN code of clip(h / s, +-448) by round to
// nearest even -- the same activation recipe as the GEMM's input (float8e4m3
// with input-scale group size 128).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace w4a8 {

// h = silu(g) * u in fp32 with the hardware exponential and reciprocal:
// e^-g = 2^n * 2^(r log2 e) with n = rint(-g log2 e) and r = -g - n ln2 by
// two fused multiply-adds (ln2 split into its fp32 value and the fp32 value
// of the rest), so the argument of v_exp_f32 lies in [-1/2, 1/2] and carries
// no error from the size of g; 2^n by an exact ldexp.  -g is clamped to
// [-104, 104]: above about 88.7 e^-g overflows to inf and silu to -0 (its
// magnitude is below 2^-120 there), below -104 it underflows and silu is g.
// The result is within about five fp32 units in the last place of
// silu(g) * u (exp, reciprocal, three roundings).
constexpr float kLog2e = 1.44269502162933349609375f;   // fp32(log2 e)
constexpr float kLn2Hi = 0.693147182464599609375f;     // fp32(ln 2)
constexpr float kLn2Lo = -1.9046542121259336e-09f;     // fp32(ln 2 - kLn2Hi)
__device__ __forceinline__ float swiglu_f32(float g, float u) {
  const float x = fminf(fmaxf(-g, -104.0f), 104.0f);
  const float n = rintf(x * kLog2e);
  const float r = fmaf(-n, kLn2Lo, fmaf(-n, kLn2Hi, x));
  const float e = ldexpf(__builtin_amdgcn_exp2f(r * kLog2e), (int)n);
  return g * __builtin_amdgcn_rcpf(1.0f + e) * u;
}

// Scale of a group from its amax: amax / 448 (IEEE division), 1 if zero.
__device__ __forceinline__ float e4m3_group_scale(float amax) {
  return amax > 0.f ? __fdiv_rn(amax, 448.0f) : 1.0f;
}

// Four values times inv (= 1/s), clipped to +-448, as four E4M3FN codes
// (round to nearest even, OCP E4M3 on gfx950: v_cvt_pk_fp8_f32), byte j of
// the result holding value j.
__device__ __forceinline__ uint32_t e4m3x4(float a, float b, float c, float d, float inv) {
  const float ya = fminf(fmaxf(a * inv, -448.0f), 448.0f);
  const float yb = fminf(fmaxf(b * inv, -448.0f), 448.0f);
  const float yc = fminf(fmaxf(c * inv, -448.0f), 448.0f);
  const float yd = fminf(fmaxf(d * inv, -448.0f), 448.0f);
  int w = __builtin_amdgcn_cvt_pk_fp8_f32(ya, yb, 0, false);
  w = __builtin_amdgcn_cvt_pk_fp8_f32(yc, yd, w, true);
  return (uint32_t)w;
}

}  // namespace w4a8
