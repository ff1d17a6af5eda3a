// Activation quantization with the gather into grouped rows, gfx950.
//
// bf16 tokens -> FP8 E4M3FN codes with one fp32 scale per (row, 128-K group),
// written to the grouped row of every (token, slot): the producer of the
// grouped GEMM's A and a_scales (humming PR #129, "Results" command:
// float8e4m3 activations with input-scale group size 128, grouped_contiguous
// rows).  Per group, s = amax / 448 (1 for an all-zero group), v =
// clip(x / s, +-448) with IEEE fp32 divisions, code = round to nearest even
// of v onto the E4M3FN grid (OCP 8-bit floating point: largest finite 448,
// subnormals m/8 * 2^-6).
//
// The work is a stream: read 2 bytes per element once, write one byte per
// element per slot.  One workgroup per token with 8 lanes per 128-element
// group (all of a row's groups in one pass up to K = 8192), 16 elements (two
// 16-byte loads) per lane, the group's amax by three lane exchanges; a wave
// stores 8 consecutive groups = 1 KB of codes per slot in one nontemporal
// 16-byte store per lane (written once, read by the GEMM later: 196 against
// 209 us with ordinary stores on 16384 x 6144).  No LDS, no barrier.  Like the cast kernels of
// TransformerEngine PR #3459 (description: register-only rowwise cast, no
// shared memory or barrier), nothing is staged; unlike them the scale is the
// fp32 amax/448 of 128 elements, not an E8M0 exponent of 32.
#include "swiglu.h"
#include "w4a8_launch.h"

#include <hip/hip_runtime.h>

namespace w4a8 {
namespace {

typedef uint32_t v4u __attribute__((ext_vector_type(4)));

// E4M3FN code of a finite v with |v| <= 448, round to nearest even, sign kept.
// Below 2^-6 the grid is the multiples of 2^-9 (the product by 512 is exact
// and rintf rounds halves to even; 8 * 2^-9 = 2^-6 is code 8).  Above, the
// fp32 mantissa is cut to 3 bits with round to nearest even; a carry out of
// the mantissa moves to the next exponent by the same addition.
__device__ __forceinline__ uint32_t e4m3_rne(float v) {
  const uint32_t bits = __float_as_uint(v);
  const uint32_t sign = (bits >> 24) & 0x80u;
  const uint32_t a = bits & 0x7fffffffu;
  uint32_t code;
  if (a < 0x3c800000u) {
    code = (uint32_t)rintf(__uint_as_float(a) * 512.0f);
  } else {
    const uint32_t e = (a >> 23) - 120u;            // biased E4M3 exponent: (e32 - 127) + 7
    const uint32_t keep = (a >> 20) & 7u, rem = a & 0xfffffu;
    const uint32_t up = (rem > 0x80000u || (rem == 0x80000u && (keep & 1u))) ? 1u : 0u;
    code = (e << 3) + keep + up;
  }
  return code | sign;
}

__global__ void __launch_bounds__(512)
quant_gather_kernel(const uint16_t* __restrict__ x, int K, const int32_t* __restrict__ row_of_slot,
                    int top_k, int R, uint8_t* __restrict__ A, float* __restrict__ SA, int layout) {
  // M-major scales: consecutive tokens on one XCD (workgroups go to the 8
  // XCDs round-robin).  The rows of consecutive tokens of one expert are
  // adjacent, so their 4-byte scales then share lines in one L2 before they
  // are written back (228 against 241 us on 16384 x 6144; for row-major
  // scales the plain order measured faster, 201 against 210 us).
  const int T = gridDim.x;
  const int t = (layout == 0 || (T & 7)) ? (int)blockIdx.x
                                         : (int)((blockIdx.x & 7) * (T >> 3) + (blockIdx.x >> 3));
  const int G = K >> 7;
  const int lane8 = threadIdx.x & 7;       // position in the group
  const int gsub = threadIdx.x >> 3;       // group slot
  const int gstep = blockDim.x >> 3;
  const uint16_t* xt = x + (size_t)t * K;
  const int32_t* rs = row_of_slot + (size_t)t * top_k;
  for (int g = gsub; g < G; g += gstep) {
    const v4u* src = reinterpret_cast<const v4u*>(xt + g * 128 + lane8 * 16);
    const v4u p = __builtin_nontemporal_load(src), q = __builtin_nontemporal_load(src + 1);
    const uint32_t w[8] = {p[0], p[1], p[2], p[3], q[0], q[1], q[2], q[3]};
    float v[16];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      v[2 * i] = __uint_as_float(w[i] << 16);            // element 2i: low half
      v[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);  // element 2i+1: high half
    }
    float m = 0.f;
#pragma unroll
    for (int i = 0; i < 16; ++i) m = fmaxf(m, fabsf(v[i]));
    m = fmaxf(m, __shfl_xor(m, 1, 8));
    m = fmaxf(m, __shfl_xor(m, 2, 8));
    m = fmaxf(m, __shfl_xor(m, 4, 8));
    const float s = m > 0.f ? __fdiv_rn(m, 448.0f) : 1.0f;
    uint32_t c[4] = {0u, 0u, 0u, 0u};
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const float y = fminf(fmaxf(__fdiv_rn(v[i], s), -448.0f), 448.0f);
      c[i >> 2] |= e4m3_rne(y) << (8 * (i & 3));
    }
    const v4u out = {c[0], c[1], c[2], c[3]};
    for (int j = 0; j < top_k; ++j) {
      const int r = rs[j];
      if (r < 0 || r >= R) continue;  // a slot that names no row
      __builtin_nontemporal_store(out, reinterpret_cast<v4u*>(A + (size_t)r * K + g * 128 + lane8 * 16));
      if (lane8 == 0) SA[layout ? (size_t)g * R + r : (size_t)r * G + g] = s;
    }
  }
}

// SwiGLU of the gate/up output and its E4M3 requantization (swiglu.h): one
// workgroup per row; 8 lanes per 128-column group, 16 columns of gate
// (columns 0 .. I-1) and the same 16 of up (columns I .. 2I-1) per lane;
// per group s = amax / 448, v = clip(h * (1/s), +-448) and its E4M3FN code
// by the hardware conversion.
__global__ void __launch_bounds__(512)
swiglu_quant_kernel(const uint16_t* __restrict__ C, int R, int I, uint8_t* __restrict__ A, float* __restrict__ SA,
                    int layout) {
  // M-major scales: consecutive rows on one XCD (see quant_gather_kernel)
  const int r = (layout == 0 || (R & 7)) ? (int)blockIdx.x
                                         : (int)((blockIdx.x & 7) * (R >> 3) + (blockIdx.x >> 3));
  const int G = I >> 7;
  const int lane8 = threadIdx.x & 7;
  const int gsub = threadIdx.x >> 3;
  const int gstep = blockDim.x >> 3;
  const uint16_t* row = C + (size_t)r * 2 * I;
  for (int g = gsub; g < G; g += gstep) {
    const v4u* gp = reinterpret_cast<const v4u*>(row + g * 128 + lane8 * 16);
    const v4u* up = reinterpret_cast<const v4u*>(row + I + g * 128 + lane8 * 16);
    const v4u g0 = __builtin_nontemporal_load(gp), g1 = __builtin_nontemporal_load(gp + 1);
    const v4u u0 = __builtin_nontemporal_load(up), u1 = __builtin_nontemporal_load(up + 1);
    const uint32_t gw[8] = {g0[0], g0[1], g0[2], g0[3], g1[0], g1[1], g1[2], g1[3]};
    const uint32_t uw[8] = {u0[0], u0[1], u0[2], u0[3], u1[0], u1[1], u1[2], u1[3]};
    float h[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const uint32_t gb = (i & 1) ? (gw[i >> 1] & 0xffff0000u) : (gw[i >> 1] << 16);
      const uint32_t ub = (i & 1) ? (uw[i >> 1] & 0xffff0000u) : (uw[i >> 1] << 16);
      h[i] = swiglu_f32(__uint_as_float(gb), __uint_as_float(ub));
    }
    float m = 0.f;
#pragma unroll
    for (int i = 0; i < 16; ++i) m = fmaxf(m, fabsf(h[i]));
    m = fmaxf(m, __shfl_xor(m, 1, 8));
    m = fmaxf(m, __shfl_xor(m, 2, 8));
    m = fmaxf(m, __shfl_xor(m, 4, 8));
    const float s = e4m3_group_scale(m);
    const float inv = __fdiv_rn(1.0f, s);
    uint32_t c[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) c[i] = e4m3x4(h[4 * i], h[4 * i + 1], h[4 * i + 2], h[4 * i + 3], inv);
    const v4u out = {c[0], c[1], c[2], c[3]};
    __builtin_nontemporal_store(out, reinterpret_cast<v4u*>(A + (size_t)r * I + g * 128 + lane8 * 16));
    if (lane8 == 0) SA[layout ? (size_t)g * R + r : (size_t)r * G + g] = s;
  }
}

}  // namespace

hipError_t launch_swiglu_quant(const uint16_t* C, int R, int I, uint8_t* A, float* SA, int layout,
                               hipStream_t stream) {
  if (R == 0) return hipSuccess;
  const int G = I >> 7;
  const int threads = 8 * (G < 64 ? ((G + 7) & ~7) : 64);
  hipLaunchKernelGGL(swiglu_quant_kernel, dim3(R), dim3(threads), 0, stream, C, R, I, A, SA, layout);
  return hipGetLastError();
}

hipError_t launch_quant_gather(const uint16_t* x, int T, int K, const int32_t* row_of_slot, int top_k, int R,
                               uint8_t* A, float* SA, int layout, hipStream_t stream) {
  if (T == 0) return hipSuccess;
  // 8 lanes per group, all groups of a row in one pass up to 64 groups (a
  // whole number of waves)
  const int G = K >> 7;
  const int threads = 8 * (G < 64 ? ((G + 7) & ~7) : 64);
  hipLaunchKernelGGL(quant_gather_kernel, dim3(T), dim3(threads), 0, stream, x, K, row_of_slot, top_k, R, A, SA,
                     layout);
  return hipGetLastError();
}

}  // namespace w4a8
