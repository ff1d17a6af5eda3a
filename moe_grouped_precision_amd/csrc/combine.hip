// Top-k weighted combine of grouped output rows back to tokens, gfx950.
//
// out[t, :] = bf16( sum_j w[t, j] * C[row_of_slot[t*top_k + j], :] ): the
// step after the grouped GEMM that returns each token's expert outputs, the
// single-GPU half of an expert-parallel combine (the routing it inverts is
// the MoE planning of MoonEP PR #38, background section).  The sum runs in
// fp32 in slot order, each term one rounded product and one rounded addition
// (no fused multiply-add), so the result is unique; one rounding to bf16.
//
// A stream: each token reads its top_k rows once and writes one row.  One
// workgroup per token, 8 columns (one 16-byte load) per lane per pass; the
// slot rows and weights are the same for the whole workgroup.  No LDS, no
// barrier.
#include "w4a8_launch.h"

#include <hip/hip_runtime.h>

namespace w4a8 {
namespace {

typedef uint32_t v4u __attribute__((ext_vector_type(4)));
typedef float v2f __attribute__((ext_vector_type(2)));
typedef __bf16 v2bf __attribute__((ext_vector_type(2)));

__global__ void __launch_bounds__(512)
combine_kernel(const uint16_t* __restrict__ C, int R, int N, const int32_t* __restrict__ row_of_slot,
               const float* __restrict__ weights, int top_k, uint16_t* __restrict__ out) {
  // separate rounded products and sums: no contraction into fused multiply-adds
#pragma clang fp contract(off)
  const int t = blockIdx.x;
  const int32_t* rs = row_of_slot + (size_t)t * top_k;
  const float* ws = weights + (size_t)t * top_k;
  for (int c0 = threadIdx.x * 8; c0 < N; c0 += blockDim.x * 8) {
    float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    // eight slots' loads in flight at once, then their terms in slot order
    for (int j0 = 0; j0 < top_k; j0 += 8) {
      v4u v[8];
      float wv[8];
      bool ok[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const int j = j0 + u;
        const int r = j < top_k ? rs[j] : -1;
        ok[u] = r >= 0 && r < R;  // a slot that names no row contributes nothing
        wv[u] = ok[u] ? ws[j] : 0.f;
        v[u] = ok[u] ? __builtin_nontemporal_load(reinterpret_cast<const v4u*>(C + (size_t)r * N + c0))
                     : v4u{0u, 0u, 0u, 0u};
      }
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        if (!ok[u]) continue;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          acc[2 * i] = acc[2 * i] + wv[u] * __uint_as_float(v[u][i] << 16);
          acc[2 * i + 1] = acc[2 * i + 1] + wv[u] * __uint_as_float(v[u][i] & 0xffff0000u);
        }
      }
    }
    v4u o;
#pragma unroll
    for (int i = 0; i < 4; ++i)  // round to nearest even (packed conversion, denormals kept)
      o[i] = __builtin_bit_cast(uint32_t, __builtin_convertvector((v2f){acc[2 * i], acc[2 * i + 1]}, v2bf));
    *reinterpret_cast<v4u*>(out + (size_t)t * N + c0) = o;
  }
}

}  // namespace

hipError_t launch_combine(const uint16_t* C, int R, int N, const int32_t* row_of_slot, const float* weights, int T,
                          int top_k, uint16_t* out, hipStream_t stream) {
  if (T == 0) return hipSuccess;
  // one 16-byte chunk per lane, whole waves, at most 512 lanes
  const int chunks = N / 8;
  const int threads = chunks >= 512 ? 512 : ((chunks + 63) & ~63);
  hipLaunchKernelGGL(combine_kernel, dim3(T), dim3(threads), 0, stream, C, R, N, row_of_slot, weights, top_k, out);
  return hipGetLastError();
}

}  // namespace w4a8
