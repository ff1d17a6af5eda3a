// Roofline probes (w4a8_probe.h): the sustained rate of the scaled f8f6f4
// MFMA for a pair of operand formats, and the sustained HBM read bandwidth
// of a plain streaming read.  gfx950 only.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "w4a8.h"
#include "w4a8_probe.h"

namespace {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));

template <int FA, int FB>
__global__ void __launch_bounds__(256) mfma_probe_kernel(int iters, float* sink) {
  const int lane = threadIdx.x & 63;
  // small finite codes in every format (E4M3 0x38 = 1.0, E2M1 nibble 2 = 1.0)
  const int fa = FA == 4 ? 0x22222222 : 0x38383838;
  const int fb = FB == 4 ? 0x22222222 : 0x38383838;
  v8i a = {fa, fa, fa, fa, fa, fa, fa, fa};
  v8i b = {fb, fb, fb, fb, fb, fb, fb, fb};
  a[0] ^= lane & 1;
  v4f acc[8];
#pragma unroll
  for (int k = 0; k < 8; ++k) acc[k] = v4f{0.f, 0.f, 0.f, 0.f};
  for (int i = 0; i < iters; ++i) {
#pragma unroll
    for (int k = 0; k < 8; ++k)
      acc[k] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, acc[k], FA, FB, 0, 127, 0, 127);
  }
  float s = 0.f;
#pragma unroll
  for (int k = 0; k < 8; ++k) s += acc[k][0] + acc[k][1] + acc[k][2] + acc[k][3];
  sink[blockIdx.x * 256 + threadIdx.x] = s;
}

// The same MFMA stream with operands loaded per lane from `ops` (16 words per
// thread: 8 for the A operand, 8 for B), so that they can be random bits
// rather than constants: the matrix core's sustained rate depends on the
// operand data (all-equal operands run about twice as fast as random ones).
template <int FA, int FB>
__global__ void __launch_bounds__(256) mfma_probe_data_kernel(int iters, const int* __restrict__ ops, float* sink) {
  const int* o = ops + ((size_t)blockIdx.x * 256 + threadIdx.x) * 16;
  v8i a, b;
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    a[k] = o[k];
    b[k] = o[8 + k];
  }
  v4f acc[8];
#pragma unroll
  for (int k = 0; k < 8; ++k) acc[k] = v4f{0.f, 0.f, 0.f, 0.f};
  for (int i = 0; i < iters; ++i) {
#pragma unroll
    for (int k = 0; k < 8; ++k)
      acc[k] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, acc[k], FA, FB, 0, 127, 0, 127);
  }
  float s = 0.f;
#pragma unroll
  for (int k = 0; k < 8; ++k) s += acc[k][0] + acc[k][1] + acc[k][2] + acc[k][3];
  sink[blockIdx.x * 256 + threadIdx.x] = s;
}

// The GEMM's MFMA-phase pattern without its memory traffic: 512 threads
// (two waves per SIMD), operands read per lane from `ops` (random bits), one
// scale per lane; each iteration issues eight MFMAs with a zero accumulator
// input (one 128-K group's partial each), and after each one the four fp32
// FMAs that promote the partial of the MFMA two back into its accumulator
// with a per-lane scale.  PROMOTE = 0 drops the FMAs (the MFMAs alone).  The
// operands are made opaque once per iteration so that nothing is hoisted or
// merged, and every partial is used.
template <int PROMOTE>
__global__ void __launch_bounds__(512, 1) mfma_promote_probe_kernel(int iters, const int* __restrict__ ops,
                                                                    float* sink) {
  const int* o = ops + ((size_t)blockIdx.x * 512 + threadIdx.x) * 16;
  v8i a, b[8];
#pragma unroll
  for (int k = 0; k < 8; ++k) a[k] = o[k];
#pragma unroll
  for (int m = 0; m < 8; ++m) {
#pragma unroll
    for (int k = 0; k < 8; ++k) b[m][k] = o[8 + ((k + m) & 7)];
  }
  const float s = 1.0f + (float)(threadIdx.x & 7) * 0.125f;
  v4f p[8], acc[8];
#pragma unroll
  for (int m = 0; m < 8; ++m) p[m] = acc[m] = v4f{0.f, 0.f, 0.f, 0.f};
  for (int i = 0; i < iters; ++i) {
    asm volatile("" : "+v"(a));
#pragma unroll
    for (int m = 0; m < 8; ++m) asm volatile("" : "+v"(b[m]));
#pragma unroll
    for (int m = 0; m < 8; ++m) {
      const v4f z = {0.f, 0.f, 0.f, 0.f};
      const v4f r = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b[m], z, 4, 0, 0, 127, 0, 127);
      if (PROMOTE) {
        const int pm = (m + 6) & 7;
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[pm][j] = fmaf(s, p[pm][j], acc[pm][j]);
      } else {
        asm volatile("" :: "v"(r));
      }
      p[m] = r;
    }
  }
  float t = 0.f;
#pragma unroll
  for (int m = 0; m < 8; ++m) t += acc[m][0] + acc[m][1] + acc[m][2] + acc[m][3] + p[m][0];
  sink[blockIdx.x * 512 + threadIdx.x] = t;
}

__global__ void __launch_bounds__(256) read_probe_kernel(const v4i* __restrict__ p, size_t n16, int* sink) {
  constexpr int U = 8;
  v4i acc = {0, 0, 0, 0};
  const size_t stride = (size_t)gridDim.x * 256;
  size_t i = (size_t)blockIdx.x * 256 + threadIdx.x;
  for (; i + (U - 1) * stride < n16; i += U * stride) {
    v4i v[U];
#pragma unroll
    for (int u = 0; u < U; ++u) v[u] = __builtin_nontemporal_load(p + i + u * stride);
#pragma unroll
    for (int u = 0; u < U; ++u) acc ^= v[u];
  }
  for (; i < n16; i += stride) acc ^= p[i];
  const int r = acc[0] ^ acc[1] ^ acc[2] ^ acc[3];
  if (r == 0x5a5a5a5a) sink[0] = r;  // data dependent, practically never taken
}

}  // namespace

extern "C" int w4a8_probe_mfma(int fmt_a, int fmt_b, int iters, int blocks, float* sink_dev, void* stream) {
  if (!sink_dev) return W4A8_ERR_NULL;
  if (iters <= 0 || blocks <= 0) return W4A8_ERR_SHAPE;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (fmt_a == 4 && fmt_b == 0)
    hipLaunchKernelGGL((mfma_probe_kernel<4, 0>), dim3(blocks), dim3(256), 0, s, iters, sink_dev);
  else if (fmt_a == 0 && fmt_b == 0)
    hipLaunchKernelGGL((mfma_probe_kernel<0, 0>), dim3(blocks), dim3(256), 0, s, iters, sink_dev);
  else if (fmt_a == 4 && fmt_b == 4)
    hipLaunchKernelGGL((mfma_probe_kernel<4, 4>), dim3(blocks), dim3(256), 0, s, iters, sink_dev);
  else
    return W4A8_ERR_SHAPE;
  return hipGetLastError() == hipSuccess ? W4A8_OK : W4A8_ERR_HIP;
}

extern "C" int w4a8_probe_read(const void* buf_dev, size_t bytes, int blocks, int32_t* sink_dev, void* stream) {
  if (!buf_dev || !sink_dev) return W4A8_ERR_NULL;
  if (bytes == 0 || bytes % 16 || blocks <= 0) return W4A8_ERR_SHAPE;
  if (reinterpret_cast<uintptr_t>(buf_dev) % 16) return W4A8_ERR_ALIGN;
  hipLaunchKernelGGL(read_probe_kernel, dim3(blocks), dim3(256), 0, static_cast<hipStream_t>(stream),
                     static_cast<const v4i*>(buf_dev), bytes / 16, sink_dev);
  return hipGetLastError() == hipSuccess ? W4A8_OK : W4A8_ERR_HIP;
}

extern "C" int w4a8_probe_mfma_data(int fmt_a, int fmt_b, int iters, int blocks, const int32_t* ops_dev,
                                    float* sink_dev, void* stream) {
  if (!sink_dev || !ops_dev) return W4A8_ERR_NULL;
  if (iters <= 0 || blocks <= 0) return W4A8_ERR_SHAPE;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (fmt_a == 4 && fmt_b == 0)
    hipLaunchKernelGGL((mfma_probe_data_kernel<4, 0>), dim3(blocks), dim3(256), 0, s, iters, ops_dev, sink_dev);
  else if (fmt_a == 0 && fmt_b == 0)
    hipLaunchKernelGGL((mfma_probe_data_kernel<0, 0>), dim3(blocks), dim3(256), 0, s, iters, ops_dev, sink_dev);
  else if (fmt_a == 4 && fmt_b == 4)
    hipLaunchKernelGGL((mfma_probe_data_kernel<4, 4>), dim3(blocks), dim3(256), 0, s, iters, ops_dev, sink_dev);
  else
    return W4A8_ERR_SHAPE;
  return hipGetLastError() == hipSuccess ? W4A8_OK : W4A8_ERR_HIP;
}

extern "C" int w4a8_probe_mfma_promote(int promote, int iters, int blocks, const int32_t* ops_dev, float* sink_dev,
                                       void* stream) {
  if (!sink_dev || !ops_dev) return W4A8_ERR_NULL;
  if (iters <= 0 || blocks <= 0) return W4A8_ERR_SHAPE;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (promote)
    hipLaunchKernelGGL((mfma_promote_probe_kernel<1>), dim3(blocks), dim3(512), 0, s, iters, ops_dev, sink_dev);
  else
    hipLaunchKernelGGL((mfma_promote_probe_kernel<0>), dim3(blocks), dim3(512), 0, s, iters, ops_dev, sink_dev);
  return hipGetLastError() == hipSuccess ? W4A8_OK : W4A8_ERR_HIP;
}
