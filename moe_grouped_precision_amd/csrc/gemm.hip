// Grouped-contiguous W4A8 GEMM kernels for gfx950.
//
// C[r, n] = bf16( sum_g SA(r, g) * P_g[r, n] ),
// P_g[r, n] = sum_{k in group g} e4m3(A[r, k]) * e2m1(B[e, n, k]) * 2^(SB[e, n, k/32] - 127)
// (humming PR #129, "Results" command: FP8 E4M3 activations with fp32 scales
// per 128 K, MXFP4 weights with E8M0 scales per 32 K, bf16 output.)
//
// One 128-K group is exactly one v_mfma_scale_f32_16x16x128_f8f6f4: the
// weights are the MFMA's A operand (16 output columns n per block, FP4, their
// E8M0 scales go through the instruction's A-scale operand), the activations
// are its B operand (16 rows m per block, FP8, unit scale).  The fp32
// activation scale is not a power of two, so each group's 16x16 partial is
// promoted with one fp32 FMA per element into the accumulator.  With this
// orientation every lane's four outputs share one row m, i.e. one scale.
//
// Operand fragments per lane (lane = 16*q + i, q = lane / 16):
//   FP4 weights   : column n = i, K = 32q .. 32q+31 of the group, 16 bytes,
//                   even K in the low nibble -- exactly the stored bytes.
//   FP8 activation: row m = i, K = 16q .. 16q+15 (bytes 0-15) and
//                   K = 64+16q .. 64+16q+15 (bytes 16-31).
//   weight scale  : lane supplies the E8M0 code of (column i, 32-K block q).
//   result        : lane holds rows-of-D 4q .. 4q+3 (= columns n) of column i
//                   (= row m), i.e. four consecutive n of one output row.
//
// Two kernels share the plan rule of w4a8_device.h:
//   gemm_stream_kernel  experts with <= S_MAX rows: weight streaming, one wave
//                       per (expert, 32-column) item, fragments loaded straight
//                       from global memory with a 4-deep prefetch ring (the
//                       weights are read from HBM exactly once);
//   gemm_mfma_kernel    larger experts: 256(n) x 128(m) workgroup tiles staged
//                       through LDS (XOR-swizzled, double buffered).
#include "w4a8_device.h"
#include "w4a8_launch.h"

namespace w4a8 {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));

__device__ __forceinline__ v4f mfma_group(v4i w, v4i x_lo, v4i x_hi, int sb) {
  v8i a = {w[0], w[1], w[2], w[3], 0, 0, 0, 0};
  v8i b = {x_lo[0], x_lo[1], x_lo[2], x_lo[3], x_hi[0], x_hi[1], x_hi[2], x_hi[3]};
  v4f z = {0.f, 0.f, 0.f, 0.f};
  // fmtA = 4 (E2M1), fmtB = 0 (E4M3); A scale = weight E8M0 code, B scale = 2^0
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, z, 4, 0, 0, sb, 0, 127);
}

__device__ __forceinline__ void promote(v4f& acc, float s, v4f p) {
  acc[0] = fmaf(s, p[0], acc[0]);
  acc[1] = fmaf(s, p[1], acc[1]);
  acc[2] = fmaf(s, p[2], acc[2]);
  acc[3] = fmaf(s, p[3], acc[3]);
}

__device__ __forceinline__ void store_bf16x4(uint16_t* dst, v4f v) {
  uint2 o;
  o.x = bf16_rne(v[0]) | (bf16_rne(v[1]) << 16);
  o.y = bf16_rne(v[2]) | (bf16_rne(v[3]) << 16);
  *reinterpret_cast<uint2*>(dst) = o;
}


// ---------------------------------------------------------------------------
// Weight-streaming kernel (small experts)
// ---------------------------------------------------------------------------
constexpr int STREAM_DEPTH = 4;

template <int MB>
struct StreamStage {
  v4i w[2];
  int s[2];
  v4i x[MB][2];
  float a[MB];
};

template <int MB>
__device__ void stream_item(const GemmArgs& p, int e, int row0, int rows, int n0, int R) {
  const int lane = threadIdx.x & 63;
  const int q = lane >> 4, r16 = lane & 15;
  const int K = p.K, N = p.N;
  const int G = K >> 7;

  const uint8_t* wp[2];
  const uint8_t* sp[2];
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const size_t col = (size_t)e * N + n0 + j * 16 + r16;
    wp[j] = p.B + col * (size_t)(K >> 1) + q * 16;
    sp[j] = p.SB + col * (size_t)(K >> 5) + q;
  }
  const uint8_t* xp[MB];
  const float* ap[MB];
  bool xv[MB];
  const size_t astride = p.layout == 0 ? 1 : (size_t)R;
#pragma unroll
  for (int i = 0; i < MB; ++i) {
    const int m = i * 16 + r16;
    xv[i] = m < rows;
    const size_t row = (size_t)row0 + (xv[i] ? m : 0);
    xp[i] = p.A + row * (size_t)K + q * 16;
    ap[i] = p.layout == 0 ? p.SA + row * (size_t)G : p.SA + row;
  }

  StreamStage<MB> st[STREAM_DEPTH];
  auto load = [&](StreamStage<MB>& S, int g) {
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      S.w[j] = __builtin_nontemporal_load(reinterpret_cast<const v4i*>(wp[j] + (size_t)g * 64));
      S.s[j] = sp[j][g * 4];
    }
#pragma unroll
    for (int i = 0; i < MB; ++i) {
      if (xv[i]) {
        const uint8_t* src = xp[i] + (size_t)g * 128;
        S.x[i][0] = *reinterpret_cast<const v4i*>(src);
        S.x[i][1] = *reinterpret_cast<const v4i*>(src + 64);
        S.a[i] = ap[i][(size_t)g * astride];
      } else {
        S.x[i][0] = v4i{0, 0, 0, 0};
        S.x[i][1] = v4i{0, 0, 0, 0};
        S.a[i] = 0.f;
      }
    }
  };

  v4f acc[2][MB];
#pragma unroll
  for (int j = 0; j < 2; ++j)
#pragma unroll
    for (int i = 0; i < MB; ++i) acc[j][i] = v4f{0.f, 0.f, 0.f, 0.f};

#pragma unroll
  for (int s = 0; s < STREAM_DEPTH; ++s)
    if (s < G) load(st[s], s);

  for (int g0 = 0; g0 < G; g0 += STREAM_DEPTH) {
#pragma unroll
    for (int s = 0; s < STREAM_DEPTH; ++s) {
      const int g = g0 + s;
      if (g < G) {
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
          for (int i = 0; i < MB; ++i)
            promote(acc[j][i], st[s].a[i], mfma_group(st[s].w[j], st[s].x[i][0], st[s].x[i][1], st[s].s[j]));
        if (g + STREAM_DEPTH < G) load(st[s], g + STREAM_DEPTH);
      }
    }
  }

#pragma unroll
  for (int i = 0; i < MB; ++i) {
    const int m = i * 16 + r16;
    if (m < rows) {
      uint16_t* crow = p.C + (size_t)(row0 + m) * N + n0 + q * 4;
#pragma unroll
      for (int j = 0; j < 2; ++j) store_bf16x4(crow + j * 16, acc[j][i]);
    }
  }
}

__global__ void __launch_bounds__(256)
gemm_stream_kernel(GemmArgs p) {
  __shared__ int s_off[MAX_EXPERTS + 1];
  __shared__ int s_base[MAX_EXPERTS + 1];
  __shared__ int s_wave[4];
  if (!plan_prologue(p.offsets, p.E, CLASS_STREAM, s_off, s_base, s_wave)) return;
  const int tiles = s_base[p.E];
  const int nb = p.N / TN_STREAM;
  const long long items = (long long)tiles * nb;
  const long long nw = (long long)gridDim.x * (blockDim.x >> 6);
  const int R = s_off[p.E];
  for (long long it = (long long)blockIdx.x * (blockDim.x >> 6) + (threadIdx.x >> 6); it < items;
       it += nw) {
    const int mt = (int)(it / nb);
    const int n0 = (int)(it % nb) * TN_STREAM;
    const int e = expert_of_tile(s_base, p.E, mt);
    const int row0 = s_off[e];
    const int rows = s_off[e + 1] - row0;
    switch ((rows + 15) >> 4) {
      case 1: stream_item<1>(p, e, row0, rows, n0, R); break;
      case 2: stream_item<2>(p, e, row0, rows, n0, R); break;
      case 3: stream_item<3>(p, e, row0, rows, n0, R); break;
      default: stream_item<4>(p, e, row0, rows, n0, R); break;
    }
  }
}

// ---------------------------------------------------------------------------
// MFMA kernel (larger experts): 256(n) x 128(m) tiles through LDS
// ---------------------------------------------------------------------------
constexpr int MF_BN = TN_MFMA;  // 256 weight columns
constexpr int MF_BM = T_MAX;    // 128 activation rows

struct MfStage {
  uint8_t w[MF_BN * 64];   // [n][64 B]  16-B chunks XOR-swizzled by (n >> 1) & 3
  uint8_t x[MF_BM * 128];  // [m][128 B] 16-B chunks XOR-swizzled by m & 7
  uint32_t sb[MF_BN];      // the 4 E8M0 codes of this group, per column
  float sa[MF_BM];         // activation scale of this group, per row
};

__device__ __forceinline__ int w_off(int n, int ch) { return n * 64 + ((ch ^ ((n >> 1) & 3)) << 4); }
__device__ __forceinline__ int x_off(int m, int ch) { return m * 128 + ((ch ^ (m & 7)) << 4); }

struct MfRegs {
  v4i w[4];
  v4i x[4];
  uint32_t sb;
  float sa;
};

__device__ __forceinline__ void mf_load(const GemmArgs& p, MfRegs& r, int e, int row0, int rows,
                                        int n0, int g, int R) {
  const int tid = threadIdx.x;
  const int K = p.K, N = p.N;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int c = tid + 256 * i;
    const int n = c >> 2, ch = c & 3;
    if (n0 + n < N) {
      const uint8_t* src = p.B + ((size_t)e * N + n0 + n) * (size_t)(K >> 1) + (size_t)g * 64 + ch * 16;
      r.w[i] = *reinterpret_cast<const v4i*>(src);
    } else {
      r.w[i] = v4i{0, 0, 0, 0};
    }
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int c = tid + 256 * i;
    const int m = c >> 3, ch = c & 7;
    if (m < rows) {
      const uint8_t* src = p.A + (size_t)(row0 + m) * (size_t)K + (size_t)g * 128 + ch * 16;
      r.x[i] = *reinterpret_cast<const v4i*>(src);
    } else {
      r.x[i] = v4i{0, 0, 0, 0};
    }
  }
  {
    const int n = tid;
    r.sb = (n0 + n < N)
               ? *reinterpret_cast<const uint32_t*>(p.SB + ((size_t)e * N + n0 + n) * (size_t)(K >> 5) + g * 4)
               : 0x7f7f7f7fu;
  }
  {
    const int m = tid;
    float s = 0.f;
    if (m < MF_BM && m < rows) {
      const size_t row = (size_t)row0 + m;
      s = p.layout == 0 ? p.SA[row * (size_t)(K >> 7) + g] : p.SA[(size_t)g * R + row];
    }
    r.sa = s;
  }
}

__device__ __forceinline__ void mf_store(MfStage& s, const MfRegs& r) {
  const int tid = threadIdx.x;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int c = tid + 256 * i;
    *reinterpret_cast<v4i*>(s.w + w_off(c >> 2, c & 3)) = r.w[i];
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int c = tid + 256 * i;
    *reinterpret_cast<v4i*>(s.x + x_off(c >> 3, c & 7)) = r.x[i];
  }
  s.sb[tid] = r.sb;
  if (tid < MF_BM) s.sa[tid] = r.sa;
}

__device__ void mfma_tile(const GemmArgs& p, MfStage* stg, int e, int row0, int rows, int n0, int R) {
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int wn = wave & 1, wm = wave >> 1;
  const int q = lane >> 4, r16 = lane & 15;
  const int G = p.K >> 7;

  v4f acc[4][8];
#pragma unroll
  for (int a = 0; a < 4; ++a)
#pragma unroll
    for (int b = 0; b < 8; ++b) acc[a][b] = v4f{0.f, 0.f, 0.f, 0.f};

  MfRegs r;
  mf_load(p, r, e, row0, rows, n0, 0, R);
  mf_store(stg[0], r);
  __syncthreads();

  for (int g = 0; g < G; ++g) {
    const int cur = g & 1;
    if (g + 1 < G) mf_load(p, r, e, row0, rows, n0, g + 1, R);
    const MfStage& s = stg[cur];
    v4i wf[8];
    int sbv[8];
#pragma unroll
    for (int nb = 0; nb < 8; ++nb) {
      const int n = wn * 128 + nb * 16 + r16;
      wf[nb] = *reinterpret_cast<const v4i*>(s.w + w_off(n, q));
      sbv[nb] = (int)((s.sb[n] >> (8 * q)) & 0xffu);
    }
#pragma unroll
    for (int mi = 0; mi < 4; ++mi) {
      const int mb = wm + 2 * mi;
      if (mb * 16 < rows) {
        const int m = mb * 16 + r16;
        const v4i x0 = *reinterpret_cast<const v4i*>(s.x + x_off(m, q));
        const v4i x1 = *reinterpret_cast<const v4i*>(s.x + x_off(m, q + 4));
        const float sa = s.sa[m];
#pragma unroll
        for (int nb = 0; nb < 8; ++nb) promote(acc[mi][nb], sa, mfma_group(wf[nb], x0, x1, sbv[nb]));
      }
    }
    if (g + 1 < G) mf_store(stg[cur ^ 1], r);
    __syncthreads();
  }

#pragma unroll
  for (int mi = 0; mi < 4; ++mi) {
    const int mb = wm + 2 * mi;
    const int m = mb * 16 + r16;
    if (m < rows) {
      uint16_t* crow = p.C + (size_t)(row0 + m) * p.N;
#pragma unroll
      for (int nb = 0; nb < 8; ++nb) {
        const int n = n0 + wn * 128 + nb * 16 + q * 4;
        if (n < p.N) store_bf16x4(crow + n, acc[mi][nb]);
      }
    }
  }
}

__global__ void __launch_bounds__(256)
gemm_mfma_kernel(GemmArgs p) {
  __shared__ MfStage stg[2];
  __shared__ int s_off[MAX_EXPERTS + 1];
  __shared__ int s_base[MAX_EXPERTS + 1];
  __shared__ int s_wave[4];
  if (!plan_prologue(p.offsets, p.E, CLASS_MFMA, s_off, s_base, s_wave)) return;
  const int tiles = s_base[p.E];
  const int nt_count = (p.N + MF_BN - 1) / MF_BN;
  const long long items = (long long)tiles * nt_count;
  const int R = s_off[p.E];
  for (long long it = blockIdx.x; it < items; it += gridDim.x) {
    const int mt = (int)(it / nt_count);
    const int n0 = (int)(it % nt_count) * MF_BN;
    const int e = expert_of_tile(s_base, p.E, mt);
    const int j = mt - s_base[e];
    const int rows_e = s_off[e + 1] - s_off[e];
    const TileChoice tc = tile_rule(rows_e);
    const int row0 = s_off[e] + j * tc.tile_m;
    const int rows = min(tc.tile_m, rows_e - j * tc.tile_m);
    mfma_tile(p, stg, e, row0, rows, n0, R);
  }
}

hipError_t launch_grouped_gemm(const GemmArgs& args, int grid_stream, int grid_mfma,
                               hipStream_t stream) {
  hipLaunchKernelGGL(gemm_stream_kernel, dim3(grid_stream), dim3(256), 0, stream, args);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(gemm_mfma_kernel, dim3(grid_mfma), dim3(256), 0, stream, args);
  return hipGetLastError();
}

hipError_t occupancy_blocks_per_cu(int* stream_blocks, int* mfma_blocks) {
  hipError_t e = hipOccupancyMaxActiveBlocksPerMultiprocessor(stream_blocks, gemm_stream_kernel, 256, 0);
  if (e != hipSuccess) return e;
  return hipOccupancyMaxActiveBlocksPerMultiprocessor(mfma_blocks, gemm_mfma_kernel, 256, 0);
}

}  // namespace w4a8
