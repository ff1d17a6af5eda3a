// Grouped-contiguous GEMM with bf16 activations and FP4 weights (A16) for
// gfx950: the BF16-activation FP4 paths humming PR #58 tunes ("Summary":
// the small-M FP4 paths of MXFP4/NVFP4 A16), on the grouped layout of the
// W4A8 path:
//
//   C[r, n] = bf16( gs[e] * sum_k A[r, k] * e2m1(B[e, n, k]) * s(e, n, k) )
//
// with s = 2^(code - 127) from an E8M0 code per 32 K (MXFP4) or the value
// of an E4M3 code per 16 K (NVFP4), and gs an fp32 scale per expert (1 when
// none is given).
//
// The FP4 weights are turned into bf16 in registers (exact: a 2-bit E2M1
// significand times a power of two or a 4-bit E4M3 significand has at most 6
// significant bits; with E8M0 scales by gfx950's scaled FP4 conversion, two
// weights per instruction) and multiplied on the matrix core in bf16
// (v_mfma_f32_16x16x16_bf16, fp32 accumulation).  The weight scale cannot
// ride in the instruction as the W4A8 path's E8M0 code does, so every weight
// element pays it in the conversion: this is the scale application the pages
// name as what dominates the remaining NVFP4 gap (humming PR #58, "H200
// performance", the BF16 FP4 expert-GEMM sweeps).
//
// Work: items (expert, 128 output columns) over a grid of workgroups of four
// waves; wave w owns columns 32 w .. 32 w + 31 of the item (two blocks of 16)
// and up to 64 of the expert's rows at a time (further rows in further
// passes over K, one code path per number of row blocks).  Per 128-K group
// and column block a lane loads 16 bytes of weights (column l % 16 of the
// block, K 32 q .. 32 q + 31, q = l / 16; two groups ahead), converts them,
// and the group's 8 MFMAs per row and column block
// take K in the order k = 32 q + 4 j + t (MFMA j, lane group q, element t):
// a lane's own 32 weights feed its 8 MFMAs, and the activation fragments
// follow the same order from LDS.  Activation rows are staged in LDS, two
// buffers, 16-byte chunk c of row r at c ^ (r & 15).
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "w4a8_launch.h"

namespace w4a8 {
namespace {

typedef float v4f __attribute__((ext_vector_type(4)));
typedef float v2f __attribute__((ext_vector_type(2)));
typedef __bf16 v2bf __attribute__((ext_vector_type(2)));
typedef short v4s __attribute__((ext_vector_type(4)));
typedef unsigned int v4u __attribute__((ext_vector_type(4)));
typedef unsigned int v2u __attribute__((ext_vector_type(2)));

constexpr int A16_THREADS = 256;
constexpr int A16_COLS = 128;                // output columns per item (32 per wave)
constexpr int A16_ROWS = 64;                 // rows per pass
constexpr int A16_ROW_BYTES = 256;           // 128 bf16 of one row per K group
constexpr int A16_BUF = A16_ROWS * A16_ROW_BYTES;   // 16 KB per buffer

// 8 E2M1 codes (one dword, element 2i in the low nibble of byte i) -> their
// fp32 values times the scale s, as bf16, packed two per dword: out[i] holds
// elements 2i (low half) and 2i + 1 (high half).  The magnitudes come from
// byte tables through v_perm (the fp32 top byte and the one below it; E2M1
// magnitudes 0, 0.5, 1, 1.5, 2, 3, 4, 6 have zero lower bytes), the sign
// from bit 3 of the nibble.  Every product is exact in fp32, so dropping the
// low half of its bits is exact too.
__device__ __forceinline__ void e2m1x8_to_bf16(uint32_t x, float s, uint32_t (&out)[4]) {
  const uint32_t m_lo = x & 0x07070707u;          // magnitude codes of elements 0, 2, 4, 6
  const uint32_t m_hi = (x >> 4) & 0x07070707u;   // elements 1, 3, 5, 7
  // byte tables: index 0..3 from the second operand, 4..7 from the first
  const uint32_t t_lo = __builtin_amdgcn_perm(0x40404040u, 0x3F3F3F00u, m_lo) | ((x << 4) & 0x80808080u);
  const uint32_t t_hi = __builtin_amdgcn_perm(0x40404040u, 0x3F3F3F00u, m_hi) | (x & 0x80808080u);
  const uint32_t b_lo = __builtin_amdgcn_perm(0xC0804000u, 0xC0800000u, m_lo);
  const uint32_t b_hi = __builtin_amdgcn_perm(0xC0804000u, 0xC0800000u, m_hi);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    // fp32 bytes {0, 0, b byte i, t byte i} (selector 0x0C gives a zero byte)
    const uint32_t sel = 0x0C0Cu | ((uint32_t)i << 16) | ((uint32_t)(4 + i) << 24);
    const float lo = __builtin_bit_cast(float, __builtin_amdgcn_perm(t_lo, b_lo, sel)) * s;
    const float hi = __builtin_bit_cast(float, __builtin_amdgcn_perm(t_hi, b_hi, sel)) * s;
    // the top halves: bf16 of lo in bits 15:0, of hi in bits 31:16
    out[i] = __builtin_amdgcn_perm(__builtin_bit_cast(uint32_t, hi), __builtin_bit_cast(uint32_t, lo), 0x07060302u);
  }
}

// The same for a power-of-two scale s (MXFP4's 2^(code - 127), the subnormal
// 2^-127 and NaN included): gfx950's scaled conversion turns the two codes
// of one byte into bf16 times s in one instruction, low nibble into the low
// half.  It takes only the exponent of s, so E4M3 scales (NVFP4) go through
// e2m1x8_to_bf16.  Every product is exact in bf16 (2 significant bits).
__device__ __forceinline__ void e2m1x8_to_bf16_pow2(uint32_t x, float s, uint32_t (&out)[4]) {
  out[0] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(x, s, 0));
  out[1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(x, s, 1));
  out[2] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(x, s, 2));
  out[3] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(x, s, 3));
}

// E4M3FN code -> fp32 (exact; 0x7F / 0xFF NaN).
__device__ __forceinline__ float e4m3_to_f32(uint32_t c) {
  const uint32_t e = (c >> 3) & 0xF, m = c & 7;
  float v;
  if (e == 0)
    v = (float)m * 0.001953125f;                      // m / 8 * 2^-6
  else
    v = __builtin_bit_cast(float, ((e + 120u) << 23) | (m << 20));
  if ((c & 0x7F) == 0x7F) v = __builtin_nanf("");
  return (c & 0x80) ? -v : v;
}

// E8M0 code -> fp32 2^(c - 127) (code 0: 2^-127, a subnormal; 0xFF NaN).
__device__ __forceinline__ float e8m0_to_f32(uint32_t c) {
  if (c == 0xFF) return __builtin_nanf("");
  if (c == 0) return __builtin_bit_cast(float, 0x00400000u);
  return __builtin_bit_cast(float, c << 23);
}

// One pass over K for rows r0 .. r0 + rows - 1 (NRB = ceil(rows / 16) row
// blocks) of expert e and the lane's two weight columns: activations staged
// in LDS one group ahead, weights and their scale codes loaded two groups
// ahead in registers.
template <int FMT, int NRB>
__device__ __forceinline__ void a16_pass(const uint16_t* __restrict__ A, const uint8_t* const (&wcol)[2],
                                         const uint8_t* const (&scol)[2], const bool (&wvalid)[2], float gs,
                                         int r0, int rows, int K, int N, int col0, uint8_t* lds,
                                         uint16_t* __restrict__ C) {
  constexpr int SPG = FMT == 0 ? 4 : 8;       // scale codes per column per K group
  const int lane = threadIdx.x & 63;
  const int q = lane >> 4, c16 = lane & 15;
  const int G = K >> 7;
  // activation staging: the pass's row blocks x 16 chunks of 16 bytes per
  // group, NRB per thread (rows past `rows` inside the last block re-read
  // the last row)
  auto load_act = [&](int g, v4u (&ra)[NRB]) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < NRB; ++i) {
      const int ch = threadIdx.x + i * A16_THREADS;
      const int rr = min(ch >> 4, rows - 1);
      ra[i] = *reinterpret_cast<const v4u*>(A + (size_t)(r0 + rr) * K + (size_t)g * 128 + (ch & 15) * 8);
    }
  };
  auto store_act = [&](int buf, const v4u (&ra)[NRB]) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < NRB; ++i) {
      const int ch = threadIdx.x + i * A16_THREADS;
      const int rr = ch >> 4;
      *reinterpret_cast<v4u*>(lds + buf * A16_BUF + rr * A16_ROW_BYTES + (((ch & 15) ^ (rr & 15)) << 4)) = ra[i];
    }
  };
  auto load_w = [&](int g, v4u (&w)[2], uint32_t (&sc)[2]) __attribute__((always_inline)) {
    const int gc = min(g, G - 1);   // past the last group: re-read it (never used)
#pragma unroll
    for (int cb = 0; cb < 2; ++cb) {
      w[cb] = *reinterpret_cast<const v4u*>(wcol[cb] + (size_t)gc * 64);
      if (FMT == 0)
        sc[cb] = scol[cb][gc * SPG + q];
      else
        sc[cb] = *reinterpret_cast<const uint16_t*>(scol[cb] + gc * SPG + 2 * q);
    }
  };

  v4f acc[NRB][2];
#pragma unroll
  for (int rb = 0; rb < NRB; ++rb)
#pragma unroll
    for (int cb = 0; cb < 2; ++cb) acc[rb][cb] = v4f{0.f, 0.f, 0.f, 0.f};
  v4u ra[NRB], w0[2], w1[2];
  uint32_t s0c[2], s1c[2];
  load_act(0, ra);
  load_w(0, w0, s0c);
  load_w(1, w1, s1c);
  store_act(0, ra);
  __syncthreads();
  for (int g = 0; g < G; ++g) {
    const int buf = g & 1;
    if (g + 1 < G) load_act(g + 1, ra);
    v4u w2[2];
    uint32_t s2c[2];
    load_w(g + 2, w2, s2c);
    // this group's weights as bf16 MFMA operands: wb[cb][2j], wb[cb][2j+1] = k 32q + 4j .. +3
    uint32_t wb[2][16];
#pragma unroll
    for (int cb = 0; cb < 2; ++cb) {
      const float sa = FMT == 0 ? e8m0_to_f32(s0c[cb]) : e4m3_to_f32(s0c[cb] & 0xFF);
      const float sb = FMT == 0 ? sa : e4m3_to_f32(s0c[cb] >> 8);
#pragma unroll
      for (int d = 0; d < 4; ++d) {
        uint32_t t[4];
        if (FMT == 0)
          e2m1x8_to_bf16_pow2(w0[cb][d], sa, t);
        else
          e2m1x8_to_bf16(w0[cb][d], d < 2 ? sa : sb, t);
#pragma unroll
        for (int i = 0; i < 4; ++i) wb[cb][4 * d + i] = t[i];
      }
    }
    const uint8_t* ab = lds + buf * A16_BUF;
#pragma unroll
    for (int rb = 0; rb < NRB; ++rb) {
      const int r = rb * 16 + c16;
      const uint8_t* arow = ab + r * A16_ROW_BYTES;
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) {
        // MFMAs 2 jj and 2 jj + 1 read bytes 64 q + 16 jj .. +15 of the row (chunk 4 q + jj)
        const v4u x = *reinterpret_cast<const v4u*>(arow + (((4 * q + jj) ^ (r & 15)) << 4));
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          const int j = 2 * jj + h;
          const v4s b = __builtin_bit_cast(v4s, v2u{x[2 * h], x[2 * h + 1]});
#pragma unroll
          for (int cb = 0; cb < 2; ++cb) {
            const v4s a = __builtin_bit_cast(v4s, v2u{wb[cb][2 * j], wb[cb][2 * j + 1]});
            acc[rb][cb] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a, b, acc[rb][cb], 0, 0, 0);
          }
        }
      }
    }
    if (g + 1 < G) store_act(buf ^ 1, ra);
#pragma unroll
    for (int cb = 0; cb < 2; ++cb) {
      w0[cb] = w1[cb];
      s0c[cb] = s1c[cb];
      w1[cb] = w2[cb];
      s1c[cb] = s2c[cb];
    }
    __syncthreads();
  }
  // D[n][m] of each (row block, column block): lane holds columns 4q .. 4q+3
  // of the block for row c16 of the row block
  const int wave = threadIdx.x >> 6;
#pragma unroll
  for (int rb = 0; rb < NRB; ++rb) {
    const int m = rb * 16 + c16;
    if (m < rows) {
#pragma unroll
      for (int cb = 0; cb < 2; ++cb) {
        if (wvalid[cb]) {
          const v4f o = acc[rb][cb] * gs;
          v2u pk;
          pk[0] = __builtin_bit_cast(uint32_t, __builtin_convertvector((v2f){o[0], o[1]}, v2bf));
          pk[1] = __builtin_bit_cast(uint32_t, __builtin_convertvector((v2f){o[2], o[3]}, v2bf));
          *reinterpret_cast<v2u*>(C + (size_t)(r0 + m) * N + col0 + wave * 32 + cb * 16 + 4 * q) = pk;
        }
      }
    }
  }
}

template <int FMT>
__global__ void __launch_bounds__(A16_THREADS)
grouped_gemm_a16_kernel(const uint16_t* __restrict__ A, const uint8_t* __restrict__ B,
                        const uint8_t* __restrict__ SB, const float* __restrict__ GS,
                        const int32_t* __restrict__ offsets, int E, int N, int K, uint16_t* __restrict__ C) {
  __shared__ __attribute__((aligned(16))) uint8_t lds[2 * A16_BUF];
  __shared__ int s_bad;
  // offsets must start at 0 and never decrease; otherwise nothing is written
  if (threadIdx.x == 0) s_bad = offsets[0] != 0;
  __syncthreads();
  for (int e = threadIdx.x; e < E; e += A16_THREADS)
    if (offsets[e + 1] < offsets[e]) s_bad = 1;
  __syncthreads();
  if (s_bad) return;

  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int c16 = lane & 15, q = lane >> 4;
  const int NB = (N + A16_COLS - 1) / A16_COLS;
  const int items = E * NB;
  for (int it = blockIdx.x; it < items; it += gridDim.x) {
    const int e = it / NB, nb = it - e * NB;
    const int lo = offsets[e], hi = offsets[e + 1];
    // this lane's two weight columns (blocks cb = 0, 1 of the wave's 32);
    // N % 16 == 0, so a block's 16 columns are all in or all out
    const uint8_t* wcol[2];
    const uint8_t* scol[2];
    bool wvalid[2];
#pragma unroll
    for (int cb = 0; cb < 2; ++cb) {
      const int nblk = nb * A16_COLS + wave * 32 + cb * 16;
      wvalid[cb] = nblk < N;
      const int ncl = min(nblk + c16, N - 1);
      wcol[cb] = B + ((size_t)e * N + ncl) * (size_t)(K >> 1) + q * 16;
      scol[cb] = SB + ((size_t)e * N + ncl) * (size_t)(FMT == 0 ? K >> 5 : K >> 4);
    }
    const float gs = GS ? GS[e] : 1.0f;
    for (int r0 = lo; r0 < hi; r0 += A16_ROWS) {
      const int rows = min(A16_ROWS, hi - r0);
      switch ((rows + 15) >> 4) {
        case 1: a16_pass<FMT, 1>(A, wcol, scol, wvalid, gs, r0, rows, K, N, nb * A16_COLS, lds, C); break;
        case 2: a16_pass<FMT, 2>(A, wcol, scol, wvalid, gs, r0, rows, K, N, nb * A16_COLS, lds, C); break;
        case 3: a16_pass<FMT, 3>(A, wcol, scol, wvalid, gs, r0, rows, K, N, nb * A16_COLS, lds, C); break;
        default: a16_pass<FMT, 4>(A, wcol, scol, wvalid, gs, r0, rows, K, N, nb * A16_COLS, lds, C); break;
      }
    }
  }
}

}  // namespace

hipError_t launch_grouped_gemm_a16(const uint16_t* A, const uint8_t* B, const uint8_t* SB, int fmt, const float* GS,
                                   const int32_t* offsets, int E, int N, int K, uint16_t* C, int grid,
                                   hipStream_t stream) {
  if (fmt == 0)
    hipLaunchKernelGGL(grouped_gemm_a16_kernel<0>, dim3(grid), dim3(A16_THREADS), 0, stream, A, B, SB, GS, offsets, E,
                       N, K, C);
  else
    hipLaunchKernelGGL(grouped_gemm_a16_kernel<1>, dim3(grid), dim3(A16_THREADS), 0, stream, A, B, SB, GS, offsets, E,
                       N, K, C);
  return hipGetLastError();
}

}  // namespace w4a8
