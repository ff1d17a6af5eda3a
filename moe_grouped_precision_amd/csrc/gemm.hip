// Grouped-contiguous W4A8 GEMM kernel for gfx950.
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
// One persistent launch of 512 threads (8 waves) per CU, two phases over the
// tile plan of w4a8_device.h.  Both phases stream their operands through LDS
// with direct global->LDS loads (global_load_lds_dwordx4 / _dword), which keep
// no data in registers while in flight:
//   * a 4-slot ring holds one K group of weights and activations per slot;
//     every wave issues the same number of ring loads per stage, waits for
//     the stage it needs with an explicit vmcnt and meets the others at one
//     barrier per stage, so three stages are in flight at all times;
//   * the E8M0 and activation scales are loaded four groups at a time (four
//     lanes read 16 contiguous bytes) into a double buffer, so that they cost
//     a small fraction of the memory requests of the weights;
//   * the XOR swizzle that keeps fragment reads free of LDS bank conflicts is
//     applied on the global-address side (a load lane always writes slot
//     base + size * lane).
// Phases:
//   1. streaming items (experts with <= S_MAX rows): one workgroup per
//      (expert, 64 or 128 columns); waves 0-3 take the first half of the K
//      groups and waves 4-7 the second half, each wave 16 or 32 columns; the
//      halves are added in LDS (always half 0 + half 1) before the bf16 store.
//   2. MFMA tiles (larger experts): 256(n) x 128(m) per workgroup, one K group
//      per stage; each wave owns 64(n) x 64(m).
#include "w4a8_device.h"
#include "w4a8_launch.h"

namespace w4a8 {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));

constexpr int BLOCK = 512;
constexpr int WAVES = BLOCK / 64;
constexpr int NS = 4;                  // ring slots (NS-1 stages in flight)
constexpr int SLOT_BYTES = 32768;      // one K group: weights 16 KB + activations 16 KB
constexpr int SLOT_X = 0;              // activation rows
constexpr int SLOT_W = 16384;          // weight columns
constexpr int SC = 4;                  // groups per scale chunk
constexpr int SB_BYTES = 4096;         // one scale chunk of E8M0 codes (1024 x u32)
constexpr int SA_BYTES = 2048;         // one scale chunk of activation scales (512 x fp32)
constexpr int LDS_SB = NS * SLOT_BYTES;          // 2 buffers
constexpr int LDS_SA = LDS_SB + 2 * SB_BYTES;    // 2 buffers
constexpr int LDS_BYTES = LDS_SA + 2 * SA_BYTES;

#define W4A8_GPTR(p) ((const __attribute__((address_space(1))) void*)(p))
#define W4A8_LPTR(p) ((__attribute__((address_space(3))) void*)(p))

// Each active lane copies 16 (or 4) bytes from its own global address to
// lds_wave_base + 16 * lane (or 4 * lane).  lds_wave_base must be wave-uniform.
__device__ __forceinline__ void dma16(const void* g, uint8_t* lds_wave_base) {
  __builtin_amdgcn_global_load_lds(W4A8_GPTR(g), W4A8_LPTR(lds_wave_base), 16, 0, 0);
}
__device__ __forceinline__ void dma4(const void* g, uint8_t* lds_wave_base) {
  __builtin_amdgcn_global_load_lds(W4A8_GPTR(g), W4A8_LPTR(lds_wave_base), 4, 0, 0);
}

// s_waitcnt with only the vector-memory counter constrained (gfx9 encoding:
// vmcnt bits 3:0 and 15:14, expcnt 6:4, lgkmcnt 11:8).
template <int N>
__device__ __forceinline__ void wait_vm() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

// Wait until at most `pending` later stages of PER_STAGE ring loads each are
// still in flight, then meet the other waves.  Scale-chunk loads issued with a
// later stage only make this wait stricter than needed, never looser.
template <int PER_STAGE>
__device__ __forceinline__ void stage_barrier(int pending) {
  static_assert((NS - 2) * PER_STAGE < 64, "too many loads in flight");
  if (pending >= 2) wait_vm<2 * PER_STAGE>();
  else if (pending == 1) wait_vm<PER_STAGE>();
  else wait_vm<0>();
  __builtin_amdgcn_s_barrier();
}

__device__ __forceinline__ int uniform(int v) { return __builtin_amdgcn_readfirstlane(v); }

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

__device__ __forceinline__ v4i lds128(const uint8_t* p) { return *reinterpret_cast<const v4i*>(p); }
__device__ __forceinline__ uint32_t lds32(const uint8_t* p) { return *reinterpret_cast<const uint32_t*>(p); }
__device__ __forceinline__ float ldsf(const uint8_t* p) { return *reinterpret_cast<const float*>(p); }

// Activation scale of (row, group) in either layout.
__device__ __forceinline__ const float* sa_ptr(const GemmArgs& p, size_t row, int g, int G, int R) {
  return p.layout == 0 ? p.SA + row * (size_t)G + g : p.SA + (size_t)g * R + row;
}

// ---------------------------------------------------------------------------
// Phase 1: weight streaming (experts with <= S_MAX rows)
//
// Stage s covers group gb[h] + s of each K half h (gb = {0, ceil(G/2)}).
// Ring slot:  X [2 halves][16*mb rows][128 B] @ SLOT_X   (row chunk c at c ^ (row & 7))
//             W [8 waves][NBW][16 cols][64 B] @ SLOT_W   (col chunk c at c ^ ((col >> 1) & 3))
// Scale chunk c (stages SC*c .. SC*c+3):
//             SB [2 halves][128 cols][SC] u32;  SA [2 halves][64 rows][SC] fp32
// ---------------------------------------------------------------------------
template <int NBW>
struct StreamItem {
  static constexpr int WIDTH = 4 * NBW * 16;  // columns per item

  // Ring loads of stage s: NBW (W) + mb (X) per wave.
  __device__ __forceinline__ static void issue_stage(const GemmArgs& p, uint8_t* slot, int e,
                                                     int row0, int rows, int mb, int n0, int s) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int kh = wave >> 2, wn = wave & 3;
    const int K = p.K, N = p.N, G = K >> 7;
    const int g0 = min(s, G - 1), g1 = min((G + 1) / 2 + s, G - 1);  // group of each K half
    const int gk = kh ? g1 : g0;
#pragma unroll
    for (int j = 0; j < NBW; ++j) {  // 16 cols x 64 B
      const int r = lane >> 2;
      const int c = (lane & 3) ^ ((r >> 1) & 3);
      const int n = min(n0 + (wn * NBW + j) * 16 + r, N - 1);
      dma16(p.B + ((size_t)e * N + n) * (size_t)(K >> 1) + (size_t)gk * 64 + c * 16,
            slot + SLOT_W + (wave * NBW + j) * 1024);
    }
    for (int i = 0; i < mb; ++i) {  // 8*mb loads of 4 rows x 128 B
      if (lane < 32) {
        const int jx = wave * mb + i;
        const int h = jx / (4 * mb), quad = jx - h * (4 * mb);
        const int r = quad * 4 + (lane >> 3);
        const int c = (lane & 7) ^ (r & 7);
        const size_t row = (size_t)row0 + min(r, rows - 1);
        dma16(p.A + row * (size_t)K + (size_t)(h ? g1 : g0) * 128 + c * 16,
              slot + SLOT_X + h * (mb * 16 * 128) + quad * 512);
      }
    }
  }

  // Scale chunk c: 2 SB + 1 SA loads per wave.
  __device__ __forceinline__ static void issue_scales(const GemmArgs& p, uint8_t* lds, int e,
                                                      int row0, int rows, int n0, int c, int R) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int K = p.K, N = p.N, G = K >> 7;
    const int gb1 = (G + 1) / 2;
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int idx = (wave * 2 + i) * 64 + lane;  // [h][col][gg]
      const int h = idx >> 9, col = (idx >> 2) & 127, gg = idx & 3;
      const int n = min(n0 + col, N - 1);
      const int g = min((h ? gb1 : 0) + SC * c + gg, G - 1);
      dma4(p.SB + ((size_t)e * N + n) * (size_t)(K >> 5) + (size_t)g * 4,
           lds + LDS_SB + (c & 1) * SB_BYTES + (wave * 2 + i) * 256);
    }
    {
      const int idx = wave * 64 + lane;  // [h][row][gg]
      const int h = idx >> 8, r = (idx >> 2) & 63, gg = idx & 3;
      const size_t row = (size_t)row0 + min(r, rows - 1);
      const int g = min((h ? gb1 : 0) + SC * c + gg, G - 1);
      dma4(sa_ptr(p, row, g, G, R), lds + LDS_SA + (c & 1) * SA_BYTES + wave * 256);
    }
  }

  __device__ __forceinline__ static void run(const GemmArgs& p, uint8_t* lds, int e, int row0,
                                             int rows, int n0, int R) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int kh = wave >> 2, wn = wave & 3;
    const int q = lane >> 4, r16 = lane & 15;
    const int G = p.K >> 7;
    const int Gh = (G + 1) / 2;
    const int gcount = kh == 0 ? Gh : G - Gh;  // groups of this wave's half
    const int S = Gh;
    const int mb = (rows + 15) >> 4;             // 1..4 row blocks

    v4f acc[NBW][4];
#pragma unroll
    for (int j = 0; j < NBW; ++j)
#pragma unroll
      for (int i = 0; i < 4; ++i) acc[j][i] = v4f{0.f, 0.f, 0.f, 0.f};

    wait_vm<0>();  // earlier stores must not be counted against this item's loads
#pragma unroll
    for (int s = 0; s < NS - 1; ++s) {
      if (s < S) {
        if (s % SC == 0) issue_scales(p, lds, e, row0, rows, n0, s / SC, R);
        issue_stage(p, lds + s * SLOT_BYTES, e, row0, rows, mb, n0, s);
      }
    }

    for (int s = 0; s < S; ++s) {
      switch (mb) {
        case 1: stage_barrier<NBW + 1>(min(NS - 2, S - 1 - s)); break;
        case 2: stage_barrier<NBW + 2>(min(NS - 2, S - 1 - s)); break;
        case 3: stage_barrier<NBW + 3>(min(NS - 2, S - 1 - s)); break;
        default: stage_barrier<NBW + 4>(min(NS - 2, S - 1 - s)); break;
      }
      const int sn = s + NS - 1;
      if (sn < S) {
        if (sn % SC == 0) issue_scales(p, lds, e, row0, rows, n0, sn / SC, R);
        issue_stage(p, lds + (sn % NS) * SLOT_BYTES, e, row0, rows, mb, n0, sn);
      }
      if (s < gcount) {
        const uint8_t* slot = lds + (s % NS) * SLOT_BYTES;
        const uint8_t* sbb = lds + LDS_SB + ((s / SC) & 1) * SB_BYTES;
        const uint8_t* sab = lds + LDS_SA + ((s / SC) & 1) * SA_BYTES;
        const int gg = s % SC;
        v4i wf[NBW];
        int sbv[NBW];
#pragma unroll
        for (int j = 0; j < NBW; ++j) {
          const int col = (wn * NBW + j) * 16 + r16;
          wf[j] = lds128(slot + SLOT_W + (wave * NBW + j) * 1024 + r16 * 64 + ((q ^ ((r16 >> 1) & 3)) << 4));
          sbv[j] = (int)((lds32(sbb + ((kh * 128 + col) * SC + gg) * 4) >> (8 * q)) & 0xffu);
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          if (i < mb) {
            const int m = i * 16 + r16;
            const uint8_t* xb = slot + SLOT_X + kh * (mb * 16 * 128) + m * 128;
            const v4i x0 = lds128(xb + ((q ^ (m & 7)) << 4));
            const v4i x1 = lds128(xb + (((q + 4) ^ (m & 7)) << 4));
            const float sa = ldsf(sab + ((kh * 64 + m) * SC + gg) * 4);
#pragma unroll
            for (int j = 0; j < NBW; ++j) promote(acc[j][i], sa, mfma_group(wf[j], x0, x1, sbv[j]));
          }
        }
      }
    }

    // add the two K halves in LDS (the ring is free: every wave passed the last
    // stage barrier with nothing in flight) and store
    __syncthreads();
    v4f* red = reinterpret_cast<v4f*>(lds);
    if (kh == 1) {
#pragma unroll
      for (int j = 0; j < NBW; ++j)
#pragma unroll
        for (int i = 0; i < 4; ++i)
          if (i < mb) red[((wn * NBW + j) * 4 + i) * 64 + lane] = acc[j][i];
    }
    __syncthreads();
    if (kh == 0) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int m = i * 16 + r16;
        if (i < mb && m < rows) {
          uint16_t* crow = p.C + (size_t)(row0 + m) * p.N;
#pragma unroll
          for (int j = 0; j < NBW; ++j) {
            const int n = n0 + (wn * NBW + j) * 16 + q * 4;
            const v4f o = red[((wn * NBW + j) * 4 + i) * 64 + lane];
            if (n < p.N) store_bf16x4(crow + n, acc[j][i] + o);
          }
        }
      }
    }
    __syncthreads();  // red is overwritten by the next item's loads
  }
};

// ---------------------------------------------------------------------------
// Phase 2: MFMA tiles (larger experts), 256(n) x 128(m), one group per stage.
// Ring slot:  X [128 rows][128 B] @ SLOT_X   (row chunk c at c ^ (row & 7))
//             W [256 cols][64 B]  @ SLOT_W   (col chunk c at c ^ ((col >> 1) & 3))
// Scale chunk c (groups SC*c .. SC*c+3):  SB [256 cols][SC] u32;  SA [128 rows][SC] fp32
// ---------------------------------------------------------------------------
constexpr int MF_BN = TN_MFMA;  // 256 weight columns
constexpr int MF_BM = T_MAX;    // 128 activation rows
constexpr int P2_PER_STAGE = 4; // W 2, X 2 ring loads per wave

__device__ __forceinline__ void mf_issue_stage(const GemmArgs& p, uint8_t* slot, int e, int row0,
                                               int rows, int n0, int g) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int K = p.K, N = p.N;
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int j = wave * 2 + i;  // 16 columns x 64 B
    const int r = j * 16 + (lane >> 2);
    const int c = (lane & 3) ^ ((r >> 1) & 3);
    const int n = min(n0 + r, N - 1);
    dma16(p.B + ((size_t)e * N + n) * (size_t)(K >> 1) + (size_t)g * 64 + c * 16, slot + SLOT_W + j * 1024);
  }
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int j = wave * 2 + i;  // 8 rows x 128 B
    const int r = j * 8 + (lane >> 3);
    const int c = (lane & 7) ^ (r & 7);
    const size_t row = (size_t)row0 + min(r, rows - 1);
    dma16(p.A + row * (size_t)K + (size_t)g * 128 + c * 16, slot + SLOT_X + j * 1024);
  }
}

__device__ __forceinline__ void mf_issue_scales(const GemmArgs& p, uint8_t* lds, int e, int row0,
                                                int rows, int n0, int c, int R) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int K = p.K, N = p.N, G = K >> 7;
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int idx = (wave * 2 + i) * 64 + lane;  // [col][gg]
    const int col = idx >> 2, gg = idx & 3;
    const int n = min(n0 + col, N - 1);
    const int g = min(SC * c + gg, G - 1);
    dma4(p.SB + ((size_t)e * N + n) * (size_t)(K >> 5) + (size_t)g * 4,
         lds + LDS_SB + (c & 1) * SB_BYTES + (wave * 2 + i) * 256);
  }
  {
    const int idx = wave * 64 + lane;  // [row][gg]
    const int r = idx >> 2, gg = idx & 3;
    const size_t row = (size_t)row0 + min(r, rows - 1);
    const int g = min(SC * c + gg, G - 1);
    dma4(sa_ptr(p, row, g, G, R), lds + LDS_SA + (c & 1) * SA_BYTES + wave * 256);
  }
}

__device__ __forceinline__ void mfma_tile(const GemmArgs& p, uint8_t* lds, int e, int row0, int rows,
                                          int n0, int R) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int wn = wave & 3, wm = wave >> 2;  // 4 waves along n (64 each), 2 along m
  const int q = lane >> 4, r16 = lane & 15;
  const int G = p.K >> 7;
  // row blocks of this wave that hold real rows: wm, wm+2, wm+4, wm+6
  const int nmb = uniform(rows > wm * 16 ? min(4, (rows - wm * 16 + 31) / 32) : 0);

  v4f acc[4][4];
#pragma unroll
  for (int a = 0; a < 4; ++a)
#pragma unroll
    for (int b = 0; b < 4; ++b) acc[a][b] = v4f{0.f, 0.f, 0.f, 0.f};

  wait_vm<0>();
#pragma unroll
  for (int s = 0; s < NS - 1; ++s) {
    if (s < G) {
      if (s % SC == 0) mf_issue_scales(p, lds, e, row0, rows, n0, s / SC, R);
      mf_issue_stage(p, lds + s * SLOT_BYTES, e, row0, rows, n0, s);
    }
  }

  for (int g = 0; g < G; ++g) {
    stage_barrier<P2_PER_STAGE>(min(NS - 2, G - 1 - g));
    const int gn = g + NS - 1;
    if (gn < G) {
      if (gn % SC == 0) mf_issue_scales(p, lds, e, row0, rows, n0, gn / SC, R);
      mf_issue_stage(p, lds + (gn % NS) * SLOT_BYTES, e, row0, rows, n0, gn);
    }
    const uint8_t* slot = lds + (g % NS) * SLOT_BYTES;
    const uint8_t* sbb = lds + LDS_SB + ((g / SC) & 1) * SB_BYTES;
    const uint8_t* sab = lds + LDS_SA + ((g / SC) & 1) * SA_BYTES;
    const int gg = g % SC;
    v4i wf[4];
    int sbv[4];
#pragma unroll
    for (int nb = 0; nb < 4; ++nb) {
      const int n = wn * 64 + nb * 16 + r16;
      wf[nb] = lds128(slot + SLOT_W + n * 64 + ((q ^ ((n >> 1) & 3)) << 4));
      sbv[nb] = (int)((lds32(sbb + (n * SC + gg) * 4) >> (8 * q)) & 0xffu);
    }
    v4i x0[4], x1[4];
    float sa[4];
#pragma unroll
    for (int mi = 0; mi < 4; ++mi) {
      const int m = (wm + 2 * mi) * 16 + r16;
      const uint8_t* xb = slot + SLOT_X + m * 128;
      x0[mi] = lds128(xb + ((q ^ (m & 7)) << 4));
      x1[mi] = lds128(xb + (((q + 4) ^ (m & 7)) << 4));
      sa[mi] = ldsf(sab + (m * SC + gg) * 4);
    }
#pragma unroll
    for (int mi = 0; mi < 4; ++mi) {
      if (mi < nmb) {
        v4f pr[4];
#pragma unroll
        for (int nb = 0; nb < 4; ++nb) pr[nb] = mfma_group(wf[nb], x0[mi], x1[mi], sbv[nb]);
#pragma unroll
        for (int nb = 0; nb < 4; ++nb) promote(acc[mi][nb], sa[mi], pr[nb]);
      }
    }
  }
  __syncthreads();  // every wave is done with the ring before the next tile's loads

#pragma unroll
  for (int mi = 0; mi < 4; ++mi) {
    const int m = (wm + 2 * mi) * 16 + r16;
    if (m < rows) {
      uint16_t* crow = p.C + (size_t)(row0 + m) * p.N;
#pragma unroll
      for (int nb = 0; nb < 4; ++nb) {
        const int n = n0 + wn * 64 + nb * 16 + q * 4;
        if (n < p.N) store_bf16x4(crow + n, acc[mi][nb]);
      }
    }
  }
}

// ---------------------------------------------------------------------------
// The kernel: plan prologue, then both phases.
// ---------------------------------------------------------------------------
__global__ void __launch_bounds__(BLOCK, 1)
grouped_gemm_kernel(GemmArgs p) {
  __shared__ __attribute__((aligned(16))) uint8_t lds[LDS_BYTES];
  __shared__ int s_off[MAX_EXPERTS + 1];
  __shared__ int s_sbase[MAX_EXPERTS + 1];
  __shared__ int s_mbase[MAX_EXPERTS + 1];
  __shared__ int s_wave[WAVES];
  if (!plan_prologue(p.offsets, p.E, s_off, s_sbase, s_mbase, s_wave)) return;
  const int R = uniform(s_off[p.E]);

  // phase 1: streaming items, one workgroup each.  Items are 128 columns wide
  // when that still gives every workgroup three or more items, else 64.
  {
    const int tiles = uniform(s_sbase[p.E]);
    const long long items128 = (long long)tiles * ((p.N + 127) / 128);
    const bool wide = items128 >= 3LL * gridDim.x;
    const int width = wide ? StreamItem<2>::WIDTH : StreamItem<1>::WIDTH;
    const int nchunks = (p.N + width - 1) / width;
    const long long items = (long long)tiles * nchunks;
    for (long long it = blockIdx.x; it < items; it += gridDim.x) {
      const int mt = (int)(it / nchunks);
      const int n0 = (int)(it % nchunks) * width;
      const int e = uniform(expert_of_tile(s_sbase, p.E, mt));
      const int row0 = uniform(s_off[e]);
      const int rows = uniform(s_off[e + 1]) - row0;
      if (wide) StreamItem<2>::run(p, lds, e, row0, rows, n0, R);
      else StreamItem<1>::run(p, lds, e, row0, rows, n0, R);
    }
  }

  // phase 2: MFMA tiles, one workgroup each
  {
    const int nt_count = (p.N + MF_BN - 1) / MF_BN;
    const long long items = (long long)uniform(s_mbase[p.E]) * nt_count;
    for (long long it = blockIdx.x; it < items; it += gridDim.x) {
      const int mt = (int)(it / nt_count);
      const int n0 = (int)(it % nt_count) * MF_BN;
      const int e = uniform(expert_of_tile(s_mbase, p.E, mt));
      const int j = mt - uniform(s_mbase[e]);
      const int base = uniform(s_off[e]);
      const int rows_e = uniform(s_off[e + 1]) - base;
      const TileChoice tc = tile_rule(rows_e);
      const int row0 = base + j * tc.tile_m;
      const int rows = min(tc.tile_m, rows_e - j * tc.tile_m);
      mfma_tile(p, lds, e, row0, rows, n0, R);
    }
  }
}

hipError_t launch_grouped_gemm(const GemmArgs& args, int grid, hipStream_t stream) {
  hipLaunchKernelGGL(grouped_gemm_kernel, dim3(grid), dim3(BLOCK), 0, stream, args);
  return hipGetLastError();
}

hipError_t occupancy_blocks_per_cu(int* blocks) {
  return hipOccupancyMaxActiveBlocksPerMultiprocessor(blocks, grouped_gemm_kernel, BLOCK, 0);
}

}  // namespace w4a8
