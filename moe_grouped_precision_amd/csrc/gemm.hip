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
// tile plan of w4a8_device.h:
//   1. streaming items (experts with <= S_MAX rows), one workgroup per
//      (expert, 64..192 columns, width picked per launch): waves 0-3 take the
//      first half of the K groups and waves 4-7 the second half, two groups
//      per stage.  Weights stream from HBM straight into MFMA operand
//      registers (a per-wave ring two stages deep); the activation rows and
//      the scales are shared through LDS.  The halves are added in LDS
//      (always half 0 + half 1) before the bf16 store.
//   2. MFMA tiles (larger experts): 256(n) x 128(m) per workgroup, one K group
//      per stage through a 4-slot LDS ring (three stages in flight); each
//      wave owns 64(n) x 64(m).
// Shared operands reach LDS through direct global->LDS loads
// (global_load_lds_dwordx4 / _dword), which hold no registers while in
// flight: every wave issues the same number of loads per stage, waits for the
// stage it needs with an explicit vmcnt and meets the others at one barrier
// per stage.  The E8M0 and activation scales are loaded four groups at a time
// (four lanes read 16 contiguous bytes) into a double buffer, so they cost a
// small fraction of the memory requests of the weights.  The XOR swizzle that
// keeps fragment reads free of LDS bank conflicts is applied on the
// global-address side (a load lane always writes slot base + size * lane).
// All loads use clamped addresses (padding rows and columns re-read a real
// one and are never stored), so no load is conditional on data.
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
constexpr int LDS_P2_BYTES = LDS_SA + 2 * SA_BYTES;

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
// A workgroup item is (expert, 64*NBW columns).  Waves 0-3 take the first half
// of the K groups, waves 4-7 the second half; a stage is KG consecutive groups
// of each half; wave w owns NBW 16-column blocks.  Weights go straight from
// HBM into the MFMA operand registers through a per-wave ring of D stages (no
// LDS: no other wave needs them); the activation rows and both scale kinds
// are shared by the workgroup and come through LDS:
//   X ring   : D+1 slots x [KG][2 halves][64 rows][128 B] @ 0  (row chunk c at c ^ (row & 7))
//   SB chunk : 2 x [2 halves][64*NBW cols][SC] u32            @ P1_SB
//   SA chunk : 2 x [2 halves][64 rows][SC] fp32               @ P1_SA
// After the K loop the halves are added through LDS (always half 0 + half 1,
// whatever the item width or stage size), then rounded to bf16 and stored.
// ---------------------------------------------------------------------------
constexpr int P1_XGROUP = 16384;          // activation rows of one group, both halves
constexpr int P1_XRING = 6 * P1_XGROUP;   // (D+1)*KG groups, at most 96 KB
constexpr int P1_MAXNBW = 3;
// groups of K per streaming stage: two halve the per-stage barriers and LDS
// round trips against one, at the same bytes in flight (four, with a single
// stage in flight, measured slower)
constexpr int P1_KG = 2;
constexpr int P1_SB = P1_XRING;
constexpr int P1_SBBUF = 2 * 64 * P1_MAXNBW * SC * 4;      // 6 KB
constexpr int P1_SA = P1_SB + 2 * P1_SBBUF;
constexpr int P1_SABUF = 2 * 64 * SC * 4;                  // 2 KB
constexpr int P1_BYTES = P1_SA + 2 * P1_SABUF;
static_assert(P1_MAXNBW * 16384 <= P1_SB, "reduction scratch must fit below the scale chunks");

template <int NBW, int KG>
struct StreamItem {
  static constexpr int WIDTH = 64 * NBW;  // columns per item
  // stages in flight: KG*D groups of weights per wave
  static constexpr int D = KG == 2 ? 2 : (NBW <= 2 ? 4 : 3);
  static constexpr int NX = D + 1;        // activation ring slots
  static constexpr int XSLOT = KG * P1_XGROUP;
  static_assert(NX * XSLOT <= P1_XRING, "activation ring");
  // a scale chunk buffer is reloaded D stages before the first stage of the
  // chunk after next: every stage of the chunk before must be done by then
  static_assert(SC % KG == 0 && D * KG <= SC, "scale chunk reuse distance");

  // Activation rows of stage s: KG*8*mb loads of 4 rows x 128 B, KG*mb per wave.
  __device__ __forceinline__ static void issue_x(const GemmArgs& p, uint8_t* slot, int row0, int rows,
                                                 int mb, int s) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int K = p.K, G = K >> 7, Gh = (G + 1) / 2;
#pragma unroll
    for (int kg = 0; kg < KG; ++kg) {
      const int g0 = min(s * KG + kg, G - 1), g1 = min(Gh + s * KG + kg, G - 1);
      for (int i = 0; i < mb; ++i) {
        if (lane < 32) {
          const int jx = wave * mb + i;
          const int h = jx / (4 * mb), quad = jx - h * (4 * mb);
          const int r = quad * 4 + (lane >> 3);
          const int c = (lane & 7) ^ (r & 7);
          const size_t row = (size_t)row0 + min(r, rows - 1);
          dma16(p.A + row * (size_t)K + (size_t)(h ? g1 : g0) * 128 + c * 16,
                slot + kg * P1_XGROUP + h * 8192 + quad * 512);
        }
      }
    }
  }

  // Scale chunk c (groups SC*c .. SC*c+3 of each half): NBW SB + 1 SA loads per wave.
  __device__ __forceinline__ static void issue_scales(const GemmArgs& p, uint8_t* lds, int e,
                                                      int row0, int rows, int n0, int c, int R) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int K = p.K, N = p.N, G = K >> 7;
    const int gb1 = (G + 1) / 2;
#pragma unroll
    for (int i = 0; i < NBW; ++i) {
      const int idx = (wave * NBW + i) * 64 + lane;  // [h][col][gg]
      const int h = idx / (WIDTH * SC), rem = idx - h * (WIDTH * SC);
      const int col = rem >> 2, gg = rem & 3;
      const int n = min(n0 + col, N - 1);
      const int g = min((h ? gb1 : 0) + SC * c + gg, G - 1);
      dma4(p.SB + ((size_t)e * N + n) * (size_t)(K >> 5) + (size_t)g * 4,
           lds + P1_SB + (c & 1) * P1_SBBUF + (wave * NBW + i) * 256);
    }
    {
      const int idx = wave * 64 + lane;  // [h][row][gg]
      const int h = idx >> 8, r = (idx >> 2) & 63, gg = idx & 3;
      const size_t row = (size_t)row0 + min(r, rows - 1);
      const int g = min((h ? gb1 : 0) + SC * c + gg, G - 1);
      dma4(sa_ptr(p, row, g, G, R), lds + P1_SA + (c & 1) * P1_SABUF + wave * 256);
    }
  }

  // Weight fragments of this wave for stage s (16 B per lane per 16-column block and group).
  __device__ __forceinline__ static void load_w(v4i (&w)[KG][NBW], const uint8_t* const (&wp)[NBW],
                                                int gfirst, int G) {
#pragma unroll
    for (int kg = 0; kg < KG; ++kg)
#pragma unroll
      for (int j = 0; j < NBW; ++j)
        w[kg][j] = __builtin_nontemporal_load(
            reinterpret_cast<const v4i*>(wp[j] + (size_t)min(gfirst + kg, G - 1) * 64));
  }

  // Wait until the activation loads of the stage about to be used have landed
  // (at most `pending` later stages of KG*(mb + NBW) loads each in flight),
  // then meet the other waves.
  template <int PER>
  __device__ __forceinline__ static void stage_wait(int pending) {
    static_assert((D - 1) * PER < 64, "too many loads in flight");
    switch (pending) {
      case 0: wait_vm<0>(); break;
      case 1: wait_vm<PER>(); break;
      case 2: wait_vm<(D >= 3 ? 2 : 1) * PER>(); break;
      default: wait_vm<(D - 1) * PER>(); break;
    }
  }
  __device__ __forceinline__ static void x_barrier(int pending, int mb) {
    switch (mb) {
      case 1: stage_wait<KG * (NBW + 1)>(pending); break;
      case 2: stage_wait<KG * (NBW + 2)>(pending); break;
      case 3: stage_wait<KG * (NBW + 3)>(pending); break;
      default: stage_wait<KG * (NBW + 4)>(pending); break;
    }
    __builtin_amdgcn_s_barrier();
  }

  __device__ __forceinline__ static void run(const GemmArgs& p, uint8_t* lds, int e, int row0,
                                             int rows, int n0, int R) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int kh = wave >> 2, wn = wave & 3;
    const int q = lane >> 4, r16 = lane & 15;
    const int K = p.K, N = p.N, G = K >> 7;
    const int Gh = (G + 1) / 2;
    const int gbase = kh ? Gh : 0;
    const int gcount = kh == 0 ? Gh : G - Gh;  // groups of this wave's half
    const int S = (Gh + KG - 1) / KG;
    const int mb = (rows + 15) >> 4;             // 1..4 row blocks

    const uint8_t* wp[NBW];
#pragma unroll
    for (int j = 0; j < NBW; ++j) {
      const int n = min(n0 + (wn * NBW + j) * 16 + r16, N - 1);
      wp[j] = p.B + ((size_t)e * N + n) * (size_t)(K >> 1) + q * 16;
    }

    v4f acc[NBW][4];
#pragma unroll
    for (int j = 0; j < NBW; ++j)
#pragma unroll
      for (int i = 0; i < 4; ++i) acc[j][i] = v4f{0.f, 0.f, 0.f, 0.f};
    v4i wr[D][KG][NBW];

    wait_vm<0>();  // earlier stores must not be counted against this item's loads
#pragma unroll
    for (int s = 0; s < D; ++s) {
      if (s < S) {
        if ((s * KG) % SC == 0) issue_scales(p, lds, e, row0, rows, n0, s * KG / SC, R);
        issue_x(p, lds + (s % NX) * XSLOT, row0, rows, mb, s);
        load_w(wr[s], wp, gbase + s * KG, G);
      }
    }

    for (int s0 = 0; s0 < S; s0 += D) {
#pragma unroll
      for (int u = 0; u < D; ++u) {
        const int s = s0 + u;
        if (s < S) {
          x_barrier(min(D - 1, S - 1 - s), mb);
          const int sn = s + D;
          if (sn < S) {
            if ((sn * KG) % SC == 0) issue_scales(p, lds, e, row0, rows, n0, sn * KG / SC, R);
            issue_x(p, lds + (sn % NX) * XSLOT, row0, rows, mb, sn);
          }
          const uint8_t* slot = lds + (s % NX) * XSLOT;
#pragma unroll
          for (int kg = 0; kg < KG; ++kg) {
            const int gl = s * KG + kg;  // group index within this wave's half
            if (gl < gcount) {
              const uint8_t* sbb = lds + P1_SB + ((gl / SC) & 1) * P1_SBBUF;
              const uint8_t* sab = lds + P1_SA + ((gl / SC) & 1) * P1_SABUF;
              const int gg = gl % SC;
              int sbv[NBW];
#pragma unroll
              for (int j = 0; j < NBW; ++j) {
                const int col = (wn * NBW + j) * 16 + r16;
                sbv[j] = (int)((lds32(sbb + ((kh * WIDTH + col) * SC + gg) * 4) >> (8 * q)) & 0xffu);
              }
#pragma unroll
              for (int i = 0; i < 4; ++i) {
                if (i < mb) {
                  const int m = i * 16 + r16;
                  const uint8_t* xb = slot + kg * P1_XGROUP + kh * 8192 + m * 128;
                  const v4i x0 = lds128(xb + ((q ^ (m & 7)) << 4));
                  const v4i x1 = lds128(xb + (((q + 4) ^ (m & 7)) << 4));
                  const float sa = ldsf(sab + ((kh * 64 + m) * SC + gg) * 4);
#pragma unroll
                  for (int j = 0; j < NBW; ++j)
                    promote(acc[j][i], sa, mfma_group(wr[u][kg][j], x0, x1, sbv[j]));
                }
              }
            }
          }
          if (sn < S) load_w(wr[u], wp, gbase + sn * KG, G);
        }
      }
    }

    // add the two K halves in LDS (nothing is in flight and every wave is past
    // its last LDS read after this barrier) and store
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
          uint16_t* crow = p.C + (size_t)(row0 + m) * N;
#pragma unroll
          for (int j = 0; j < NBW; ++j) {
            const int n = n0 + (wn * NBW + j) * 16 + q * 4;
            const v4f o = red[((wn * NBW + j) * 4 + i) * 64 + lane];
            if (n < N) store_bf16x4(crow + n, acc[j][i] + o);
          }
        }
      }
    }
    __syncthreads();  // red is overwritten by the next item's loads
  }
};

// Item width for the streaming phase: the width (64*NBW columns) that
// minimises rounds x per-item bytes, per-item bytes ~ weights (32*NBW per K)
// plus activation rows (about 32 per K).  Wider items re-read the activation
// rows less often; narrower items spread few experts over more workgroups.
__device__ __forceinline__ int stream_width_blocks(int tiles, int N, int grid) {
  int best = 1;
  long long best_cost = -1;
  for (int nbw = 1; nbw <= P1_MAXNBW; ++nbw) {
    const long long items = (long long)tiles * ((N + 64 * nbw - 1) / (64 * nbw));
    const long long rounds = (items + grid - 1) / grid;
    const long long cost = rounds * (32LL * nbw + 32);
    if (best_cost < 0 || cost <= best_cost) {
      best_cost = cost;
      best = nbw;
    }
  }
  return best;
}

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
  __shared__ __attribute__((aligned(16))) uint8_t lds[LDS_P2_BYTES > P1_BYTES ? LDS_P2_BYTES : P1_BYTES];
  __shared__ int s_off[MAX_EXPERTS + 1];
  __shared__ int s_sbase[MAX_EXPERTS + 1];
  __shared__ int s_mbase[MAX_EXPERTS + 1];
  __shared__ int s_wave[WAVES];
  if (!plan_prologue(p.offsets, p.E, s_off, s_sbase, s_mbase, s_wave)) return;
  const int R = uniform(s_off[p.E]);

  // phase 1: streaming items, one workgroup each
  {
    const int tiles = uniform(s_sbase[p.E]);
    const int nbw = stream_width_blocks(tiles, p.N, gridDim.x);
    const int width = 64 * nbw;
    const int nchunks = (p.N + width - 1) / width;
    const long long items = (long long)tiles * nchunks;
    for (long long it = blockIdx.x; it < items; it += gridDim.x) {
      const int mt = (int)(it / nchunks);
      const int n0 = (int)(it % nchunks) * width;
      const int e = uniform(expert_of_tile(s_sbase, p.E, mt));
      const int row0 = uniform(s_off[e]);
      const int rows = uniform(s_off[e + 1]) - row0;
      switch (nbw) {
        case 1: StreamItem<1, P1_KG>::run(p, lds, e, row0, rows, n0, R); break;
        case 2: StreamItem<2, P1_KG>::run(p, lds, e, row0, rows, n0, R); break;
        default: StreamItem<3, P1_KG>::run(p, lds, e, row0, rows, n0, R); break;
      }
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
