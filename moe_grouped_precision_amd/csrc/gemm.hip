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
//   2. MFMA tiles (larger experts): 512(n) x 128(m) per workgroup, one K group
//      per stage; each wave owns 64 columns x all 128 rows, its weights in a
//      register ring, the activation rows in an LDS ring; tiles are dealt so
//      that each XCD works on a compact block.
// Shared operands reach LDS through direct global->LDS loads
// (global_load_lds_dwordx4 / _dword), which hold no registers while in
// flight: every wave issues the same number of loads per stage, waits for the
// stage it needs with one explicit vmcnt and meets the others at one barrier
// per stage.  All vector-memory ops of the K loops are inline asm (see the
// helpers below for why).  The E8M0 and activation scales are loaded four groups at a time
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
constexpr int SC = 4;                  // groups per scale chunk

// ---------------------------------------------------------------------------
// Vector-memory operations of the K loops are written as inline asm, and every
// wait for them is explicit.  The compiler cannot tell one LDS ring slot from
// another, so for a direct-to-LDS load it knows about it would wait for the
// load to land before any later LDS read, i.e. drain the pipeline every stage;
// and a mix of loads it sees and loads it does not would make its own register
// waits force the unseen ones too.  Hence: no compiler-visible vector-memory
// op inside a K loop, one explicit vmcnt wait per stage (counted from the
// issue order, which is the completion order of loads), and register loads
// tied to that wait so that no instruction reads them earlier.
// ---------------------------------------------------------------------------
// LDS byte address of a pointer into the kernel's shared array: the low 32
// bits of its flat address (the shared aperture is 4 GB aligned).  Taking
// them directly avoids the null test of a generic-to-local address cast.
__device__ __forceinline__ uint32_t lds_u32(const uint8_t* p) { return (uint32_t)(uintptr_t)p; }

// Scalar operands of the asm below must be wave-uniform values the compiler
// keeps in SGPRs; readfirstlane makes that explicit (and is free when the
// value already is scalar).  A vector-memory instruction that reads an SGPR
// written by a VALU instruction (readfirstlane is one) needs 5 wait states in
// between, and M0 written by SALU needs 1 before a direct-to-LDS load; the
// compiler inserts such waits for instructions it sees, not inside asm, so
// each asm below carries its own.
__device__ __forceinline__ const void* sgpr_ptr(const void* p) {
  const uint64_t v = (uint64_t)p;
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)v);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(v >> 32));
  return (const void*)(((uint64_t)hi << 32) | lo);
}

// Loads that a stage issues past the end of the K loop run with exec = 0: the
// instruction still issues and counts toward vmcnt (so every wait stays one
// constant) but reads no memory and writes no register.  `mask` is the exec
// mask to load with: live_mask(true) = the current exec, live_mask(false) = 0.
__device__ __forceinline__ uint64_t live_mask(bool live) {
  return live ? __builtin_amdgcn_read_exec() : 0ull;
}

// 16 bytes per lane from sbase + voff (sbase wave-uniform) to LDS at
// lds + 16 * lane (lds wave-uniform; lanes outside mask write nothing).
__device__ __forceinline__ void vm_dma16(const void* sbase, uint32_t voff, uint32_t lds, uint64_t mask) {
  uint64_t saved;
  asm volatile("s_mov_b64 %0, exec\n\ts_mov_b64 exec, %4\n\ts_mov_b32 m0, %3\n\ts_nop 3\n\t"
               "global_load_lds_dwordx4 %1, %2\n\ts_mov_b64 exec, %0"
               : "=&s"(saved)
               : "v"(voff), "s"(sgpr_ptr(sbase)), "s"(__builtin_amdgcn_readfirstlane(lds)), "s"(mask)
               : "memory", "m0", "exec");
}
// 4 bytes per lane from a per-lane address to LDS at lds + 4 * lane.
__device__ __forceinline__ void vm_dma4(const void* addr, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dword %0, off"
               :: "v"(addr), "s"(__builtin_amdgcn_readfirstlane(lds)) : "memory", "m0");
}
// 16 bytes per lane into r (lanes outside mask load nothing); r may be read
// only after a wait that covers this load, followed by tie() on it.  _nt
// marks the data nontemporal (streamed once).  r is an input as well as the
// output, so a ring slot reloaded in a loop is one live range in one
// register: the compiler never moves a slot between registers (a copy of a
// register whose load is still in flight would copy stale data).
__device__ __forceinline__ void vm_load16(v4i& r, const void* sbase, uint32_t voff, uint64_t mask) {
  uint64_t saved;
  asm volatile("s_mov_b64 %1, exec\n\ts_mov_b64 exec, %4\n\ts_nop 4\n\t"
               "global_load_dwordx4 %0, %2, %3\n\ts_mov_b64 exec, %1"
               : "+v"(r), "=&s"(saved)
               : "v"(voff), "s"(sgpr_ptr(sbase)), "s"(mask)
               : "exec");
}
__device__ __forceinline__ void vm_load16_nt(v4i& r, const void* sbase, uint32_t voff, uint64_t mask) {
  uint64_t saved;
  asm volatile("s_mov_b64 %1, exec\n\ts_mov_b64 exec, %4\n\ts_nop 4\n\t"
               "global_load_dwordx4 %0, %2, %3 nt\n\ts_mov_b64 exec, %1"
               : "+v"(r), "=&s"(saved)
               : "v"(voff), "s"(sgpr_ptr(sbase)), "s"(mask)
               : "exec");
}
__device__ __forceinline__ void tie(v4i& r) { asm volatile("" : "+v"(r)); }


// s_waitcnt vmcnt(N): at most N of this wave's vector-memory ops in flight.
// Also a compiler barrier, so no LDS read moves above it.
template <int N>
__device__ __forceinline__ void wait_vm() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  asm volatile("s_waitcnt vmcnt(%0)" :: "n"(N) : "memory");
}

// Workgroup barrier that is also a compiler barrier for memory operations
// (no fence: the explicit waits decide what has landed).
__device__ __forceinline__ void wg_barrier() { asm volatile("s_barrier" ::: "memory"); }

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

// Activation rows are stored 128 B per row in LDS with 16-byte chunk c of
// row r at position c ^ xkey(r).  A 16-byte read serves 16 lanes per pass
// over 64 four-byte banks, i.e. two rows' worth of banks: the 16 lanes of a
// fragment read (rows 16j .. 16j+15, one chunk index) then hit 16 distinct
// 4-bank groups -- rows of one parity share a bank half and differ in r >> 1.
__device__ __forceinline__ int xkey(int r) { return (r >> 1) & 7; }

// Scale words are stored in rows of SCW 4-byte words (one row per weight column
// or activation row), word gg of row r at position gg ^ skey<SCW>(r).  A 4-byte
// read of 16 consecutive rows is served by 32 banks: without the key, rows r
// and r + 32/SCW would share a bank; with it they differ in position.
template <int SCW>
__device__ __forceinline__ int skey(int r) { return (r / (32 / SCW)) & (SCW - 1); }

// A lane index the compiler cannot see through, so that address arithmetic
// done once per scale chunk is not hoisted out of the K loop (where its
// registers would compete with the accumulators).
__device__ __forceinline__ int opaque_lane() {
  int lane = threadIdx.x & 63;
  asm volatile("" : "+v"(lane));
  return lane;
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
// Stage s: wait (the weights of stage s and, older, its activation rows have
// landed), barrier, issue the activation rows of stage s + D, MFMAs, then the
// weights of stage s + D into the register slot just used.  After the K loop
// the halves are added through LDS (always half 0 + half 1, whatever the item
// width or stage size), then rounded to bf16 and stored.
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

template <int NBW, int KG, int MB>
struct StreamItem {
  static constexpr int WIDTH = 64 * NBW;  // columns per item
  // stages in flight: KG*D groups of weights per wave
  static constexpr int D = KG == 2 ? 2 : (NBW <= 2 ? 4 : 3);
  static constexpr int NX = D + 1;        // activation ring slots
  static constexpr int XSLOT = KG * P1_XGROUP;
  static constexpr int PER = KG * (NBW + MB);  // ring loads per wave per stage
  static_assert(NX * XSLOT <= P1_XRING, "activation ring");
  static_assert((D - 1) * PER < 64, "vmcnt range");
  // a scale chunk buffer is reloaded D stages before the first stage of the
  // chunk after next: every stage of the chunk before must be done by then
  static_assert(SC % KG == 0 && D * KG <= SC, "scale chunk reuse distance");
  static_assert(KG == 2, "a stage's weight loads cover one 128-byte line (two groups) per column");

  // Activation rows of stage s: 8*MB loads of 4 rows x 128 B per group, MB per
  // wave (half a wave each).  xt = the item's first row.
  __device__ __forceinline__ static void issue_x(const uint8_t* xt, const uint32_t (&xo)[MB], uint8_t* slot,
                                                 int G, int s, bool live) {
    const int wave = uniform(threadIdx.x >> 6);
    const int Gh = (G + 1) / 2;
    const uint64_t mask = live_mask(live) & 0xffffffffull;  // lanes 0-31 load
#pragma unroll
    for (int kg = 0; kg < KG; ++kg) {
      const int g0 = min(s * KG + kg, G - 1), g1 = min(Gh + s * KG + kg, G - 1);
#pragma unroll
      for (int i = 0; i < MB; ++i) {
        const int jx = wave * MB + i;
        const int h = jx / (4 * MB), quad = jx - h * (4 * MB);
        vm_dma16(xt + (size_t)(h ? g1 : g0) * 128, xo[i],
                 lds_u32(slot + kg * P1_XGROUP + h * 8192 + quad * 512), mask);
      }
    }
  }

  // Scale chunk c (groups SC*c .. SC*c+3 of each half): NBW SB + 1 SA loads per wave.
  __device__ __forceinline__ static void issue_scales(const GemmArgs& p, uint8_t* lds, int e,
                                                      int row0, int rows, int n0, int c, int R) {
    const int lane = opaque_lane(), wave = uniform(threadIdx.x >> 6);
    const int K = p.K, N = p.N, G = K >> 7;
    const int gb1 = (G + 1) / 2;
#pragma unroll
    for (int i = 0; i < NBW; ++i) {
      const int idx = (wave * NBW + i) * 64 + lane;  // [h][col][gg]
      const int h = idx / (WIDTH * SC), rem = idx - h * (WIDTH * SC);
      const int col = rem >> 2, gg = rem & 3;
      const int n = min(n0 + col, N - 1);
      const int g = min((h ? gb1 : 0) + SC * c + gg, G - 1);
      vm_dma4(p.SB + ((size_t)e * N + n) * (size_t)(K >> 5) + (size_t)g * 4,
              lds_u32(lds + P1_SB + (c & 1) * P1_SBBUF + (wave * NBW + i) * 256));
    }
    {
      const int idx = wave * 64 + lane;  // [h][row][gg]
      const int h = idx >> 8, r = (idx >> 2) & 63, gg = idx & 3;
      const size_t row = (size_t)row0 + min(r, rows - 1);
      const int g = min((h ? gb1 : 0) + SC * c + gg, G - 1);
      vm_dma4(sa_ptr(p, row, g, G, R), lds_u32(lds + P1_SA + (c & 1) * P1_SABUF + wave * 256));
    }
  }

  // Weights of this wave for the stage whose groups are gfirst, gfirst + 1:
  // per 16-column block j, load w[h][j] covers columns 8h .. 8h+7 of the block
  // with one full 128-byte line (both groups) per column, lane 16q + i reading
  // column 8h + (i & 7), group gfirst + (i >> 3), bytes 16q .. 16q+15.  Whole
  // lines per request stream from HBM at the rate of contiguous reads; two
  // 64-byte requests per line (one per group) do not.  pair_operands() turns
  // the two loads into the MFMA operands of the two groups.  wt = the item's
  // first column; wo = this lane's column offsets; goff = its group offset
  // (the second group is clamped to the last one when G is odd).
  __device__ __forceinline__ static void load_w(v4i (&w)[KG][NBW], const uint8_t* wt,
                                                const uint32_t (&wo)[2][NBW], int gfirst, int G, bool live) {
    const uint64_t mask = live_mask(live);
    const uint32_t goff = (uint32_t)min(gfirst + ((threadIdx.x & 15) >> 3), G - 1) * 64u;
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
      for (int j = 0; j < NBW; ++j) vm_load16_nt(w[h][j], wt, wo[h][j] + goff, mask);
  }

  // MFMA operand of group gfirst + g of block j: lane 16q + i needs column i,
  // bytes 16q.. of that group.  Load h holds it in lane 16q + (i & 7) + 8g
  // when i >> 3 == h, so the operand is load g's own lanes in one half of each
  // 16-lane row and the other load's lanes rotated by 8 in the other half.
  __device__ __forceinline__ static void pair_operands(const v4i& a, const v4i& b, v4i& g0, v4i& g1) {
#pragma unroll
    for (int d = 0; d < 4; ++d) {
      // row_ror:8 (dpp_ctrl 0x128); bank_mask picks the 4-lane banks written
      g0[d] = __builtin_amdgcn_update_dpp(a[d], b[d], 0x128, 0xf, 0xc, false);
      g1[d] = __builtin_amdgcn_update_dpp(b[d], a[d], 0x128, 0xf, 0x3, false);
    }
  }

  // Wait until the weights of the stage about to be used have landed: every
  // stage issues its loads (those past the end with exec = 0), so
  // exactly D-1 later stages of PER loads each may still be in flight; the
  // stage's activation rows were issued before its weights.  Then make the
  // weights readable and meet the other waves.
  __device__ __forceinline__ static void stage_wait(v4i (&w)[KG][NBW]) {
    wait_vm<(D - 1) * PER>();
#pragma unroll
    for (int kg = 0; kg < KG; ++kg)
#pragma unroll
      for (int j = 0; j < NBW; ++j) tie(w[kg][j]);
    wg_barrier();
  }

  __device__ __forceinline__ static void run(const GemmArgs& p, uint8_t* lds, int e, int row0,
                                             int rows, int n0, int R) {
    const int lane = opaque_lane(), wave = threadIdx.x >> 6;
    const int kh = wave >> 2, wn = wave & 3;
    const int q = lane >> 4, r16 = lane & 15;
    const int K = p.K, N = p.N, G = K >> 7;
    const int Gh = (G + 1) / 2;
    const int gbase = kh ? Gh : 0;
    const int gcount = kh == 0 ? Gh : G - Gh;  // groups of this wave's half
    const int S = (Gh + KG - 1) / KG;

    const uint8_t* xt = p.A + (size_t)row0 * K;
    uint32_t xo[MB];
#pragma unroll
    for (int i = 0; i < MB; ++i) {
      const int jx = uniform(wave) * MB + i;
      const int quad = jx % (4 * MB);
      const int r = quad * 4 + (lane >> 3);
      const int c = (lane & 7) ^ (r & 7);
      xo[i] = (uint32_t)min(r, rows - 1) * (uint32_t)K + c * 16;
    }
    const uint8_t* wt = p.B + ((size_t)e * N + n0) * (size_t)(K >> 1);
    uint32_t wo[2][NBW];
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
      for (int j = 0; j < NBW; ++j) {
        const int n = min(n0 + (wn * NBW + j) * 16 + 8 * h + (r16 & 7), N - 1);
        wo[h][j] = (uint32_t)(n - n0) * (uint32_t)(K >> 1) + q * 16;
      }

    v4f acc[NBW][MB];
#pragma unroll
    for (int j = 0; j < NBW; ++j)
#pragma unroll
      for (int i = 0; i < MB; ++i) acc[j][i] = v4f{0.f, 0.f, 0.f, 0.f};
    v4i wr[D][KG][NBW];
#pragma unroll
    for (int u = 0; u < D; ++u)
#pragma unroll
      for (int kg = 0; kg < KG; ++kg)
#pragma unroll
        for (int j = 0; j < NBW; ++j) wr[u][kg][j] = v4i{0, 0, 0, 0};

    // Every stage issues its loads (past the last stage with exec = 0 and
    // addresses clamped in range), so each wait is the same constant; the loop
    // body is D whole stages and the last S % D stages follow it, so no
    // control-flow path skips a stage and then runs a later one.
#pragma unroll
    for (int s = 0; s < D; ++s) {
      if (s < S && (s * KG) % SC == 0) issue_scales(p, lds, e, row0, rows, n0, s * KG / SC, R);
      issue_x(xt, xo, lds + (s % NX) * XSLOT, G, min(s, S - 1), s < S);
      load_w(wr[s], wt, wo, gbase + min(s, S - 1) * KG, G, s < S);
    }

    auto stage = [&](int s, int u) __attribute__((always_inline)) {
      stage_wait(wr[u]);
      const int sn = s + D;
      if (sn < S && (sn * KG) % SC == 0) issue_scales(p, lds, e, row0, rows, n0, sn * KG / SC, R);
      issue_x(xt, xo, lds + (sn % NX) * XSLOT, G, min(sn, S - 1), sn < S);
      const uint8_t* slot = lds + (s % NX) * XSLOT;
      v4i wop[KG][NBW];
#pragma unroll
      for (int j = 0; j < NBW; ++j) pair_operands(wr[u][0][j], wr[u][1][j], wop[0][j], wop[1][j]);
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
          for (int i = 0; i < MB; ++i) {
            const int m = i * 16 + r16;
            const uint8_t* xb = slot + kg * P1_XGROUP + kh * 8192 + m * 128;
            const v4i x0 = lds128(xb + ((q ^ (m & 7)) << 4));
            const v4i x1 = lds128(xb + (((q + 4) ^ (m & 7)) << 4));
            const float sa = ldsf(sab + ((kh * 64 + m) * SC + gg) * 4);
#pragma unroll
            for (int j = 0; j < NBW; ++j)
              promote(acc[j][i], sa, mfma_group(wop[kg][j], x0, x1, sbv[j]));
          }
        }
      }
      load_w(wr[u], wt, wo, gbase + min(sn, S - 1) * KG, G, sn < S);
    };

    static_assert(D == 2, "the stage loop below is written for two stages in flight");
    int s0 = 0;
    for (; s0 + 2 <= S; s0 += 2) {
      stage(s0, 0);
      stage(s0 + 1, 1);
    }
    if (s0 < S) stage(s0, 0);
    // every load has retired; the ties keep the ring registers reserved until
    // here (a value never read would otherwise be reused while its load is
    // still in flight)
    wait_vm<0>();
#pragma unroll
    for (int u = 0; u < D; ++u)
#pragma unroll
      for (int kg = 0; kg < KG; ++kg)
#pragma unroll
        for (int j = 0; j < NBW; ++j) tie(wr[u][kg][j]);

    // add the two K halves in LDS (nothing is in flight -- the last wait was
    // for zero -- and every wave is past its last LDS read after this barrier)
    __syncthreads();
    v4f* red = reinterpret_cast<v4f*>(lds);
    if (kh == 1) {
#pragma unroll
      for (int j = 0; j < NBW; ++j)
#pragma unroll
        for (int i = 0; i < MB; ++i) red[((wn * NBW + j) * 4 + i) * 64 + lane] = acc[j][i];
    }
    __syncthreads();
    if (kh == 0) {
#pragma unroll
      for (int i = 0; i < MB; ++i) {
        const int m = i * 16 + r16;
        if (m < rows) {
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

template <int NBW>
__device__ __forceinline__ void stream_item(const GemmArgs& p, uint8_t* lds, int e, int row0, int rows,
                                            int n0, int R) {
  switch ((rows + 15) >> 4) {
    case 1: StreamItem<NBW, P1_KG, 1>::run(p, lds, e, row0, rows, n0, R); break;
    case 2: StreamItem<NBW, P1_KG, 2>::run(p, lds, e, row0, rows, n0, R); break;
    case 3: StreamItem<NBW, P1_KG, 3>::run(p, lds, e, row0, rows, n0, R); break;
    default: StreamItem<NBW, P1_KG, 4>::run(p, lds, e, row0, rows, n0, R); break;
  }
}

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
// Phase 2: MFMA tiles (larger experts), 512(n) x 128(m) per workgroup.
//
// Wave w owns columns 64w .. 64w+63 of the tile and all of its rows (4 x 8
// MFMA blocks, 128 fp32 accumulators per lane).  Every weight byte of the
// tile is needed by exactly one wave, so weights go from global memory
// straight into that wave's MFMA operand registers (the next group's weights
// load while the current group's are in use); only the activation rows and
// the scales, which every wave needs, are staged in LDS:
//   X ring   : P2_NX slots x [128 rows][128 B]  (row chunk c at c ^ key(row))
//   SB chunk : 2 x [512 cols][SC] u32  (E8M0 codes of groups SC*c .. SC*c+3)
//   SA chunk : 2 x [128 rows][SC] fp32
// Stage s (one K group): wait (weights of group s and, older, its activation
// rows have landed), barrier, issue the weights of group s + 1 and then the
// activation rows of group s + 2 (with their scale chunk), then 32 MFMAs per
// wave.  One in-order counter per wave is what sets the depths: waiting for
// the weights of group s also waits for everything issued before them, so
// activation rows are issued right after a weight load and run one stage
// further ahead than the weights.
// Per 128-K group a workgroup reads 32 KB of weights and 16 KB of activations
// for 256 MFMAs, the fewest bytes per MFMA of the tile shapes whose
// accumulators fit two waves per SIMD.
// ---------------------------------------------------------------------------
constexpr int MF_BN = TN_MFMA;          // 512 weight columns
constexpr int MF_BM = T_MAX;            // 128 activation rows
constexpr int P2_DW = 1;                // weight groups ahead (register slots: P2_DW + 1)
constexpr int P2_DX = P2_DW + 1;        // activation groups ahead
constexpr int P2_NX = P2_DX + 1;        // activation ring slots
constexpr int P2_XSLOT = MF_BM * 128;   // 16 KB
constexpr int P2_SB = P2_NX * P2_XSLOT;
constexpr int P2_SBBUF = MF_BN * SC * 4;  // 8 KB
constexpr int P2_SA = P2_SB + 2 * P2_SBBUF;
constexpr int P2_SABUF = MF_BM * SC * 4;  // 2 KB
constexpr int P2_BYTES = P2_SA + 2 * P2_SABUF;
constexpr int P2_X_OPS = 2;             // activation loads per wave per stage
constexpr int P2_W_OPS = 4;             // weight loads per wave per stage
// a scale buffer is refilled P2_DX stages ahead, after every stage of the
// chunk two back has passed the barrier of the stage that refills it
static_assert(P2_DX <= SC, "scale chunk reuse distance");
static_assert(P2_DW == 1, "the stage loop is unrolled for two weight slots");

// Activation rows of group g: 128 rows x 128 B, two 8-row loads per wave
// (xt = the tile's first row, xo = this lane's byte offsets from it).
__device__ __forceinline__ void p2_issue_x(const uint8_t* xt, const uint32_t (&xo)[P2_X_OPS],
                                           uint8_t* slot, int g, bool live) {
  const int wave = uniform(threadIdx.x >> 6);
  const uint8_t* xg = xt + (size_t)g * 128;
  const uint64_t mask = live_mask(live);
#pragma unroll
  for (int i = 0; i < P2_X_OPS; ++i)
    vm_dma16(xg, xo[i], lds_u32(slot + (wave * P2_X_OPS + i) * 1024), mask);
}

// Scale chunk c: 512 columns x SC groups of E8M0 words (four loads per wave)
// and 128 rows x SC groups of activation scales (one load per wave).
__device__ __forceinline__ void p2_issue_scales(const GemmArgs& p, uint8_t* lds, int e, int row0,
                                                int rows, int n0, int c, int R) {
  const int lane = opaque_lane(), wave = uniform(threadIdx.x >> 6);
  const int K = p.K, N = p.N, G = K >> 7;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int col = ((wave * 4 + i) * 64 + lane) >> 2;  // rows [col] of SC words
    const int g = min(SC * c + ((lane & 3) ^ skey<SC>(col)), G - 1);
    const int n = min(n0 + col, N - 1);
    vm_dma4(p.SB + ((size_t)e * N + n) * (size_t)(K >> 5) + (size_t)g * 4,
            lds_u32(lds + P2_SB + (c & 1) * P2_SBBUF + (wave * 4 + i) * 256));
  }
  const int r = (wave * 64 + lane) >> 2;  // rows [row] of SC words
  const int g = min(SC * c + ((lane & 3) ^ skey<SC>(r)), G - 1);
  const size_t row = (size_t)row0 + min(r, rows - 1);
  vm_dma4(sa_ptr(p, row, g, G, R), lds_u32(lds + P2_SA + (c & 1) * P2_SABUF + wave * 256));
}

// Weights of group g for this wave's four 16-column blocks (wt = the tile's
// first column, wo = this lane's byte offsets from it).
__device__ __forceinline__ void p2_load_w(v4i (&w)[4], const uint8_t* wt, const uint32_t (&wo)[4], int g,
                                          bool live) {
  const uint8_t* wg = wt + (size_t)g * 64;
  const uint64_t mask = live_mask(live);
#pragma unroll
  for (int nb = 0; nb < 4; ++nb) vm_load16(w[nb], wg, wo[nb], mask);
}

// LDS addresses of this lane's fragments in a stage slot / scale buffer: row
// block mi adds the immediate mi * 2048 (X) or mi * 256 (SA).  Row m = 16 mi
// + i has activation key xkey(m) = xkey(i) for every mi, and scale key
// skey<SC>(m) = ((2 mi) & 3) ^ (i >> 3): one scale address for even mi, one
// for odd.
struct P2Lds {
  const uint8_t* x0;   // chunk q of row i
  const uint8_t* x1;   // chunk q + 4 of row i
  const uint8_t* sa0;  // scale (row i, group gg), even mi
  const uint8_t* sa1;  // odd mi
};

__device__ __forceinline__ void p2_read_x(const P2Lds& a, int mi, v4i& x0, v4i& x1, float& sa) {
  x0 = lds128(a.x0 + mi * 2048);
  x1 = lds128(a.x1 + mi * 2048);
  sa = ldsf(((mi & 1) ? a.sa1 : a.sa0) + mi * 16 * SC * 4);
}

// One K group for NMB row blocks.  Step mi issues the LDS reads of block
// mi+1, the four MFMAs of block mi and the promotion of the previous step's
// partials (carried across stages in prev/sprev, so the first step of a stage
// has arithmetic to do while its reads are in flight); the scheduling fences
// keep each step's work together.
template <int NMB>
__device__ __forceinline__ void p2_group(v4f (&acc)[8][4], v4f (&prev)[4], float& sprev, const v4i (&w)[4],
                                         const P2Lds& a, const int (&sbv)[4]) {
  v4i xa0, xa1;
  float saa;
  p2_read_x(a, 0, xa0, xa1, saa);
#pragma unroll
  for (int mi = 0; mi < NMB; ++mi) {
    v4i xb0 = xa0, xb1 = xa1;
    float sab_n = saa;
    if (mi + 1 < NMB) p2_read_x(a, mi + 1, xb0, xb1, sab_n);
    // the previous step's block: the last block of the previous group when mi == 0
    const int pm = mi == 0 ? NMB - 1 : mi - 1;
    v4f pn[4];
#pragma unroll
    for (int nb = 0; nb < 4; ++nb) pn[nb] = mfma_group(w[nb], xa0, xa1, sbv[nb]);
#pragma unroll
    for (int nb = 0; nb < 4; ++nb) promote(acc[pm][nb], sprev, prev[nb]);
#pragma unroll
    for (int nb = 0; nb < 4; ++nb) prev[nb] = pn[nb];
    sprev = saa;
    xa0 = xb0;
    xa1 = xb1;
    saa = sab_n;
    // step order: the next block's LDS reads, then each MFMA followed by four
    // of the promotions, which run while the matrix core works
    if (mi + 1 < NMB) __builtin_amdgcn_sched_group_barrier(0x100, 3, 0);
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x002, 4, 0);
    }
    __builtin_amdgcn_sched_barrier(0);
  }
}

template <int NMB>
struct MfmaTile {
  const GemmArgs& p;
  uint8_t* lds;
  int e, row0, rows, n0, R, G, wn, q, r16, xl0, xl1;
  bool wvalid;
  const uint8_t* xt;
  const uint8_t* wt;
  uint32_t xo[P2_X_OPS];
  uint32_t wo[4];

  __device__ __forceinline__ MfmaTile(const GemmArgs& p_, uint8_t* lds_, int e_, int row0_, int rows_,
                                      int n0_, int R_)
      : p(p_), lds(lds_), e(e_), row0(row0_), rows(rows_), n0(n0_), R(R_) {
    // opaque lane: the per-lane constants below are computed per tile, not
    // hoisted out of the tile loop where they would be live across it
    const int lane = opaque_lane(), wave = threadIdx.x >> 6;
    const int K = p.K, N = p.N;
    G = K >> 7;
    wn = wave;
    q = lane >> 4;
    r16 = lane & 15;
    wvalid = uniform(n0 + wn * 64) < N;  // wave has columns inside N
    // tile bases (uniform) and per-lane 32-bit offsets: K <= 2^20 keeps every
    // in-tile offset below 2^32
    xt = p.A + (size_t)row0 * K;
    wt = p.B + ((size_t)e * N + n0) * (size_t)(K >> 1);
#pragma unroll
    for (int i = 0; i < P2_X_OPS; ++i) {
      const int r = (wave * P2_X_OPS + i) * 8 + (lane >> 3);
      const int c = (lane & 7) ^ xkey(r);
      xo[i] = (uint32_t)min(r, rows - 1) * (uint32_t)K + c * 16;
    }
#pragma unroll
    for (int nb = 0; nb < 4; ++nb) {
      const int n = min(n0 + wn * 64 + nb * 16 + r16, N - 1);
      wo[nb] = (uint32_t)(n - n0) * (uint32_t)(K >> 1) + q * 16;
    }
    // LDS byte offsets of this lane's activation fragments within a slot
    xl0 = r16 * 128 + ((q ^ xkey(r16)) << 4);
    xl1 = r16 * 128 + (((q + 4) ^ xkey(r16)) << 4);
  }

  // loads of iteration t of the issue rule: W(t + P2_DW) into wnext, then
  // X(t + P2_DX); past the last group they issue with exec = 0 (addresses
  // clamped in range), so every stage issues the same number of loads
  __device__ __forceinline__ void issue(int t, v4i (&wnext)[4]) {
    const int sw = t + P2_DW;
    if (sw >= 0) p2_load_w(wnext, wt, wo, min(sw, G - 1), sw < G);
    const int sx = t + P2_DX;
    if (sx < G && sx % SC == 0) p2_issue_scales(p, lds, e, row0, rows, n0, sx / SC, R);
    p2_issue_x(xt, xo, lds + (sx % P2_NX) * P2_XSLOT, min(sx, G - 1), sx < G);
  }

  // the weights of stage s and (issued before them) its activation rows have
  // landed once at most the P2_X_OPS newest loads are in flight
  __device__ __forceinline__ void stage(int s, v4i (&wcur)[4], v4i (&wnext)[4], v4f (&acc)[8][4],
                                        v4f (&prev)[4], float& sprev) {
    wait_vm<P2_X_OPS>();
#pragma unroll
    for (int nb = 0; nb < 4; ++nb) tie(wcur[nb]);
    wg_barrier();
    issue(s, wnext);
    if (wvalid) {
      const uint8_t* slot = lds + (s % P2_NX) * P2_XSLOT;
      const uint8_t* sbb = lds + P2_SB + ((s / SC) & 1) * P2_SBBUF;
      const uint8_t* sab = lds + P2_SA + ((s / SC) & 1) * P2_SABUF;
      const int gg = s % SC;
      int sbv[4];
      // column wn*64 + 16 nb + r16 has scale key ((2 nb) & 3) ^ (r16 >> 3)
      const int k0 = gg ^ (r16 >> 3);
      const uint8_t* sbl0 = sbb + ((wn * 64 + r16) * SC + k0) * 4;
      const uint8_t* sbl1 = sbb + ((wn * 64 + r16) * SC + (k0 ^ 2)) * 4;
#pragma unroll
      for (int nb = 0; nb < 4; ++nb)
        sbv[nb] = (int)((lds32(((nb & 1) ? sbl1 : sbl0) + nb * 16 * SC * 4) >> (8 * q)) & 0xffu);
      P2Lds a;
      a.x0 = slot + xl0;
      a.x1 = slot + xl1;
      a.sa0 = sab + (r16 * SC + k0) * 4;
      a.sa1 = sab + (r16 * SC + (k0 ^ 2)) * 4;
      p2_group<NMB>(acc, prev, sprev, wcur, a, sbv);
    }
  }

  __device__ __forceinline__ void run() {
    // zero accumulators, made opaque so that the compiler does not peel the
    // first K group to specialise it for zero inputs (a second copy of the
    // loop body with its own register assignment)
    v4f acc[8][4];
#pragma unroll
    for (int a = 0; a < 8; ++a)
#pragma unroll
      for (int b = 0; b < 4; ++b) {
        acc[a][b] = v4f{0.f, 0.f, 0.f, 0.f};
        asm volatile("" : "+v"(acc[a][b]));
      }
    v4f prev[4];
#pragma unroll
    for (int b = 0; b < 4; ++b) {
      prev[b] = v4f{0.f, 0.f, 0.f, 0.f};
      asm volatile("" : "+v"(prev[b]));
    }
    float sprev = 0.f;
    asm volatile("" : "+v"(sprev));
    v4i w0[4], w1[4];
#pragma unroll
    for (int nb = 0; nb < 4; ++nb) w0[nb] = w1[nb] = v4i{0, 0, 0, 0};

    // prologue = iterations -P2_DX .. -1 of the issue rule; W(0) lands in w0
    issue(-2, w1);
    issue(-1, w0);
    // whole pairs of stages, then the last odd one: no control-flow path
    // skips a stage and then runs a later one
    int s = 0;
    for (; s + 2 <= G; s += 2) {
      stage(s, w0, w1, acc, prev, sprev);
      stage(s + 1, w1, w0, acc, prev, sprev);
    }
    if (s < G) stage(s, w0, w1, acc, prev, sprev);
    wait_vm<0>();  // every load has retired; the ties keep their registers reserved until here
#pragma unroll
    for (int nb = 0; nb < 4; ++nb) {
      tie(w0[nb]);
      tie(w1[nb]);
    }
#pragma unroll
    for (int nb = 0; nb < 4; ++nb) promote(acc[NMB - 1][nb], sprev, prev[nb]);
    __syncthreads();  // every wave is done with the ring before the next tile's loads

    if (wvalid) {
      // lane coordinates recomputed (opaque) rather than kept live through the K loop
      int t = threadIdx.x;
      asm volatile("" : "+v"(t));
      const int eq = (t >> 4) & 3, er = t & 15;
      const int ncol = n0 + (t >> 6) * 64 + eq * 4;
      const int N = p.N;
#pragma unroll
      for (int mi = 0; mi < NMB; ++mi) {
        const int m = mi * 16 + er;
        if (m < rows) {
          uint16_t* crow = p.C + (size_t)(row0 + m) * N;
#pragma unroll
          for (int nb = 0; nb < 4; ++nb) {
            const int n = ncol + nb * 16;
            if (n < N) store_bf16x4(crow + n, acc[mi][nb]);
          }
        }
      }
    }
  }
};
static_assert(P2_DX == 2, "the prologue issues iterations -2 and -1");

__device__ __forceinline__ void mfma_tile(const GemmArgs& p, uint8_t* lds, int e, int row0, int rows,
                                          int n0, int R) {
  switch ((rows + 15) >> 4) {
    case 1: MfmaTile<1>(p, lds, e, row0, rows, n0, R).run(); break;
    case 2: MfmaTile<2>(p, lds, e, row0, rows, n0, R).run(); break;
    case 3: MfmaTile<3>(p, lds, e, row0, rows, n0, R).run(); break;
    case 4: MfmaTile<4>(p, lds, e, row0, rows, n0, R).run(); break;
    case 5: MfmaTile<5>(p, lds, e, row0, rows, n0, R).run(); break;
    case 6: MfmaTile<6>(p, lds, e, row0, rows, n0, R).run(); break;
    case 7: MfmaTile<7>(p, lds, e, row0, rows, n0, R).run(); break;
    default: MfmaTile<8>(p, lds, e, row0, rows, n0, R).run(); break;
  }
}

// Work item of round r for workgroup b.  Workgroups are dealt to the eight
// XCDs round-robin (b % 8), each XCD with its own L2, so the items of one
// round are regrouped to give every XCD a contiguous block of item numbers.
__device__ __forceinline__ int xcd_item(int r, int b, int grid) {
  if ((grid & 7) != 0) return r * grid + b;
  return r * grid + (b & 7) * (grid >> 3) + (b >> 3);
}

// Item number -> (m-tile, n-tile): bands of P2_SUPER m-tiles, n-tiles in
// order within a band and m fastest, so a block of consecutive items shares
// a few m-tiles (activation rows) and a few n-tiles (weight columns).
constexpr int P2_SUPER = 4;
__device__ __forceinline__ void item_tile(int L, int MT, int NT, int* mt, int* nt) {
  const int band = L / (P2_SUPER * NT);
  const int rem = L - band * P2_SUPER * NT;
  const int rg = min(P2_SUPER, MT - band * P2_SUPER);
  *mt = band * P2_SUPER + rem % rg;
  *nt = rem / rg;
}

// ---------------------------------------------------------------------------
// The kernel: plan prologue, then both phases.
// ---------------------------------------------------------------------------
__global__ void __launch_bounds__(BLOCK, 1)
grouped_gemm_kernel(GemmArgs p) {
  __shared__ __attribute__((aligned(16))) uint8_t lds[P2_BYTES > P1_BYTES ? P2_BYTES : P1_BYTES];
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
        case 1: stream_item<1>(p, lds, e, row0, rows, n0, R); break;
        case 2: stream_item<2>(p, lds, e, row0, rows, n0, R); break;
        default: stream_item<3>(p, lds, e, row0, rows, n0, R); break;
      }
    }
  }

  // phase 2: MFMA tiles, one workgroup each
  {
    // MT <= R / 65 + E and NT <= 2^31 / 512 keep the item count in 32 bits
    const int MT = uniform(s_mbase[p.E]);
    const int NT = (p.N + MF_BN - 1) / MF_BN;
    const int items = MT * NT;
    const int grid = gridDim.x;
    const int rounds = (items + grid - 1) / grid;
    for (int r = 0; r < rounds; ++r) {
      const int L = xcd_item(r, blockIdx.x, grid);
      if (L >= items) continue;
      int mt, nt;
      item_tile(L, MT, NT, &mt, &nt);
      const int e = uniform(expert_of_tile(s_mbase, p.E, mt));
      const int j = mt - uniform(s_mbase[e]);
      const int base = uniform(s_off[e]);
      const int rows_e = uniform(s_off[e + 1]) - base;
      const TileChoice tc = tile_rule(rows_e);
      const int row0 = base + j * tc.tile_m;
      const int rows = min(tc.tile_m, rows_e - j * tc.tile_m);
      mfma_tile(p, lds, e, row0, rows, nt * MF_BN, R);
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
