// MFMA-tile phase of the grouped W4A8 GEMM kernel (gemm.hip): the experts
// with more than S_MAX rows, whose m-tiles (at most T_MAX rows each, sized
// per expert by the tile rule) make the contraction compute-bound.  All
// vector-memory ops of the K loop are inline asm with explicit waits
// (w4a8_kernel.h); all loads use clamped addresses (padding rows and columns
// re-read a real one and are never stored).  gfx950 only.
#pragma once

#include "swiglu.h"
#include "w4a8_kernel.h"

namespace w4a8 {

// ---------------------------------------------------------------------------
// Tiles of 512 (n) x 128 (m) per workgroup.
//
// Wave w owns columns 64w .. 64w+63 of the tile and all of its rows (4 x 8
// MFMA blocks, 128 fp32 accumulators per lane).  Every weight byte of the
// tile is needed by exactly one wave, so weights go from global memory
// straight into that wave's MFMA operand registers (two register slots: the
// next group's weights load while the current group's are in use); only the
// activation rows and the scales, which every wave needs, are staged in LDS
// through direct global->LDS loads:
//   X ring   : 6 slots (three pairs of groups) x [128 rows][128 B]
//              (row chunk c at c ^ xkey(row))
//   SB chunk : 2 x [512 cols][SC] u32  (E8M0 codes of groups SC*c .. SC*c+3,
//              word gg of column n at n * SC + gg)
//   SA chunk : 2 x [128 rows][SC] fp32 (word gg of row r at gg ^ skey(r))
// The K loop runs in pairs of groups with one barrier per pair (a barrier per
// group measured 2-3% slower): wait for the weights of the pair's first group,
// barrier, its 32 MFMAs; wait for the weights of the second group, issue the
// activation rows of the two groups four ahead, the scale chunk they open (if
// any) and the weights of the next pair's first group into the register slot
// just used; the second group's MFMAs; the weights of the next pair's second
// group.  Each weight load has one group of lead, each activation load one
// and a half pairs.  One in-order counter per wave: every wait is counted
// from the issue order (see pair()).
// Per 128-K group a workgroup reads 32 KB of weights and 16 KB of activations
// for 256 MFMAs, the fewest bytes per MFMA of the tile shapes whose
// accumulators fit two waves per SIMD.
// ---------------------------------------------------------------------------
constexpr int MF_THREADS = 512;
constexpr int MF_WAVES = MF_THREADS / 64;
constexpr int MF_BN = TN_MFMA;          // 512 weight columns
constexpr int MF_BM = T_MAX;            // 128 activation rows
constexpr int P2_NX = 6;                // activation ring slots: three pairs of groups
constexpr int P2_XSLOT = MF_BM * 128;   // 16 KB
constexpr int P2_SB = P2_NX * P2_XSLOT;
constexpr int P2_SBBUF = MF_BN * SC * 4;  // 8 KB
constexpr int P2_SA = P2_SB + 2 * P2_SBBUF;
constexpr int P2_SABUF = MF_BM * SC * 4;  // 2 KB
constexpr int P2_BYTES = P2_SA + 2 * P2_SABUF;
constexpr int P2_X_OPS = MF_BM * 128 / 1024 / MF_WAVES;  // activation loads per wave per stage
static_assert(MF_BN == 64 * MF_WAVES, "each wave owns 64 columns");
static_assert(P2_X_OPS * 1024 * MF_WAVES == MF_BM * 128, "activation loads cover the slot");
static_assert(MF_BN == MF_WAVES * 64, "one 16-byte E8M0 load per column covers a chunk");
static_assert(MF_BM * SC == MF_WAVES * 64, "one 4-byte activation-scale load per lane covers a chunk");
// a scale chunk (two pairs) is refilled during the pair two before its first
// one, after every pair of the chunk two back has passed that pair's barrier
static_assert(SC == 4, "a scale chunk is two pairs of groups");


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

// Fused SwiGLU GEMM: weight column of tile-local column t (0 .. 511) of the
// tile whose output columns start at c0.  Each wave's 64 columns are the
// gate (first 32) and the up projection (last 32) of the same 32 output
// columns c0 + 32 w .. c0 + 32 w + 31, so a lane holds gate and up of its
// outputs in the same accumulator positions (blocks nb and nb + 2).
// Output columns past I read the last one (never stored).
__device__ __forceinline__ int fused_col(int c0, int t, int I) {
  const int oc = min(c0 + (t >> 6) * 32 + (t & 31), I - 1);
  return (t & 32) ? I + oc : oc;
}

// Coordinates of an MFMA tile: expert, first row, rows, first column
// (an output column of A2 for the fused SwiGLU GEMM).
struct TileCoord {
  int e, row0, rows, n0;
  bool valid;
};

template <int NMB, bool FUSED = false>
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
    // wave has columns inside N (inside I for the fused GEMM)
    wvalid = FUSED ? uniform(n0 + wn * 32) < p.I : uniform(n0 + wn * 64) < N;
    // tile bases (uniform) and per-lane 32-bit offsets: K <= 2^20 keeps every
    // in-tile offset below 2^32 (the fused GEMM's offsets are from the
    // expert's first column: N * K / 2 < 2^31 is checked on the host)
    xt = p.A + (size_t)row0 * K;
    wt = FUSED ? p.B + (size_t)e * N * (size_t)(K >> 1) : p.B + ((size_t)e * N + n0) * (size_t)(K >> 1);
#pragma unroll
    for (int i = 0; i < P2_X_OPS; ++i) {
      const int r = (wave * P2_X_OPS + i) * 8 + (lane >> 3);
      const int c = (lane & 7) ^ xkey(r);
      xo[i] = (uint32_t)min(r, rows - 1) * (uint32_t)K + c * 16;
    }
#pragma unroll
    for (int nb = 0; nb < 4; ++nb) {
      if constexpr (FUSED) {
        wo[nb] = (uint32_t)fused_col(n0, wn * 64 + nb * 16 + r16, p.I) * (uint32_t)(K >> 1) + q * 16;
      } else {
        const int n = min(n0 + wn * 64 + nb * 16 + r16, N - 1);
        wo[nb] = (uint32_t)(n - n0) * (uint32_t)(K >> 1) + q * 16;
      }
    }
    // LDS byte offsets of this lane's activation fragments within a slot
    xl0 = r16 * 128 + ((q ^ xkey(r16)) << 4);
    xl1 = r16 * 128 + (((q + 4) ^ xkey(r16)) << 4);
  }

  // One weight load of group g: 16 columns (block nb) x 64 B into w.
  __device__ __forceinline__ void load_w(v4i& w, int nb, int g) const {
    vm_load16(w, wt + (size_t)max(0, min(g, G - 1)) * 64, wo[nb], live_mask(g >= 0 && g < G));
  }

  // One activation load of group g: 8 rows x 128 B into ring slot g % P2_NX.
  __device__ __forceinline__ void load_x(int i, int g) const {
    const int wave = uniform(threadIdx.x >> 6);
    vm_dma16(xt + (size_t)min(g, G - 1) * 128, xo[i],
             lds_u32(lds + (g % P2_NX) * P2_XSLOT + (wave * P2_X_OPS + i) * 1024), live_mask(g < G));
  }

  // Scale chunk c (groups SC*c .. SC*c+3).  E8M0: a column's codes of SC
  // consecutive groups are 16 contiguous bytes, so one 16-byte load per column
  // (wave w: columns 64w .. 64w+63), word gg of column n at n * SC + gg (a
  // 4-byte read of 16 consecutive columns then hits 16 distinct banks); the
  // load starts at group SC*c clamped to G - SC so that it stays inside the
  // column, and the word of group g then sits at g - load start (sb_word).
  // With fewer than SC groups in all, four 4-byte loads per wave, groups
  // clamped.  Activation scales: 128 rows x SC groups, one 4-byte load per
  // lane; four lanes read one row's SC words (row-major) and word gg of row r
  // lands at position gg ^ skey(r).
  __device__ __forceinline__ void load_scales(int c) const {
    const int lane = opaque_lane(), wave = uniform(threadIdx.x >> 6);
    const int K = p.K, N = p.N;
    if (G >= SC) {
      const int col = wave * 64 + lane;
      const int n = FUSED ? fused_col(n0, col, p.I) : min(n0 + col, N - 1) - n0;
      const int g = min(SC * c, G - SC);
      const uint8_t* base = p.SB + ((size_t)e * N + (FUSED ? 0 : n0)) * (size_t)(K >> 5) + (size_t)g * 4;
      vm_dma16(base, (uint32_t)n * (uint32_t)(K >> 5), lds_u32(lds + P2_SB + (c & 1) * P2_SBBUF + wave * 1024),
               live_mask(true));
    } else {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int col = ((wave * 4 + i) * 64 + lane) >> 2;
        const int g = min(SC * c + (lane & 3), G - 1);
        const int n = FUSED ? fused_col(n0, col, p.I) : min(n0 + col, N - 1);
        vm_dma4(p.SB + ((size_t)e * N + n) * (size_t)(K >> 5) + (size_t)g * 4,
                lds_u32(lds + P2_SB + (c & 1) * P2_SBBUF + (wave * 4 + i) * 256));
      }
    }
    const int r = (wave * 64 + lane) >> 2;  // rows [row] of SC words
    const int g = min(SC * c + ((lane & 3) ^ skey<SC>(r)), G - 1);
    const size_t row = (size_t)row0 + min(r, rows - 1);
    vm_dma4(sa_ptr(p, row, g, G, R), lds_u32(lds + P2_SA + (c & 1) * P2_SABUF + wave * 256));
  }
  __device__ __forceinline__ int sb_word(int g) const {
    return (g % SC) + (G >= SC ? max(0, SC * (g / SC) - (G - SC)) : 0);
  }

  // One K group: step mi issues the LDS reads of block mi+1 and the four
  // MFMAs of block mi; after each MFMA come the four promotion FMAs of the
  // partial two MFMAs back (the last two partials of a group are carried into
  // the next group in pq, with their row block's scale in sprev), so the
  // FMAs never wait for the MFMA just issued and only three partials are
  // live at a time.  The scheduling fences keep each step's work together.
  __device__ __forceinline__ void group(v4f (&acc)[8][4], v4f (&pq)[2], float& sprev, const v4i (&w)[4],
                                        const P2Lds& a, const int (&sbv)[4]) const {
    v4i xa0, xa1;
    float saa;
    p2_read_x(a, 0, xa0, xa1, saa);
#pragma unroll
    for (int mi = 0; mi < NMB; ++mi) {
      v4i xb0 = xa0, xb1 = xa1;
      float sab_n = saa;
      if (mi + 1 < NMB) p2_read_x(a, mi + 1, xb0, xb1, sab_n);
      // the block before this one: the last block of the previous group when mi == 0
      const int pm = mi == 0 ? NMB - 1 : mi - 1;
#pragma unroll
      for (int nb = 0; nb < 4; ++nb) {
        const v4f r = mfma_group(w[nb], xa0, xa1, sbv[nb]);
        if (nb >= 2)
          promote(acc[mi][nb - 2], saa, pq[nb & 1]);
        else
          promote(acc[pm][nb + 2], sprev, pq[nb & 1]);
        pq[nb & 1] = r;
      }
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

  // Operand pointers of group g for this lane.
  __device__ __forceinline__ void group_ptrs(int g, P2Lds& a, int (&sbv)[4]) const {
    const uint8_t* slot = lds + (g % P2_NX) * P2_XSLOT;
    const uint8_t* sbb = lds + P2_SB + ((g / SC) & 1) * P2_SBBUF;
    const uint8_t* sab = lds + P2_SA + ((g / SC) & 1) * P2_SABUF;
    const int gg = g % SC;
    const int k0 = gg ^ (r16 >> 3);
    const uint8_t* sbl = sbb + ((wn * 64 + r16) * SC + sb_word(g)) * 4;
#pragma unroll
    for (int nb = 0; nb < 4; ++nb) sbv[nb] = (int)((lds32(sbl + nb * 16 * SC * 4) >> (8 * q)) & 0xffu);
    a.x0 = slot + xl0;
    a.x1 = slot + xl1;
    a.sa0 = sab + (r16 * SC + k0) * 4;
    a.sa1 = sab + (r16 * SC + (k0 ^ 2)) * 4;
  }

  // Pair t = groups 2t and 2t+1, one barrier.  Issue order: after group 2t,
  // activation rows of groups 2t+4, 2t+5 (ring slots of pair t-1, which every
  // wave finished before this pair's barrier), the scale chunk group 2t+4
  // opens, the weights of 2t+2 (into w0, free now); after group 2t+1, the
  // weights of 2t+3.  So at the start of pair t+1 only the weights of 2t+3
  // may still be in flight (wait for at most 4), and before group 2t+3
  // nothing newer than them was issued (wait for 0).  Loads past the last
  // group run with exec = 0 from clamped addresses.
  __device__ __forceinline__ void pair(int t, v4i (&w0)[4], v4i (&w1)[4], v4f (&acc)[8][4], v4f (&pq)[2],
                                       float& sprev) {
    const int g0 = 2 * t, g1 = 2 * t + 1;
    wait_vm<4>();  // weights of g0 (only those of g1 may be in flight)
#pragma unroll
    for (int nb = 0; nb < 4; ++nb) tie(w0[nb]);
    wg_barrier();
    P2Lds a;
    int sbv[4];
    if (wvalid) {
      group_ptrs(g0, a, sbv);
      group(acc, pq, sprev, w0, a, sbv);
    }
    wait_vm<0>();  // weights of g1
#pragma unroll
    for (int nb = 0; nb < 4; ++nb) tie(w1[nb]);
#pragma unroll
    for (int i = 0; i < P2_X_OPS; ++i) load_x(i, g0 + 4);
#pragma unroll
    for (int i = 0; i < P2_X_OPS; ++i) load_x(i, g1 + 4);
    if (g0 + 4 < G && (g0 + 4) % SC == 0) load_scales((g0 + 4) / SC);
#pragma unroll
    for (int nb = 0; nb < 4; ++nb) load_w(w0[nb], nb, g0 + 2);
    if (wvalid && g1 < G) {
      group_ptrs(g1, a, sbv);
      group(acc, pq, sprev, w1, a, sbv);
    }
#pragma unroll
    for (int nb = 0; nb < 4; ++nb) load_w(w1[nb], nb, g1 + 2);
  }

  // The first shared-operand loads of this tile: activation rows of groups
  // 0-3 into ring slots 0-3 and scale chunk 0.  The workgroup's previous tile
  // issues them before its epilogue (so they land while it stores), or the
  // tile itself if it is the workgroup's first.  They hold no registers.
  __device__ __forceinline__ void prologue_shared() const {
#pragma unroll
    for (int g = 0; g < 4; ++g)
#pragma unroll
      for (int i = 0; i < P2_X_OPS; ++i) load_x(i, g);
    load_scales(0);
  }

  // The K loop of this tile (its shared-operand prologue issued already if
  // shared_ready), then, once every wave is done with the ring, the shared-
  // operand prologue of the workgroup's next tile (next() gives its
  // coordinates, valid == false if there is none; it is called only after
  // the K loop, so its results are not live across it), then the bf16
  // epilogue of this one.  Returns the next tile's coordinates.
  template <class Next>
  __device__ __forceinline__ TileCoord run(bool shared_ready, Next next) {
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
    v4f pq[2];
#pragma unroll
    for (int b = 0; b < 2; ++b) {
      pq[b] = v4f{0.f, 0.f, 0.f, 0.f};
      asm volatile("" : "+v"(pq[b]));
    }
    float sprev = 0.f;
    asm volatile("" : "+v"(sprev));
    v4i w0[4], w1[4];
#pragma unroll
    for (int nb = 0; nb < 4; ++nb) w0[nb] = w1[nb] = v4i{0, 0, 0, 0};
    // prologue: activation rows of groups 0-3 and scale chunk 0 (unless the
    // previous tile issued them), weights of groups 0 and 1 -- the loads the
    // first pair's waits count
    if (!shared_ready) prologue_shared();
#pragma unroll
    for (int nb = 0; nb < 4; ++nb) load_w(w0[nb], nb, 0);
#pragma unroll
    for (int nb = 0; nb < 4; ++nb) load_w(w1[nb], nb, 1);
    const int P = (G + 1) / 2;
    for (int t = 0; t < P; ++t) pair(t, w0, w1, acc, pq, sprev);
    wait_vm<0>();  // every load has retired; the ties keep their registers reserved until here
#pragma unroll
    for (int nb = 0; nb < 4; ++nb) {
      tie(w0[nb]);
      tie(w1[nb]);
    }
    promote(acc[NMB - 1][2], sprev, pq[0]);
    promote(acc[NMB - 1][3], sprev, pq[1]);
    __syncthreads();  // every wave is done with the ring before the next tile's loads
    // (the epilogue's stores, issued after these loads, only make the next
    // tile's first wait, which counts the newest operations, wait for more
    // than it needs)
    const TileCoord nt = next();
    if (nt.valid) MfmaTile<1, FUSED>(p, lds, nt.e, nt.row0, nt.rows, nt.n0, R).prologue_shared();

    if constexpr (FUSED) {
      fused_epilogue(acc);
    } else if (wvalid) {
      plain_epilogue(acc);
    }
    return nt;
  }

  // bf16 epilogue.  A lane holds 4 consecutive columns (8 bytes) of one row
  // per accumulator block; stored as they are, a store instruction writes 32-
  // byte pieces of 16 rows, and the tile's stores touch four times as many
  // cache lines as it has, all workgroups at once.  So each wave passes its
  // 64 columns through 4 KB of its own in ring slots 4-5 (free: the next
  // tile's first loads fill slots 0-3 and scale chunk 0, and slots 4-5 are
  // refilled only after that tile's first barrier, which every wave reaches
  // after this), two row blocks at a time, and stores whole rows: 128 bytes
  // (8 lanes x 16) per row.  In the staging rows 16-byte chunk c of row r is
  // at c ^ (r & 7).
  __device__ __forceinline__ void plain_epilogue(v4f (&acc)[8][4]) {
    // lane coordinates recomputed (opaque) rather than kept live through the K loop
    int t = threadIdx.x;
    asm volatile("" : "+v"(t));
    const int w = t >> 6, l = t & 63;
    const int eq = (t >> 4) & 3, er = t & 15;
    const int N = p.N;
    uint8_t* st = lds + 4 * P2_XSLOT + w * 4096;
    const int lr = l >> 3, lc = l & 7;              // read: row lr (+8u), chunk lc
    const int col = n0 + w * 64 + lc * 8;           // first of the chunk's 8 columns
#pragma unroll
    for (int rb = 0; rb < (NMB + 1) / 2; ++rb) {
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int mi = 2 * rb + h;
        if (mi < NMB) {
          const int r = h * 16 + er;
#pragma unroll
          for (int nb = 0; nb < 4; ++nb) {
            const int c = 2 * nb + (eq >> 1);
            const v4f v = acc[mi][nb];
            const v2bf lo = __builtin_convertvector((v2f){v[0], v[1]}, v2bf);
            const v2bf hi = __builtin_convertvector((v2f){v[2], v[3]}, v2bf);
            uint2 o;
            o.x = __builtin_bit_cast(uint32_t, lo);
            o.y = __builtin_bit_cast(uint32_t, hi);
            *reinterpret_cast<uint2*>(st + r * 128 + ((c ^ (r & 7)) << 4) + (eq & 1) * 8) = o;
          }
        }
      }
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int r = u * 8 + lr;               // staging row
        const int m = rb * 32 + r;              // tile row
        if (m < rows && (2 * rb + (r >> 4)) < NMB) {
          const v4i v = *reinterpret_cast<const v4i*>(st + r * 128 + ((lc ^ (r & 7)) << 4));
          if (col < N) *reinterpret_cast<v4i*>(p.C + (size_t)(row0 + m) * N + col) = v;
        }
      }
    }
  }

  // Fused SwiGLU epilogue: lane (q, i) holds, for row block mi, gate in
  // acc[mi][0..1] and up in acc[mi][2..3] of output columns c0 + 32 w +
  // 16 j + 4 q .. +3 (j = 0, 1) of row 16 mi + i.  h = silu(gate) * up
  // replaces the gate accumulators; each row's amax over the wave's 32
  // columns goes through LDS to the four waves of its 128-column group
  // (waves 0-3: c0 .. c0+127, waves 4-7: c0+128 ..).  The LDS words used
  // are in ring slots 4-5, which the next tile's first loads (slots 0-3,
  // scale chunk 0) leave alone and its first K pair refills only after its
  // first barrier.  Every wave reaches the barrier, with columns or not.
  __device__ __forceinline__ void fused_epilogue(v4f (&acc)[8][4]) {
    float* s_amax = reinterpret_cast<float*>(lds + 4 * P2_XSLOT);  // [8 waves][128 rows]
    int t = threadIdx.x;
    asm volatile("" : "+v"(t));
    const int w = t >> 6, eq = (t >> 4) & 3, er = t & 15;
    if (wvalid) {
#pragma unroll
      for (int mi = 0; mi < NMB; ++mi) {
        float m = 0.f;
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
          for (int c = 0; c < 4; ++c) {
            acc[mi][j][c] = swiglu_f32(acc[mi][j][c], acc[mi][j + 2][c]);
            m = fmaxf(m, fabsf(acc[mi][j][c]));
          }
        m = fmaxf(m, __shfl_xor(m, 16));
        m = fmaxf(m, __shfl_xor(m, 32));
        if (eq == 0) s_amax[w * 128 + mi * 16 + er] = m;
      }
    }
    __syncthreads();
    if (wvalid) {
      const int I = p.I, G2 = I >> 7;
      const int grp = (n0 >> 7) + (w >> 2);          // 128-column group of this wave's columns
      const float* am = s_amax + (w & 4) * 128;      // the group's four waves
#pragma unroll
      for (int mi = 0; mi < NMB; ++mi) {
        const int m = mi * 16 + er;
        if (m < rows) {
          const float amax = fmaxf(fmaxf(am[m], am[128 + m]), fmaxf(am[256 + m], am[384 + m]));
          const float s = e4m3_group_scale(amax);
          const float inv = __fdiv_rn(1.0f, s);
          const size_t row = (size_t)row0 + m;
          uint8_t* arow = p.A2 + row * I + n0 + w * 32 + eq * 4;
#pragma unroll
          for (int j = 0; j < 2; ++j) {
            const v4f h = acc[mi][j];
            *reinterpret_cast<uint32_t*>(arow + 16 * j) = e4m3x4(h[0], h[1], h[2], h[3], inv);
          }
          if ((w & 3) == 0 && eq == 0)
            p.SA2[p.layout2 ? (size_t)grp * R + row : row * G2 + grp] = s;
        }
      }
    }
  }
};

template <bool FUSED = false, class Next>
__device__ __forceinline__ TileCoord mfma_tile(const GemmArgs& p, uint8_t* lds, const TileCoord& t, int R,
                                               bool shared_ready, Next next) {
  switch ((t.rows + 15) >> 4) {
    case 1: return MfmaTile<1, FUSED>(p, lds, t.e, t.row0, t.rows, t.n0, R).run(shared_ready, next);
    case 2: return MfmaTile<2, FUSED>(p, lds, t.e, t.row0, t.rows, t.n0, R).run(shared_ready, next);
    case 3: return MfmaTile<3, FUSED>(p, lds, t.e, t.row0, t.rows, t.n0, R).run(shared_ready, next);
    case 4: return MfmaTile<4, FUSED>(p, lds, t.e, t.row0, t.rows, t.n0, R).run(shared_ready, next);
    case 5: return MfmaTile<5, FUSED>(p, lds, t.e, t.row0, t.rows, t.n0, R).run(shared_ready, next);
    case 6: return MfmaTile<6, FUSED>(p, lds, t.e, t.row0, t.rows, t.n0, R).run(shared_ready, next);
    case 7: return MfmaTile<7, FUSED>(p, lds, t.e, t.row0, t.rows, t.n0, R).run(shared_ready, next);
    default: return MfmaTile<8, FUSED>(p, lds, t.e, t.row0, t.rows, t.n0, R).run(shared_ready, next);
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
// a few m-tiles (activation rows) and a few n-tiles (weight columns): the 32
// items an XCD runs at once cover 8 m-tiles x 4 n-tiles, whose 128 KB of
// activations and 128 KB of weights per K group are what its L2 fetches.
constexpr int P2_SUPER = 8;
__device__ __forceinline__ void item_tile(int L, int MT, int NT, int* mt, int* nt) {
  const int band = L / (P2_SUPER * NT);
  const int rem = L - band * P2_SUPER * NT;
  const int rg = min(P2_SUPER, MT - band * P2_SUPER);
  *mt = band * P2_SUPER + rem % rg;
  *nt = rem / rg;
}

}  // namespace w4a8
