// Weight-streaming phase of the grouped W4A8 GEMM kernel (gemm.hip): the
// experts with at most S_MAX rows (decode-sized batches, where HBM bandwidth
// is the limit).  gfx950 only.
//
// One workgroup of 512 threads (8 waves) per item (expert, 64..192 columns,
// width picked per launch): waves 0-3 take the first half of the K groups
// and waves 4-7 the second half, two groups per stage.  Weights stream from
// HBM straight into MFMA operand registers (a per-wave ring two stages deep);
// the activation rows and the scales are shared through LDS with direct
// global->LDS loads (global_load_lds_dwordx4 / _dword), which hold no
// registers while in flight: every wave issues the same number of loads per
// stage, waits for the stage it needs with one explicit vmcnt and meets the
// others at one barrier per stage.  The halves are added in LDS (always half
// 0 + half 1) before the bf16 store.  The E8M0 and activation scales are
// loaded four groups at a time (four lanes read 16 contiguous bytes) into a
// double buffer.  The XOR swizzle that keeps fragment reads free of LDS bank
// conflicts is applied on the global-address side (a load lane always writes
// slot base + size * lane).  All loads use clamped addresses (padding rows and
// columns re-read a real one and are never stored), so no load is
// conditional on data.
#pragma once

#include "w4a8_kernel.h"

namespace w4a8 {

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
//   SA chunk : 2 x [2 halves][64 rows][SC] fp32               @ P1_SB + 2 * SBS
// Stage s: wait (the weights of stage s and, older, its activation rows have
// landed), barrier, issue the activation rows of stage s + D, MFMAs, then the
// weights of stage s + D into the register slot just used.  After the K loop
// the halves are added through LDS (always half 0 + half 1, whatever the item
// width or stage size), then rounded to bf16 and stored.
// ---------------------------------------------------------------------------
constexpr int P1_XGROUP = 16384;          // activation rows of one group, both halves
constexpr int P1_XRING = 6 * P1_XGROUP;   // (D+1)*KG groups, at most 96 KB
// widest item in 64-column units, per row blocks of the expert (the weight
// ring, 16*NBW registers, and the accumulators, 4*NBW*MB, share the
// register file with the MFMA operands)
constexpr int P1_MAXNBW = 4;
__host__ __device__ constexpr int stream_max_nbw(int mb) { return mb <= 2 ? 4 : 3; }
// items of a contiguous range are at most this wide (wider measured no faster)
constexpr int P1_RANGE_MAXNBW = 3;
// groups of K per streaming stage: two halve the per-stage barriers and LDS
// round trips against one, at the same bytes in flight (four, with a single
// stage in flight, measured slower)
constexpr int P1_KG = 2;
constexpr int P1_SB = P1_XRING;
// SB chunk buffers are max(6 KB, NBW * 2 KB) apart: items up to three units
// wide keep the 6 KB spacing (an 8 KB spacing measured 5% slower for them)
__host__ __device__ constexpr int stream_sb_stride(int nbw) { return nbw <= 3 ? 6144 : 2048 * nbw; }
constexpr int P1_SBMAX = 2 * stream_sb_stride(P1_MAXNBW);
constexpr int P1_SABUF = 2 * 64 * SC * 4;                  // 2 KB
constexpr int P1_BYTES = P1_SB + P1_SBMAX + 2 * P1_SABUF;

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
  static_assert(NBW <= stream_max_nbw(MB), "register budget");
  static constexpr int SBS = stream_sb_stride(NBW);  // SB chunk buffer spacing
  static constexpr int SAB = P1_SB + 2 * SBS;        // SA chunk buffers
  static_assert(SBS >= 2 * 64 * NBW * SC * 4 && SAB + 2 * P1_SABUF <= P1_BYTES, "scale chunk buffers");
  static_assert(4 * NBW * MB * 1024 <= P1_SB, "reduction scratch must fit below the scale chunks");

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
              lds_u32(lds + P1_SB + (c & 1) * SBS + (wave * NBW + i) * 256));
    }
    {
      const int idx = wave * 64 + lane;  // [h][row][gg]
      const int h = idx >> 8, r = (idx >> 2) & 63, gg = idx & 3;
      const size_t row = (size_t)row0 + min(r, rows - 1);
      const int g = min((h ? gb1 : 0) + SC * c + gg, G - 1);
      vm_dma4(sa_ptr(p, row, g, G, R), lds_u32(lds + SAB + (c & 1) * P1_SABUF + wave * 256));
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
      // the ring slot is free once paired: its next loads go out before the
      // MFMAs, so two stages stay in flight while this one computes
      load_w(wr[u], wt, wo, gbase + min(sn, S - 1) * KG, G, sn < S);
#pragma unroll
      for (int kg = 0; kg < KG; ++kg) {
        const int gl = s * KG + kg;  // group index within this wave's half
        if (gl < gcount) {
          const uint8_t* sbb = lds + P1_SB + ((gl / SC) & 1) * SBS;
          const uint8_t* sab = lds + SAB + ((gl / SC) & 1) * P1_SABUF;
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
    // one per-lane base (the wave's slice of the scratch is a uniform offset),
    // constant offsets per (unit, row block)
    v4f* red = reinterpret_cast<v4f*>(lds) + uniform(wn) * (NBW * MB * 64) + lane;
    if (kh == 1) {
#pragma unroll
      for (int j = 0; j < NBW; ++j)
#pragma unroll
        for (int i = 0; i < MB; ++i) red[(j * MB + i) * 64] = acc[j][i];
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
            const v4f o = red[(j * MB + i) * 64];
            if (n < N) store_bf16x4(crow + n, acc[j][i] + o);
          }
        }
      }
    }
    __syncthreads();  // red is overwritten by the next item's loads
  }
};

template <int MB>
__device__ __forceinline__ void stream_item_mb(const GemmArgs& p, uint8_t* lds, int e, int row0, int rows, int n0,
                                               int nbw, int R) {
  switch (nbw) {
    case 1: StreamItem<1, P1_KG, MB>::run(p, lds, e, row0, rows, n0, R); break;
    case 2: StreamItem<2, P1_KG, MB>::run(p, lds, e, row0, rows, n0, R); break;
    case 3: StreamItem<3, P1_KG, MB>::run(p, lds, e, row0, rows, n0, R); break;
    default: if constexpr (stream_max_nbw(MB) >= 4) StreamItem<4, P1_KG, MB>::run(p, lds, e, row0, rows, n0, R); break;
  }
}

// One streaming item of nbw units (nbw <= stream_max_nbw of its row blocks).
__device__ __forceinline__ void stream_item(const GemmArgs& p, uint8_t* lds, int e, int row0, int rows, int n0,
                                            int nbw, int R) {
  switch ((rows + 15) >> 4) {
    case 1: stream_item_mb<1>(p, lds, e, row0, rows, n0, nbw, R); break;
    case 2: stream_item_mb<2>(p, lds, e, row0, rows, n0, nbw, R); break;
    case 3: stream_item_mb<3>(p, lds, e, row0, rows, n0, nbw, R); break;
    default: stream_item_mb<4>(p, lds, e, row0, rows, n0, nbw, R); break;
  }
}

// Items dealt round-robin (experts of different row blocks).  Expert e's
// items are w = min(W, stream_max_nbw(its row blocks)) units wide, with the
// cap W that minimises rounds x per-item bytes, per-item bytes ~ weights (32
// per unit per K) plus activation rows (about 32 per K): wider items re-read
// the activation rows less often and pay the pipeline fill and drain fewer
// times, narrower ones spread few experts over more workgroups.  Items are
// numbered in decreasing order of their cost, w * (4 + row blocks), in four
// classes (the row blocks), and dealt in a snake order (round r gives
// workgroup b item r*G + b for even r, r*G + G-1-b for odd r), so that a
// workgroup's second item is light when its first was heavy.
//   s_eord[k]   expert at class-ordered position k
//   s_rrc[r]    class of rank r: {first item, first position, items per expert, width}
//   s_rrc[4][0] total items
// Wave 0 fills them; every thread must call it.
__device__ __forceinline__ void stream_rr_plan(const int* s_off, int E, int nu, int grid, int* s_eord,
                                               int (*s_rrc)[4]) {
  if (threadIdx.x < 64) {
    const int lane = threadIdx.x;
    const int per = (E + 63) / 64;
    const int i0 = lane * per;
    int cnt[4] = {0, 0, 0, 0};
    for (int k = 0; k < per; ++k) {
      const int e = i0 + k;
      if (e < E) {
        const int rows = s_off[e + 1] - s_off[e];
        if (rows > 0 && rows <= S_MAX) {
          const int c = (rows - 1) >> 4;
#pragma unroll
          for (int j = 0; j < 4; ++j) cnt[j] += j == c;
        }
      }
    }
    int pre[4], tot[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int incl = wave_inclusive_sum(cnt[j]);
      pre[j] = incl - cnt[j];
      tot[j] = __builtin_amdgcn_readlane(incl, 63);
    }
    // items per expert of width d = 1..4: ceil(nu / d), the thirds by a
    // multiply-shift (exact for any 32-bit nu)
    const int ipd[4] = {nu, (nu + 1) >> 1, (int)(((uint64_t)(uint32_t)(nu + 2) * 0xAAAAAAABull) >> 33), (nu + 3) >> 2};
    static_assert(P1_MAXNBW == 4, "items per expert are tabulated for widths 1..4");
    // the cap W (ties go to the wider cap); rounds by a float division,
    // exact below 2^24 items
    int W = 1;
    float best_cost = -1.f;
#pragma unroll
    for (int w = 1; w <= P1_MAXNBW; ++w) {
      int items = 0;
#pragma unroll
      for (int j = 0; j < 4; ++j) items += tot[j] * ipd[min(w, stream_max_nbw(j + 1)) - 1];
      const float cost = ceilf((float)items / (float)grid) * (float)(32 * w + 32);
      if (best_cost < 0.f || cost <= best_cost) {
        best_cost = cost;
        W = w;
      }
    }
    // classes ranked by decreasing item cost (ties: more row blocks first)
    int wd[4], ipe[4], key[4], rank_of[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      wd[j] = min(W, stream_max_nbw(j + 1));
      ipe[j] = ipd[wd[j] - 1];
      key[j] = wd[j] * (5 + j);
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      int r = 0;
#pragma unroll
      for (int i = 0; i < 4; ++i) r += key[i] > key[j] || (key[i] == key[j] && i > j);
      rank_of[j] = r;
    }
    int pos0[4], item0[4], total = 0;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      pos0[j] = 0;
      item0[j] = 0;
      total += tot[j] * ipe[j];
#pragma unroll
      for (int i = 0; i < 4; ++i)
        if (rank_of[i] < rank_of[j]) {
          pos0[j] += tot[i];
          item0[j] += tot[i] * ipe[i];
        }
    }
    int next[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) next[j] = pos0[j] + pre[j];
    for (int k = 0; k < per; ++k) {
      const int e = i0 + k;
      if (e < E) {
        const int rows = s_off[e + 1] - s_off[e];
        if (rows > 0 && rows <= S_MAX) {
          const int c = (rows - 1) >> 4;
          int pos = 0;
#pragma unroll
          for (int j = 0; j < 4; ++j)
            if (j == c) pos = next[j]++;
          s_eord[pos] = e;
        }
      }
    }
#pragma unroll
    for (int j = 0; j < 4; ++j)
      if (lane == rank_of[j]) {
        s_rrc[lane][0] = item0[j];
        s_rrc[lane][1] = pos0[j];
        s_rrc[lane][2] = tot[j] > 0 ? ipe[j] : 0;
        s_rrc[lane][3] = wd[j];
      }
    if (lane == 0) s_rrc[4][0] = total;
  }
  __syncthreads();
}

// Work split of the streaming phase when every streaming tile has the same
// row blocks and there are at least two units per workgroup: the contiguous
// range [*u0, *u1) of the
// U = tiles * nu units of 64 columns (unit u = column block u % nu of
// streaming m-tile u / nu) that workgroup b of `grid` streams.  Every expert
// tile's units cost the same weight bytes whatever its rows, so
//   tiles < grid:  tile t gets workgroups [t*grid/tiles, (t+1)*grid/tiles)
//                  (21 or 22 each at 12 tiles on 256 CUs) and splits its nu
//                  units evenly among them: no range spans two experts;
//   tiles >= grid: workgroup b gets units [U*b/grid, U*(b+1)/grid).
// A range is run as items of at most P1_RANGE_MAXNBW units that never span two
// experts.  Against dealing fixed 192-column items round-robin this lowers
// the largest share (E=12, 64 routed rows, N=6144: 5 units instead of 6).
__device__ __forceinline__ void stream_range(int tiles, int nu, int b, int grid, long long* u0, long long* u1) {
  if (tiles < grid) {
    const int t = (int)(((long long)(b + 1) * tiles - 1) / grid);
    const int s0 = (int)((long long)t * grid / tiles);
    const int k = (int)((long long)(t + 1) * grid / tiles) - s0;  // >= 1 since grid > tiles
    const int j = b - s0;
    *u0 = (long long)t * nu + (long long)j * nu / k;
    *u1 = (long long)t * nu + (long long)(j + 1) * nu / k;
  } else {
    const long long U = (long long)tiles * nu;
    *u0 = U * b / grid;
    *u1 = U * (b + 1) / grid;
  }
}


}  // namespace w4a8
