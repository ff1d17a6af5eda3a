// Weight-streaming phase of the grouped W4A8 GEMM kernel (gemm.hip): the
// experts with at most S_MAX rows (decode-sized batches, where HBM bandwidth
// is the limit).  gfx950 only.
//
// An item is (expert, nb blocks of 16 weight columns, the whole K).  Its 8
// waves own distinct blocks (block 8j + w is wave w's j-th, so every wave has
// at most one block more than another) and each wave walks the whole K for
// them: no partial sums are exchanged, the accumulators go straight to bf16.
// Weights stream from HBM straight into MFMA operand registers through a
// per-wave ring of D stages (no LDS: no other wave needs them); the
// activation rows and the scales are shared by the workgroup and come
// through LDS with direct global->LDS loads (global_load_lds_dwordx4 /
// _dword), which hold no registers while in flight.  Every wave issues the
// same number of ring loads per stage (blocks past the item's end load with
// exec = 0), waits for the stage it needs with one explicit vmcnt and meets
// the others at one barrier per stage.  The depth D is two stages (four for
// whole-K items of at most two blocks per wave), so a workgroup keeps 8 waves
// x D stages x NBW blocks x 2 KB = 64-128 KB of weights in flight.
// The XOR swizzle that keeps fragment reads free of LDS bank conflicts is
// applied on the global-address side (a load lane always writes slot base +
// size * lane).  All loads use clamped addresses (padding rows and columns
// re-read a real one and are never stored), so no load is conditional on
// data.
#pragma once

#include "w4a8_kernel.h"

namespace w4a8 {

// groups of K per stage: a stage's weight loads cover one whole 128-byte
// line (two groups) per column, paired into the two groups' operands by DPP
constexpr int P1_KG = 2;
// blocks per wave: the accumulators (4 * NBW * MB), the weight ring
// (8 * D * NBW) and the paired operands (8 * NBW) share the register file
constexpr int P1_MAXNBW = 4;
__host__ __device__ constexpr int stream_max_nbw(int mb) { return mb <= 3 ? 4 : 3; }
// stages in flight: two for the shapes items take (three or four blocks per
// wave with the whole K, any width with the K split): a workgroup then keeps
// 96-128 KB of weights in flight, and deeper rings only queue more requests
// at HBM (three stages of three blocks measured slower than two, one stage
// far slower); four for narrower whole-K items
__host__ __device__ constexpr int stream_depth(int nbw, int ks) { return ks == 2 || nbw >= 3 ? 2 : 4; }
// scale chunks (SC groups each) in LDS at once: a chunk is loaded D stages
// ahead of its first use, while up to D * P1_KG / SC earlier chunks are live
__host__ __device__ constexpr int stream_nbuf(int nbw, int ks) {
  return (stream_depth(nbw, ks) * P1_KG + SC - 1) / SC + 1;
}
// activation ring slot: P1_KG groups x ks parts x 64 rows x 128 B; E8M0
// chunk: 8 * nbw blocks x 16 columns x SC words; activation-scale chunk:
// ks parts x 64 rows x SC words
__host__ __device__ constexpr int stream_lds_bytes(int nbw, int ks) {
  return (stream_depth(nbw, ks) + 1) * P1_KG * ks * 8192 +
         stream_nbuf(nbw, ks) * (128 * nbw * SC * 4 + ks * 64 * SC * 4);
}
__host__ __device__ constexpr int cmax(int a, int b) { return a > b ? a : b; }
constexpr int P1_BYTES = cmax(cmax(cmax(stream_lds_bytes(3, 1), stream_lds_bytes(4, 1)),
                                   cmax(stream_lds_bytes(1, 2), stream_lds_bytes(2, 2))),
                              cmax(stream_lds_bytes(3, 2), stream_lds_bytes(4, 2)));
// an item holds at most this many 16-column blocks
constexpr int P1_MAXNB = 8 * P1_MAXNBW;

// An item of the streaming phase.  KS = 1: the 8 waves own distinct blocks
// (block 8j + w is wave w's j-th) and walk the whole K.  KS = 2 (narrow
// items, at most 16 blocks): waves 0-3 take the first ceil(G/2) groups of K
// and waves 4-7 the rest, each half owning all the item's blocks (block 4j +
// (w & 3)), so a narrow item runs half as many stages with twice the blocks
// per wave; the halves are added in LDS (always half 0 + half 1) before the
// bf16 store.
template <int NBW, int MB, int KS>
struct StreamItem {
  static constexpr int KG = P1_KG;
  static constexpr int WPK = 8 / KS;                 // waves per K part
  static constexpr int D = stream_depth(NBW, KS);
  static constexpr int NX = D + 1;                   // activation ring slots
  static constexpr int NBUF = stream_nbuf(NBW, KS);  // scale chunk buffers
  static constexpr int WIDTH = 16 * WPK * NBW;       // columns per item, at most
  static constexpr int XSLOT = KG * KS * 8192;       // [group][part][64 rows][128 B]
  static constexpr int SBB = KS * WIDTH * SC * 4;    // E8M0 words of a chunk: [part][column][group]
  static constexpr int SAB = KS * 64 * SC * 4;       // activation scales of a chunk: [part][row][group]
  static constexpr int SB0 = NX * XSLOT;
  static constexpr int SA0 = SB0 + NBUF * SBB;
  static constexpr int NXL = KS * MB;                // activation loads per wave per stage
  static constexpr int PER = 2 * NBW + NXL;          // ring loads per wave per stage
  static_assert(KS == 1 || KS == 2, "K parts");
  static_assert(SA0 + NBUF * SAB <= P1_BYTES, "LDS layout");
  static_assert((D - 1) * PER < 64, "vmcnt range");
  static_assert(SC % KG == 0 && (NBUF - 1) * SC >= D * KG, "scale chunk reuse distance");
  static_assert(NBW <= stream_max_nbw(MB), "register budget");
  static_assert(SBB == KS * WIDTH * SC * 4 && KS * WIDTH <= 512, "one 16-byte E8M0 load per column covers a chunk");
  static_assert(SBB == 8 * NBW * 256, "NBW 4-byte E8M0 loads per wave cover a chunk");
  static_assert(4 * NBW * MB * 1024 * (KS - 1) <= SB0, "reduction scratch fits in the activation ring");

  // Activation rows of stage s: KG groups x KS parts x 16*MB rows x 128 B in
  // 8*NXL half-wave loads of 4 rows, NXL per wave.  xt = the item's first
  // row; xo = this lane's row offsets; xg / xs = each load's group (from the
  // part's first) and LDS offset; gbeg = the first group of each part.
  __device__ __forceinline__ static void issue_x(const uint8_t* xt, const uint32_t (&xo)[NXL], const int (&xg)[NXL],
                                                 const int (&xs)[NXL], uint8_t* slot, int G, int s, bool live) {
    const uint64_t mask = live_mask(live) & 0xffffffffull;  // lanes 0-31 load
#pragma unroll
    for (int i = 0; i < NXL; ++i) {
      const int g = min(s * KG + xg[i], G - 1);
      vm_dma16(xt + (size_t)g * 128, xo[i], lds_u32(slot + xs[i]), mask);
    }
  }

  // Scale chunk c (groups SC*c .. SC*c+SC-1 of each part) into buffer c % NBUF.
  // E8M0: a column's codes of SC consecutive groups are 16 contiguous bytes,
  // so one 16-byte load per column (lane idx = part * WIDTH + column; waves
  // past the KS * WIDTH columns issue none; columns past the item's last
  // real one re-read that one).  The load starts at chunk_start(c) clamped to
  // G - SC so that it stays inside the column, and the word of group g then
  // sits at g - load start (sb_shift).  With fewer than SC groups in all, one
  // 4-byte load per (column, group) instead, the groups past the last clamped
  // to it.  Activation scales: one 4-byte load per (part, row, group) on 4*KS
  // waves.
  __device__ __forceinline__ static void issue_scales(const GemmArgs& p, uint8_t* lds, int e, int row0, int rows,
                                                      int n0, int nlast, int gh, int c, int R) {
    const int lane = opaque_lane(), wave = uniform(threadIdx.x >> 6);
    const int K = p.K, N = p.N, G = K >> 7;
    const int buf = c % NBUF;
    if (G >= SC) {
      if (wave * 64 < KS * WIDTH) {
        const int idx = wave * 64 + lane;  // [part][col]
        const int h = idx / WIDTH, col = idx - h * WIDTH;
        const int n = min(n0 + col, nlast);
        const int g = min(h * gh + SC * c, G - SC);
        const uint32_t off = (uint32_t)(n - n0) * (uint32_t)(K >> 5) + (uint32_t)g * 4u;
        vm_dma16(p.SB + ((size_t)e * N + n0) * (size_t)(K >> 5), off,
                 lds_u32(lds + SB0 + buf * SBB + wave * 1024), live_mask(true));
      }
    } else {
#pragma unroll
      for (int i = 0; i < NBW; ++i) {
        const int idx = (wave * NBW + i) * 64 + lane;  // [part][col][gg]
        const int h = idx / (WIDTH * SC), rem = idx - h * (WIDTH * SC);
        const int col = rem >> 2, gg = rem & 3;
        const int n = min(n0 + col, nlast);
        const int g = min(h * gh + SC * c + gg, G - 1);
        vm_dma4(p.SB + ((size_t)e * N + n) * (size_t)(K >> 5) + (size_t)g * 4,
                lds_u32(lds + SB0 + buf * SBB + (wave * NBW + i) * 256));
      }
    }
    if (wave < 4 * KS) {
      const int idx = wave * 64 + lane;  // [part][row][gg]
      const int h = idx >> 8, r = (idx >> 2) & 63, gg = idx & 3;
      const size_t row = (size_t)row0 + min(r, rows - 1);
      const int g = min(h * gh + SC * c + gg, G - 1);
      vm_dma4(sa_ptr(p, row, g, G, R), lds_u32(lds + SA0 + buf * SAB + wave * 256));
    }
  }
  // Word of the E8M0 chunk holding group gl (index within the part) of the
  // part that starts at group gbase: gl % SC, plus the clamp of the load.
  __device__ __forceinline__ static int sb_word(int gl, int gbase, int G) {
    const int start = gbase + SC * (gl / SC);
    return gl % SC + (G >= SC ? max(0, start - (G - SC)) : 0);
  }

  // Weights of this wave for the stage whose groups are gfirst, gfirst + 1:
  // per block j, load w[h][j] covers columns 8h .. 8h+7 of the block with one
  // full 128-byte line (both groups) per column, lane 16q + i reading column
  // 8h + (i & 7), group gfirst + (i >> 3), bytes 16q .. 16q+15.  Whole lines
  // per request stream from HBM at the rate of contiguous reads; two 64-byte
  // requests per line (one per group) do not.  pair_operands() turns the two
  // loads into the MFMA operands of the two groups.  wt = the item's first
  // column; wo = this lane's column offsets; jmask[j] = exec of block j (0
  // past the item's end); the second group is clamped to the last one when G
  // is odd.
  __device__ __forceinline__ static void load_wh(int h, v4i (&w)[KG][NBW], const uint8_t* wt,
                                                 const uint32_t (&wo)[2][NBW], const uint64_t (&jmask)[NBW], int gfirst,
                                                 int G, bool live) {
    const uint64_t mask = live_mask(live);
    const uint32_t goff = (uint32_t)min(gfirst + ((threadIdx.x & 15) >> 3), G - 1) * 64u;
#pragma unroll
    for (int j = 0; j < NBW; ++j) vm_load16_nt(w[h][j], wt, wo[h][j] + goff, mask & jmask[j]);
  }
  __device__ __forceinline__ static void load_w(v4i (&w)[KG][NBW], const uint8_t* wt, const uint32_t (&wo)[2][NBW],
                                                const uint64_t (&jmask)[NBW], int gfirst, int G, bool live) {
    load_wh(0, w, wt, wo, jmask, gfirst, G, live);
    load_wh(1, w, wt, wo, jmask, gfirst, G, live);
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
  // stage issues its ring loads (those past the end with exec = 0), so
  // exactly D-1 later stages of PER loads each may still be in flight (scale
  // loads issued in between only make the wait stricter); the stage's
  // activation rows and its scale chunk were issued before its weights.
  // Then make the weights readable and meet the other waves.
  __device__ __forceinline__ static void stage_wait(v4i (&w)[KG][NBW]) {
    wait_vm<(D - 1) * PER>();
#pragma unroll
    for (int kg = 0; kg < KG; ++kg)
#pragma unroll
      for (int j = 0; j < NBW; ++j) tie(w[kg][j]);
    wg_barrier();
  }

  // The item (expert e, rows row0 .. row0+rows-1, blocks of columns n0 ..
  // n0 + 16*nb - 1); 1 <= nb <= WPK*NBW.
  __device__ __forceinline__ static void run(const GemmArgs& p, uint8_t* lds, int e, int row0, int rows, int n0,
                                             int nb, int R) {
    const int lane = opaque_lane(), wave = uniform(threadIdx.x >> 6);
    const int kh = KS == 1 ? 0 : uniform(wave / WPK), wn = KS == 1 ? wave : uniform(wave % WPK);
    const int q = lane >> 4, r16 = lane & 15;
    const int K = p.K, N = p.N, G = K >> 7;
    const int gh = (G + KS - 1) / KS;             // groups of part 0 (part 1 has G - gh)
    const int gcount = kh == 0 ? gh : G - gh;     // groups of this wave's part
    const int S = (gh + KG - 1) / KG;             // stages
    const int Sp = (S + D - 1) / D * D;           // padded to whole ring turns
    const int nlast = min(n0 + 16 * nb, N) - 1;

    const uint8_t* xt = p.A + (size_t)row0 * K;
    uint32_t xo[NXL];
    int xg[NXL], xs[NXL];
#pragma unroll
    for (int i = 0; i < NXL; ++i) {
      const int jx = wave * NXL + i;              // [group][part][quad]
      const int quad = jx % (4 * MB), rest = jx / (4 * MB);
      const int h = rest % KS, kg = rest / KS;
      xg[i] = uniform(h * gh + kg);
      xs[i] = uniform((kg * KS + h) * 8192 + quad * 512);
      const int r = quad * 4 + (lane >> 3);
      const int c = (lane & 7) ^ (r & 7);
      xo[i] = (uint32_t)min(r, rows - 1) * (uint32_t)K + c * 16;
    }
    const uint8_t* wt = p.B + ((size_t)e * N + n0) * (size_t)(K >> 1);
    uint32_t wo[2][NBW];
    uint64_t jmask[NBW];
#pragma unroll
    for (int j = 0; j < NBW; ++j) {
      const int blk = j * WPK + wn;
      jmask[j] = blk < nb ? ~0ull : 0ull;
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int n = min(n0 + blk * 16 + 8 * h + (r16 & 7), nlast);
        wo[h][j] = (uint32_t)(n - n0) * (uint32_t)(K >> 1) + q * 16;
      }
    }
    const int gbase = kh * gh;                    // first group of this wave's part

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

    // Every stage issues its ring loads (past the last stage with exec = 0
    // and addresses clamped in range), so each wait is the same constant; the
    // loop body is D whole stages and the stage count is padded to a multiple
    // of D, so no control-flow path skips a stage and then runs a later one.
#pragma unroll
    for (int s = 0; s < D; ++s) {
      if (s < S && (s * KG) % SC == 0) issue_scales(p, lds, e, row0, rows, n0, nlast, gh, s * KG / SC, R);
      issue_x(xt, xo, xg, xs, lds + s * XSLOT, G, min(s, S - 1), s < S);
      load_w(wr[s], wt, wo, jmask, gbase + min(s, S - 1) * KG, G, s < S);
    }

    auto stage = [&](int s, int u) __attribute__((always_inline)) {
      stage_wait(wr[u]);
      const int sn = s + D;
      if (sn < S && (sn * KG) % SC == 0) issue_scales(p, lds, e, row0, rows, n0, nlast, gh, sn * KG / SC, R);
      issue_x(xt, xo, xg, xs, lds + (sn % NX) * XSLOT, G, min(sn, S - 1), sn < S);
      const uint8_t* slot = lds + (s % NX) * XSLOT;
      v4i wop[KG][NBW];
#pragma unroll
      for (int j = 0; j < NBW; ++j) pair_operands(wr[u][0][j], wr[u][1][j], wop[0][j], wop[1][j]);
      // the ring slot is free once paired: its next loads go out in two
      // halves, each before one group's MFMAs, so D stages stay in flight
      // while this one computes and the issue is spread over the stage
#pragma unroll
      for (int kg = 0; kg < KG; ++kg) {
        load_wh(kg, wr[u], wt, wo, jmask, gbase + min(sn, S - 1) * KG, G, sn < S);
        const int gl = s * KG + kg;               // group index within this wave's part
        if (gl < gcount) {
          const int buf = (gl / SC) % NBUF, gg = gl % SC, sw = sb_word(gl, gbase, G);
          const uint8_t* sbb = lds + SB0 + buf * SBB + kh * (WIDTH * SC * 4);
          const uint8_t* sab = lds + SA0 + buf * SAB + kh * (64 * SC * 4);
          int sbv[NBW];
#pragma unroll
          for (int j = 0; j < NBW; ++j) {
            const int col = (j * WPK + wn) * 16 + r16;
            sbv[j] = (int)((lds32(sbb + (col * SC + sw) * 4) >> (8 * q)) & 0xffu);
          }
#pragma unroll
          for (int i = 0; i < MB; ++i) {
            const int m = i * 16 + r16;
            const uint8_t* xb = slot + (kg * KS + kh) * 8192 + m * 128;
            const v4i x0 = lds128(xb + ((q ^ (m & 7)) << 4));
            const v4i x1 = lds128(xb + (((q + 4) ^ (m & 7)) << 4));
            const float sa = ldsf(sab + (m * SC + gg) * 4);
#pragma unroll
            for (int j = 0; j < NBW; ++j)
              promote(acc[j][i], sa, mfma_group(wop[kg][j], x0, x1, sbv[j]));
          }
        }
      }
    };

    for (int s0 = 0; s0 < Sp; s0 += D) {
#pragma unroll
      for (int u = 0; u < D; ++u) stage(s0 + u, u);
    }
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

    if constexpr (KS == 2) {
      // add the halves through LDS (every wave is past its last ring read
      // after this barrier): one per-lane base, constant offsets per (block,
      // row block)
      wg_barrier();
      v4f* red = reinterpret_cast<v4f*>(lds) + wn * (NBW * MB * 64) + lane;
      if (kh == 1) {
#pragma unroll
        for (int j = 0; j < NBW; ++j)
#pragma unroll
          for (int i = 0; i < MB; ++i) red[(j * MB + i) * 64] = acc[j][i];
      }
      __syncthreads();
      if (kh == 0) {
#pragma unroll
        for (int j = 0; j < NBW; ++j)
#pragma unroll
          for (int i = 0; i < MB; ++i) acc[j][i] += red[(j * MB + i) * 64];
      }
    }
    if (kh == 0) {
#pragma unroll
      for (int i = 0; i < MB; ++i) {
        const int m = i * 16 + r16;
        if (m < rows) {
          uint16_t* crow = p.C + (size_t)(row0 + m) * N;
#pragma unroll
          for (int j = 0; j < NBW; ++j) {
            const int blk = j * WPK + wn;
            const int n = n0 + blk * 16 + q * 4;
            if (blk < nb && n < N) store_bf16x4(crow + n, acc[j][i]);
          }
        }
      }
    }
    // the next item's first loads overwrite ring slots and scale buffers
    // (and the reduction scratch) that slower waves may still be reading
    wg_barrier();
  }
};

template <int MB>
__device__ __forceinline__ void stream_item_mb(const GemmArgs& p, uint8_t* lds, int e, int row0, int rows, int n0,
                                               int nb, int R) {
  if (nb <= 4 * stream_max_nbw(MB) && nb <= 16) {
    switch ((nb + 3) >> 2) {
      case 1: StreamItem<1, MB, 2>::run(p, lds, e, row0, rows, n0, nb, R); break;
      case 2: StreamItem<2, MB, 2>::run(p, lds, e, row0, rows, n0, nb, R); break;
      case 3: StreamItem<3, MB, 2>::run(p, lds, e, row0, rows, n0, nb, R); break;
      default: if constexpr (stream_max_nbw(MB) >= 4) StreamItem<4, MB, 2>::run(p, lds, e, row0, rows, n0, nb, R); break;
    }
  } else if (nb <= 24) {
    StreamItem<3, MB, 1>::run(p, lds, e, row0, rows, n0, nb, R);
  } else {
    if constexpr (stream_max_nbw(MB) >= 4) StreamItem<4, MB, 1>::run(p, lds, e, row0, rows, n0, nb, R);
  }
}

// One streaming item: nb blocks of 16 columns from column n0, 1 <= nb <=
// 8 * stream_max_nbw(row blocks).  Items of up to 16 blocks (12 with four row
// blocks) split K between two halves of the workgroup.
__device__ __forceinline__ void stream_item(const GemmArgs& p, uint8_t* lds, int e, int row0, int rows, int n0,
                                            int nb, int R) {
  switch ((rows + 15) >> 4) {
    case 1: stream_item_mb<1>(p, lds, e, row0, rows, n0, nb, R); break;
    case 2: stream_item_mb<2>(p, lds, e, row0, rows, n0, nb, R); break;
    case 3: stream_item_mb<3>(p, lds, e, row0, rows, n0, nb, R); break;
    default: stream_item_mb<4>(p, lds, e, row0, rows, n0, nb, R); break;
  }
}

// Workgroup order that keeps neighbours on one XCD: consecutive workgroup
// numbers go to the eight XCDs in turn, so workgroups b, b + 8, b + 16, ...
// share an XCD (and its L2); numbering them consecutively gives the
// workgroups of one expert one XCD, whose L2 then fetches that expert's
// activation rows once.
__device__ __forceinline__ int xcd_rank(int b, int grid) {
  if ((grid & 7) != 0) return b;
  return (b & 7) * (grid >> 3) + (b >> 3);
}

// Work split when there are no more streaming experts than workgroups.
// Every block costs the same weight bytes, but a stage costs more than its
// bytes (the barrier, the loads issued after it, the MFMAs, more of them with
// more row blocks), so a block of an expert with more row blocks takes longer,
// and a workgroup should run its blocks as one item (at most 8 *
// stream_max_nbw(row blocks) blocks).  Per-block weights 16, 17, 22 and 25
// for 1-4 row blocks: per-stage timestamps on the decode gate/up workload
// read 2.6 us per stage of about 30 blocks with one or two row blocks, 2.85
// with three and 2.65 per stage of 24 blocks with four, and a sweep of the
// weights around those ratios (back-to-back launches) measured these fastest.  Streaming expert t (in tile order) gets one
// workgroup plus its weight's share of the other grid - tiles workgroups of
// the XCD-grouped order,
//   first(t) = t + floor(Wcum(t) * (grid - tiles) / Wtot),
// and splits its NB blocks evenly among them.  Wave 0 writes, for t <= tiles,
//   s_tab[t]             first(t) (first(tiles) = grid)
//   s_tab[ST_EXP + t]    expert of tile t
// so that a workgroup finds its tile with one compare per lane.  Every thread
// must call it; 32-bit arithmetic throughout (Wtot < 2^16, grid < 2^12).
constexpr int ST_EXP = 1024;
__device__ __forceinline__ int stream_block_weight(int rows) {
  const int mb = (rows + 15) >> 4;
  return mb == 1 ? 16 : mb == 2 ? 17 : mb == 3 ? 22 : 25;
}
__device__ __forceinline__ void stream_alloc(const int* s_off, const int* s_sbase, int E, int grid, int* s_tab) {
  if (threadIdx.x < 64) {
    const int lane = threadIdx.x;
    const int per = (E + 63) / 64;
    const int i0 = lane * per;
    int sum = 0;
    for (int k = 0; k < per; ++k) {
      const int e = i0 + k;
      if (e < E) {
        const int rows = s_off[e + 1] - s_off[e];
        if (rows > 0 && rows <= S_MAX) sum += stream_block_weight(rows);
      }
    }
    const int incl = wave_inclusive_sum(sum);
    const uint32_t wtot = (uint32_t)__builtin_amdgcn_readlane(incl, 63);
    const int tiles = s_sbase[E];
    const uint32_t spare = (uint32_t)(grid - tiles);
    uint32_t run = (uint32_t)(incl - sum);
    for (int k = 0; k < per; ++k) {
      const int e = i0 + k;
      if (e < E) {
        const int rows = s_off[e + 1] - s_off[e];
        if (rows > 0 && rows <= S_MAX) {
          const int t = s_sbase[e];
          s_tab[t] = t + (int)(run * spare / wtot);
          s_tab[ST_EXP + t] = e;
          run += (uint32_t)stream_block_weight(rows);
        }
      }
    }
    if (lane == 0) s_tab[tiles] = grid;
  }
  __syncthreads();
}

// Workgroup b's expert e and its block range [b0, b1) (see above).
__device__ __forceinline__ void stream_expert_range(const int* s_tab, int tiles, int NB, int b, int grid, int* e,
                                                    int* b0, int* b1) {
  const int v = xcd_rank(b, grid);
  const int lane = threadIdx.x & 63;
  int t = 0;
  for (int x0 = 0; x0 < tiles; x0 += 64) {
    const int x = x0 + lane;
    const uint64_t m = __ballot(x < tiles && s_tab[x] <= v && v < s_tab[x + 1]);
    if (m) t = x0 + (int)__builtin_ctzll(m);
  }
  t = uniform(t);
  *e = uniform(s_tab[ST_EXP + t]);
  const int s0 = uniform(s_tab[t]);
  const uint32_t k = (uint32_t)(uniform(s_tab[t + 1]) - s0);  // >= 1
  const uint32_t j = (uint32_t)(v - s0);
  *b0 = (int)((uint32_t)NB * j / k);
  *b1 = (int)((uint32_t)NB * (j + 1) / k);
}

// The same split for pools of fewer than 64 experts, computed by every wave
// in registers (lane e holds expert e; one scan per quantity, one ballot), so
// that a workgroup's first loads do not wait for LDS tables and barriers:
// the offsets are checked (offsets[0] = 0, nondecreasing), then the
// workgroup's streaming expert and block range are found as above, and
// whether any expert needs the MFMA phase.  grid must be at least 64 (so that
// tiles <= E < grid) and below 4096 (32-bit products).
struct StreamAssign {
  bool valid;      // offsets usable
  bool any_mfma;   // some expert has more than S_MAX rows
  int tiles;       // streaming experts
  int e, b0, b1;   // this workgroup's expert and blocks (tiles > 0)
  int row0, rows;  // that expert's rows
  int R;           // offsets[E]
};
__device__ __forceinline__ StreamAssign stream_assign_small(const int32_t* __restrict__ offsets, int E, int NB, int b,
                                                            int grid) {
  StreamAssign a;
  const int lane = threadIdx.x & 63;
  const int lo = lane <= E ? offsets[lane] : 0;
  const int hi = __shfl_down(lo, 1, 64);         // offsets[lane + 1] for lane < E
  const bool in = lane < E;
  const int rows = in ? hi - lo : 0;
  a.valid = __ballot((lane == 0 && lo != 0) || (in && rows < 0)) == 0;
  a.R = __builtin_amdgcn_readlane(lo, E);
  a.any_mfma = __ballot(in && rows > S_MAX) != 0;
  const bool st = in && rows > 0 && rows <= S_MAX;
  const int w = st ? stream_block_weight(rows) : 0;
  const int winc = wave_inclusive_sum(w);
  const int tinc = wave_inclusive_sum(st ? 1 : 0);
  const uint32_t wtot = (uint32_t)__builtin_amdgcn_readlane(winc, 63);
  a.tiles = __builtin_amdgcn_readlane(tinc, 63);
  a.e = a.b0 = a.b1 = a.row0 = a.rows = 0;
  if (!a.valid || a.tiles == 0) return a;
  const uint32_t spare = (uint32_t)(grid - a.tiles);
  // first workgroup of this lane's expert and of the next streaming expert
  const int f0 = tinc - (st ? 1 : 0) + (int)((uint32_t)(winc - w) * spare / wtot);
  const int f1 = tinc + (int)((uint32_t)winc * spare / wtot);
  const int v = xcd_rank(b, grid);
  const uint64_t m = __ballot(st && f0 <= v && v < f1);
  const int el = (int)__builtin_ctzll(m);       // exactly one lane holds v
  a.e = el;
  const int s0 = __builtin_amdgcn_readlane(f0, el);
  const uint32_t k = (uint32_t)(__builtin_amdgcn_readlane(f1, el) - s0);
  const uint32_t j = (uint32_t)(v - s0);
  a.b0 = (int)((uint32_t)NB * j / k);
  a.b1 = (int)((uint32_t)NB * (j + 1) / k);
  a.row0 = __builtin_amdgcn_readlane(lo, el);
  a.rows = __builtin_amdgcn_readlane(rows, el);
  return a;
}

// Items dealt round-robin (more streaming experts than workgroups).  A unit
// is 128 columns (8 blocks); expert e's items are w = min(W, stream_max_nbw
// of its row blocks) units wide, with the cap W that minimises rounds x
// per-item bytes, per-item bytes ~ weights (64 per unit per K) plus
// activation rows (up to 64 per K): wider items re-read the activation rows
// less often and pay the pipeline fill and drain fewer times, narrower ones
// spread few experts over more workgroups.  Items are numbered in decreasing
// order of their cost, w * (4 + row blocks), in four classes (the row
// blocks), and dealt in a snake order (round r gives workgroup b item r*G +
// b for even r, r*G + G-1-b for odd r), so that a workgroup's second item is
// light when its first was heavy.
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
      const float cost = ceilf((float)items / (float)grid) * (float)(64 * w + 64);
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

}  // namespace w4a8
