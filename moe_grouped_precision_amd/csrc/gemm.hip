// Grouped-contiguous W4A8 GEMM kernel for gfx950.
//
// C[r, n] = bf16( sum_g SA(r, g) * P_g[r, n] ),
// P_g[r, n] = sum_{k in group g} e4m3(A[r, k]) * e2m1(B[e, n, k]) * 2^(SB[e, n, k/32] - 127)
// (humming PR #129, "Results" command: FP8 E4M3 activations with fp32 scales
// per 128 K, MXFP4 weights with E8M0 scales per 32 K, bf16 output.)
//
// The fused variant (grouped_gemm_kernel<true>) is the gate/up projection
// with SwiGLU and the E4M3 requantization for the down projection in its
// epilogue (swiglu.h): it writes A2 [R][I] codes and their scales instead of
// the bf16 C.
//
// One persistent launch of 512 threads (8 waves) per CU.  Every workgroup
// first runs the plan prologue (offsets into LDS, validity check, per-expert
// tile counts of both classes), then the two phases over the tile plan:
//   1. streaming items, experts with <= S_MAX rows (stream_phase.h);
//   2. MFMA tiles, experts with more rows (mfma_phase.h).
// A workgroup that runs out of streaming items goes straight on to MFMA
// tiles, so one launch serves any mix of expert sizes.
#include "mfma_phase.h"
#include "stream_phase.h"

namespace w4a8 {

constexpr int BLOCK = 512;
static_assert(BLOCK == MF_THREADS, "both phases run on the same workgroup");
constexpr int LDS_BYTES = P1_BYTES > P2_BYTES ? P1_BYTES : P2_BYTES;

// FUSED: the gate/up GEMM with the SwiGLU + E4M3 requantization epilogue
// (weights [E][2I][K/2], gate columns first); every expert with rows runs as
// MFMA tiles of 256 output columns (the epilogue needs a row's 128-column
// group inside one workgroup), so the streaming phase has no work.
template <bool FUSED>
__global__ void __launch_bounds__(BLOCK, 1)
grouped_gemm_kernel(GemmArgs p) {
  __shared__ __attribute__((aligned(16))) uint8_t lds[LDS_BYTES];
  __shared__ int s_off[MAX_EXPERTS + 1];
  __shared__ int s_sbase[MAX_EXPERTS + 1];
  __shared__ int s_mbase[MAX_EXPERTS + 1];
  __shared__ int s_info[3];
  __shared__ int s_eord[MAX_EXPERTS];
  __shared__ int s_rrc[5][4];
  constexpr int smax = FUSED ? 0 : S_MAX;
  bool have_plan = false;

  // phase 1: streaming items.  The workgroup's items come either from one
  // block range of one expert (split into ceil(range / cap) items) or from
  // the round-robin dealing; one call site runs them all, so each item shape
  // is compiled once.
  if constexpr (!FUSED) {
    int mode = 0;                          // 1: block range, 2: round robin
    bool need_mfma = true;
    int e = 0, row0 = 0, rows = 0, b0 = 0, b1 = 0, R = 0, items = 0;
    if (p.E < 64 && (int)gridDim.x >= 64 && (int)gridDim.x < 4096) {
      // small pools: every wave finds the workgroup's expert and blocks in
      // registers; the plan tables of the MFMA phase are built afterwards
      const StreamAssign a = stream_assign_small(p.offsets, p.E, p.N >> 4, blockIdx.x, gridDim.x);
      if (!a.valid) return;
      if (a.tiles > 0) {
        mode = 1;
        e = uniform(a.e); row0 = uniform(a.row0); rows = uniform(a.rows);
        b0 = uniform(a.b0); b1 = uniform(a.b1); R = uniform(a.R);
      }
      need_mfma = a.any_mfma;
    } else {
      if (!plan_prologue(p.offsets, p.E, s_off, s_sbase, s_mbase, s_info, smax)) return;
      have_plan = true;
      need_mfma = uniform(s_mbase[p.E]) > 0;
      R = uniform(s_off[p.E]);
      const int tiles = uniform(s_sbase[p.E]);
      if (tiles > 0 && tiles <= (int)gridDim.x && (int)gridDim.x < ST_EXP) {
        // one expert per workgroup: its share of that expert's 16-column
        // blocks, as few items as the register budget allows
        stream_alloc(s_off, s_sbase, p.E, gridDim.x, s_eord);
        stream_expert_range(s_eord, tiles, p.N >> 4, blockIdx.x, gridDim.x, &e, &b0, &b1);
        row0 = uniform(s_off[e]);
        rows = uniform(s_off[e + 1]) - row0;
        mode = 1;
      } else if (tiles > 0) {
        // more experts than workgroups: items of 128-column units dealt
        // round-robin in a snake order of decreasing cost, each expert's
        // items as wide as its row blocks allow up to the cap the plan picks
        stream_rr_plan(s_off, p.E, (p.N + 127) / 128, gridDim.x, s_eord, s_rrc);
        items = uniform(s_rrc[4][0]);
        mode = 2;
      }
    }
    // block range: ceil(range / cap) items of nearly equal width (cap 32
    // blocks, 24 with four row blocks)
    static_assert(stream_max_nbw(3) == 4 && stream_max_nbw(4) == 3, "items of 32 or 24 blocks");
    const uint32_t n = (uint32_t)(b1 - b0);
    const uint32_t ni = mode != 1 ? 0 : (rows + 15) >> 4 <= 3 ? (n + 31) >> 5 : (n + 23) / 24;
    const int G = gridDim.x;
    for (int r = 0; mode != 0; ++r) {
      int n0, nb;
      if (mode == 1) {
        if ((uint32_t)r >= ni) break;
        const int c0 = b0 + (int)(n * r / ni), c1 = b0 + (int)(n * (r + 1) / ni);
        n0 = c0 * 16;
        nb = c1 - c0;
      } else {
        const int it = r * G + ((r & 1) ? G - 1 - (int)blockIdx.x : (int)blockIdx.x);
        if (it >= items) break;  // item numbers never decrease from one round to the next
        int k = 0;
        while (k < 3 && it >= uniform(s_rrc[k + 1][0])) ++k;
        const int rel = it - uniform(s_rrc[k][0]);
        const int ipe = uniform(s_rrc[k][2]), w = uniform(s_rrc[k][3]);
        const int q = rel / ipe;
        e = uniform(s_eord[uniform(s_rrc[k][1]) + q]);
        row0 = uniform(s_off[e]);
        rows = uniform(s_off[e + 1]) - row0;
        const int c0 = (rel - q * ipe) * w;
        n0 = c0 * 128;
        nb = min(8 * w, (p.N >> 4) - 8 * c0);
      }
      stream_item(p, lds, uniform(e), uniform(row0), uniform(rows), uniform(n0), uniform(nb), uniform(R));
    }
    if (!need_mfma) return;
  }
  if (!have_plan && !plan_prologue(p.offsets, p.E, s_off, s_sbase, s_mbase, s_info, smax)) return;
  const int R = uniform(s_off[p.E]);

  // phase 2: MFMA tiles, one workgroup each; each tile issues the first
  // shared-operand loads of the workgroup's next tile before its epilogue
  {
    // MT <= R / 65 + E and NT <= 2^31 / 512 keep the item count in 32 bits
    const int MT = uniform(s_mbase[p.E]);
    constexpr int TILE_N = FUSED ? MF_BN / 2 : MF_BN;   // output columns per tile
    const int NT = FUSED ? (p.I + TILE_N - 1) / TILE_N : (p.N + MF_BN - 1) / MF_BN;
    const int items = MT * NT;
    const int grid = gridDim.x;
    // this workgroup's round-r tile; invalid past its last one (item numbers
    // grow with r)
    auto tile_of = [&](int r) -> TileCoord {
      TileCoord t{0, 0, 0, 0, false};
      const int L = xcd_item(r, blockIdx.x, grid);
      if (L >= items) return t;
      int mt, nt;
      item_tile(L, MT, NT, &mt, &nt);
      t.e = uniform(expert_of_tile(s_mbase, p.E, mt));
      const int j = mt - uniform(s_mbase[t.e]);
      const int base = uniform(s_off[t.e]);
      const int rows_e = uniform(s_off[t.e + 1]) - base;
      const TileChoice tc = tile_rule(rows_e, smax);
      t.row0 = base + j * tc.tile_m;
      t.rows = min(tc.tile_m, rows_e - j * tc.tile_m);
      t.n0 = nt * TILE_N;
      t.valid = true;
      return t;
    };
    TileCoord t = tile_of(0);
    for (int r = 0; t.valid; ++r) t = mfma_tile<FUSED>(p, lds, t, R, r > 0, [&]() { return tile_of(r + 1); });
  }
}

// The grouped GEMM driven by a tile list built beforehand (w4a8_plan's
// format: header, then {expert, first row, rows, tile_m | class << 16} per
// m-tile, streaming tiles first): no per-expert tables in LDS, so the
// number of experts is bounded only by the plan (the shared expert pools of
// thousands of experts of MoonEP PR #38, background section), and any rule
// that respects the two phases' limits can be run (a streaming tile holds at
// most S_MAX rows, an MFMA tile at most T_MAX).  Every tile is checked
// against the offsets before use -- its rows inside its expert's rows and
// inside [0, R) -- and skipped otherwise, so no plan can make the kernel
// touch rows outside A, a_scales and C.  A plan whose status word is not 0
// makes the kernel write nothing.
__device__ __forceinline__ bool planned_tile(const GemmArgs& p, int R, int idx, int cls, int max_rows, int* e,
                                             int* row0, int* rows) {
  const int32_t* t = p.plan + PLAN_HEADER_WORDS + (size_t)idx * PLAN_TILE_WORDS;
  *e = uniform(t[0]);
  *row0 = uniform(t[1]);
  *rows = uniform(t[2]);
  const int tc = uniform(t[3]);
  if ((tc >> 16) != cls || *e < 0 || *e >= p.E || *rows < 1 || *rows > max_rows) return false;
  const int lo = uniform(p.offsets[*e]), hi = uniform(p.offsets[*e + 1]);
  return *row0 >= lo && *row0 >= 0 && (long long)*row0 + *rows <= hi && (long long)*row0 + *rows <= R;
}

__global__ void __launch_bounds__(BLOCK, 1)
grouped_gemm_planned_kernel(GemmArgs p) {
  __shared__ __attribute__((aligned(16))) uint8_t lds[LDS_BYTES];
  const int R = uniform(p.offsets[p.E]);
  if (uniform(p.plan[0]) != PLAN_OK || uniform(p.offsets[0]) != 0) return;
  const int ns = max(0, min(uniform(p.plan[2]), p.max_tiles));
  const int nm = max(0, min(uniform(p.plan[3]), p.max_tiles - ns));
  const int G = gridDim.x;

  // phase 1: streaming tiles, items of up to P1_MAXNB blocks of 16 columns
  // dealt round-robin in a snake order
  {
    const int NB = p.N >> 4;
    const int ipt = (NB + P1_MAXNB - 1) / P1_MAXNB;
    const long long items = (long long)ns * ipt;
    for (long long r = 0;; ++r) {
      const long long it = r * G + ((r & 1) ? G - 1 - (int)blockIdx.x : (int)blockIdx.x);
      if (it >= items) break;
      const int t = (int)(it / ipt), c = (int)(it - (long long)t * ipt);
      int e, row0, rows;
      if (!planned_tile(p, R, t, CLASS_STREAM, S_MAX, &e, &row0, &rows)) continue;
      // as one or two items, as the tile's row blocks allow
      const int b0 = c * P1_MAXNB, nb = min(P1_MAXNB, NB - b0);
      const int cap = 8 * stream_max_nbw((rows + 15) >> 4);
      const int ni = (nb + cap - 1) / cap;
      for (int k = 0; k < ni; ++k) {
        const int c0 = b0 + nb * k / ni, c1 = b0 + nb * (k + 1) / ni;
        stream_item(p, lds, e, row0, rows, c0 * 16, c1 - c0, R);
      }
    }
  }

  // phase 2: MFMA tiles, dealt as in grouped_gemm_kernel; tiles that fail
  // the check are passed over
  {
    const int NT = (p.N + MF_BN - 1) / MF_BN;
    const int items = nm * NT;  // nm <= R / 65 + E keeps it in 32 bits
    int r = 0;
    auto next_tile = [&]() -> TileCoord {
      for (;; ++r) {
        TileCoord t{0, 0, 0, 0, false};
        const int L = xcd_item(r, blockIdx.x, G);
        if (L >= items) return t;
        int mt, nt;
        item_tile(L, nm, NT, &mt, &nt);
        if (planned_tile(p, R, ns + mt, CLASS_MFMA, T_MAX, &t.e, &t.row0, &t.rows)) {
          t.n0 = nt * MF_BN;
          t.valid = true;
          ++r;
          return t;
        }
      }
    };
    TileCoord t = next_tile();
    for (bool ready = false; t.valid; ready = true) t = mfma_tile<false>(p, lds, t, R, ready, next_tile);
  }
}

hipError_t launch_grouped_gemm_planned(const GemmArgs& args, int grid, hipStream_t stream) {
  hipLaunchKernelGGL(grouped_gemm_planned_kernel, dim3(grid), dim3(BLOCK), 0, stream, args);
  return hipGetLastError();
}

hipError_t launch_grouped_gemm(const GemmArgs& args, int grid, hipStream_t stream) {
  hipLaunchKernelGGL(grouped_gemm_kernel<false>, dim3(grid), dim3(BLOCK), 0, stream, args);
  return hipGetLastError();
}

hipError_t launch_grouped_gemm_swiglu(const GemmArgs& args, int grid, hipStream_t stream) {
  hipLaunchKernelGGL(grouped_gemm_kernel<true>, dim3(grid), dim3(BLOCK), 0, stream, args);
  return hipGetLastError();
}

hipError_t grouped_gemm_occupancy(int* blocks) {
  return hipOccupancyMaxActiveBlocksPerMultiprocessor(blocks, grouped_gemm_kernel<false>, BLOCK, 0);
}

}  // namespace w4a8
