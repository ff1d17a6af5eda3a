// Device-side pieces shared by the prep, plan and GEMM kernels of libw4a8:
// the per-expert tile rule, block-wide scans, wave scans and the plan
// prologue that every GEMM workgroup runs.  gfx950 only.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace w4a8 {

// ---------------------------------------------------------------------------
// Tile rule.  The pages ask that each expert's M tile come from that expert's
// own row count (humming PR #129, commit 1 "Row-major tile model"): a fixed
// M128 tile gives experts routed slightly past a multiple of 128 an extra,
// mostly empty tile, while rows that fill tiles exactly must get full tiles
// (last note under that page's tables).  Small experts go to a separate
// small-M schedule below a cutoff (commit 2 "Small-expert seed tile").
// Constants are this library's own: GRAN is one MFMA block of rows, S_MAX the
// largest expert the weight-streaming phase serves (four MFMA blocks), T_MAX
// the MFMA phase's m-tile; TN_STREAM is the n granularity by which the plan
// counts streaming work (a workgroup item spans 1-8 of these), TN_MFMA the
// MFMA phase's n-tile.
// ---------------------------------------------------------------------------
constexpr int GRAN = 16;
constexpr int S_MAX = 64;
constexpr int T_MAX = 128;
constexpr int TN_STREAM = 64;
constexpr int TN_MFMA = 512;
constexpr int PLAN_HEADER_WORDS = 8;
constexpr int PLAN_TILE_WORDS = 4;

constexpr int CLASS_NONE = 0;
constexpr int CLASS_STREAM = 1;
constexpr int CLASS_MFMA = 2;

constexpr int PLAN_OK = 0;
constexpr int PLAN_BAD_OFFSETS = 1;
constexpr int PLAN_CAPACITY = 2;

// per-expert tables of the GEMM prologue live in LDS beside the staging
// buffers: 2048 experts keep the total under 160 KB
constexpr int MAX_EXPERTS = 2048;

struct TileChoice {
  int cls;
  int tile_m;
  int n_m;
};

// smax = S_MAX for the plain GEMM; the fused SwiGLU GEMM, whose epilogue
// lives in the MFMA phase only, passes 0 (every expert with rows is MFMA).
__host__ __device__ inline TileChoice tile_rule(int rows, int smax = S_MAX) {
  TileChoice t;
  if (rows <= 0) {
    t.cls = CLASS_NONE; t.tile_m = 0; t.n_m = 0;
  } else if (rows <= smax) {
    t.cls = CLASS_STREAM; t.tile_m = (rows + GRAN - 1) / GRAN * GRAN; t.n_m = 1;
  } else {
    t.cls = CLASS_MFMA;
    t.n_m = (rows + T_MAX - 1) / T_MAX;
    int per = (rows + t.n_m - 1) / t.n_m;
    t.tile_m = (per + GRAN - 1) / GRAN * GRAN;
  }
  return t;
}

// ---------------------------------------------------------------------------
// Block-wide exclusive scan of one int per thread (wave64 shuffles + LDS).
// `wave_tot` must hold blockDim.x/64 ints.  Returns the exclusive prefix and
// writes the block total to *total.  All threads of the block must call it.
// ---------------------------------------------------------------------------
__device__ inline int block_exclusive_scan(int v, int* wave_tot, int* total) {
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int nwaves = blockDim.x >> 6;
  int x = v;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    int y = __shfl_up(x, d, 64);
    if (lane >= d) x += y;
  }
  if (lane == 63) wave_tot[wave] = x;
  __syncthreads();
  if (wave == 0) {
    int t = lane < nwaves ? wave_tot[lane] : 0;
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
      int y = __shfl_up(t, d, 64);
      if (lane >= d) t += y;
    }
    if (lane < nwaves) wave_tot[lane] = t;  // inclusive wave totals
  }
  __syncthreads();
  int base = wave > 0 ? wave_tot[wave - 1] : 0;
  int tot = wave_tot[nwaves - 1];
  __syncthreads();
  *total = tot;
  return base + x - v;
}

// ---------------------------------------------------------------------------
// Inclusive sum / max over the 64 lanes of a wave: DPP row shifts inside each
// 16-lane row, then the row broadcasts of lane 15 and lane 31 across rows.
// Disabled lanes and lanes without a source read 0 (the `old` operand), which
// is neutral for sums and for maxima of non-negative values.
// ---------------------------------------------------------------------------
__device__ inline int wave_inclusive_sum(int x) {
  x += __builtin_amdgcn_update_dpp(0, x, 0x111, 0xf, 0xf, false);  // row_shr:1
  x += __builtin_amdgcn_update_dpp(0, x, 0x112, 0xf, 0xf, false);  // row_shr:2
  x += __builtin_amdgcn_update_dpp(0, x, 0x114, 0xf, 0xf, false);  // row_shr:4
  x += __builtin_amdgcn_update_dpp(0, x, 0x118, 0xf, 0xf, false);  // row_shr:8
  x += __builtin_amdgcn_update_dpp(0, x, 0x142, 0xa, 0xf, false);  // row_bcast:15 -> rows 1, 3
  x += __builtin_amdgcn_update_dpp(0, x, 0x143, 0xc, 0xf, false);  // row_bcast:31 -> rows 2, 3
  return x;
}
__device__ inline int wave_max_nonneg(int x) {
  x = max(x, __builtin_amdgcn_update_dpp(0, x, 0x111, 0xf, 0xf, false));
  x = max(x, __builtin_amdgcn_update_dpp(0, x, 0x112, 0xf, 0xf, false));
  x = max(x, __builtin_amdgcn_update_dpp(0, x, 0x114, 0xf, 0xf, false));
  x = max(x, __builtin_amdgcn_update_dpp(0, x, 0x118, 0xf, 0xf, false));
  x = max(x, __builtin_amdgcn_update_dpp(0, x, 0x142, 0xa, 0xf, false));
  x = max(x, __builtin_amdgcn_update_dpp(0, x, 0x143, 0xc, 0xf, false));
  return __builtin_amdgcn_readlane(x, 63);
}

// ---------------------------------------------------------------------------
// Plan prologue run by every GEMM workgroup: offsets into LDS, validity check,
// and the exclusive scans of the m-tile counts of both classes.  Wave 0 does
// the work (lane l owns a contiguous run of experts); the other waves wait at
// one barrier.
//   s_off[0..E]    expert offsets
//   s_sbase[0..E]  first streaming-class m-tile of each expert; [E] = total
//   s_mbase[0..E]  first MFMA-class m-tile of each expert;      [E] = total
//   s_info[0]      nonzero if the offsets are invalid
//   s_info[1]      row blocks (GRAN rows) of the largest streaming tile
//   s_info[2]      row blocks of the smallest streaming tile (0 if none)
// Returns false (uniformly across the block) if the offsets are invalid.
// ---------------------------------------------------------------------------
__device__ inline bool plan_prologue(const int32_t* __restrict__ offsets, int E, int* s_off,
                                     int* s_sbase, int* s_mbase, int* s_info, int smax = S_MAX) {
  if (threadIdx.x < 64) {
    const int lane = threadIdx.x;
    const int per = (E + 64) / 64;  // offsets per lane, so that 64 * per > E
    const int i0 = lane * per;
    int bad = 0, ls = 0, lm = 0, mb = 0, mbi = 0;  // mbi: S_MAX/GRAN - row blocks
    for (int k = 0; k < per; ++k) {
      const int e = i0 + k;
      if (e <= E) {
        const int a = offsets[e];
        s_off[e] = a;
        if (e == 0) bad |= a != 0;
        if (e < E) {
          const int b = offsets[e + 1];
          bad |= b < a;
          const TileChoice t = tile_rule(b - a, smax);
          if (t.cls == CLASS_STREAM) {
            ls += t.n_m;
            mb = max(mb, t.tile_m / GRAN);
            mbi = max(mbi, S_MAX / GRAN - t.tile_m / GRAN);
          }
          if (t.cls == CLASS_MFMA) lm += t.n_m;
        }
      }
    }
    const bool any_bad = __ballot(bad != 0) != 0;
    const int is = wave_inclusive_sum(ls), im = wave_inclusive_sum(lm);
    const int mbmax = wave_max_nonneg(mb);
    const int mbimax = wave_max_nonneg(mbi);
    if (!any_bad) {
      int rs = is - ls, rm = im - lm;
      for (int k = 0; k < per; ++k) {
        const int e = i0 + k;
        if (e < E) {
          s_sbase[e] = rs;
          s_mbase[e] = rm;
          const TileChoice t = tile_rule(s_off[e + 1] - s_off[e], smax);
          rs += t.cls == CLASS_STREAM ? t.n_m : 0;
          rm += t.cls == CLASS_MFMA ? t.n_m : 0;
        }
      }
    }
    if (lane == 0) {
      s_sbase[E] = __builtin_amdgcn_readlane(is, 63);
      s_mbase[E] = __builtin_amdgcn_readlane(im, 63);
      s_info[0] = any_bad;
      s_info[1] = mbmax;
      s_info[2] = mbmax > 0 ? S_MAX / GRAN - mbimax : 0;
    }
  }
  __syncthreads();
  return s_info[0] == 0;
}

// Expert owning class-local m-tile `mt`: the e with s_base[e] <= mt < s_base[e+1].
__device__ inline int expert_of_tile(const int* s_base, int E, int mt) {
  int lo = 0, hi = E;  // invariant: s_base[lo] <= mt < s_base[hi]
  while (hi - lo > 1) {
    int mid = (lo + hi) >> 1;
    if (s_base[mid] <= mt) lo = mid; else hi = mid;
  }
  return lo;
}

}  // namespace w4a8
