// Routing prep (histogram, exclusive-scan offsets, stable row map) and the
// device-side tile plan.  gfx950 only.
//
// The routing prep is the grouping step that produces the contiguous rows the
// grouped GEMM consumes (humming PR #129, "--gemm_type grouped_contiguous").
// Its structure -- per-wave expert histograms in LDS, a prefix over waves and
// experts, then ranks -- follows the MoE planning kernel of MoonEP PR #38
// (background section: per-warp histograms and length-E prefix arrays in
// shared memory), re-laid for 64-wide waves.  Ranks inside an expert come
// from wave ballots in flat slot order, never from atomic order, so the row
// map is unique (MoonEP PR #38, correctness section, requires exact equality
// with an independent reference).
#include "w4a8_device.h"
#include "w4a8_launch.h"

namespace w4a8 {

// One workgroup of W waves.  Dynamic LDS: hist[W*E] + s_tot[E] + s_wave[16].
__global__ void __launch_bounds__(1024)
route_prep_kernel(const int32_t* __restrict__ ids, int n, int E, int nbits,
                  int32_t* __restrict__ counts, int32_t* __restrict__ offsets,
                  int32_t* __restrict__ row_of_slot) {
  extern __shared__ int smem[];
  const int W = blockDim.x >> 6;
  int* hist = smem;               // [W][E]: counts, then running row per (wave, expert)
  int* s_tot = smem + W * E;      // [E]
  int* s_wave = s_tot + E;        // [16]
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;

  for (int i = tid; i < W * E; i += blockDim.x) hist[i] = 0;
  __syncthreads();

  // each wave owns one contiguous span of flat slots, a multiple of 64 long
  const int span = (((n + W - 1) / W) + 63) & ~63;
  const int begin = min(n, wave * span);
  const int end = min(n, begin + span);

  // phase 1: per-wave histograms (order of the LDS atomics does not matter)
  for (int i = begin + lane; i < end; i += 64) {
    int id = ids[i];
    if (id >= 0 && id < E) atomicAdd(&hist[wave * E + id], 1);
  }
  __syncthreads();

  // phase 2: prefix over waves per expert, totals, exclusive scan over experts
  const int per = (E + blockDim.x - 1) / blockDim.x;
  const int e0 = tid * per;
  int local = 0;
  for (int j = 0; j < per; ++j) {
    int e = e0 + j;
    if (e < E) {
      int run = 0;
      for (int w = 0; w < W; ++w) {
        int c = hist[w * E + e];
        hist[w * E + e] = run;
        run += c;
      }
      s_tot[e] = run;
      counts[e] = run;
      local += run;
    }
  }
  int total;
  int ex = block_exclusive_scan(local, s_wave, &total);
  for (int j = 0; j < per; ++j) {
    int e = e0 + j;
    if (e < E) {
      offsets[e] = ex;
      for (int w = 0; w < W; ++w) hist[w * E + e] += ex;
      ex += s_tot[e];
    }
  }
  if (tid == 0) offsets[E] = total;
  __syncthreads();

  // phase 3: stable ranks.  Lanes holding the same expert find each other with
  // one ballot per id bit; rank = number of such lanes below this one.
  const uint64_t below = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  for (int i0 = begin; i0 < end; i0 += 64) {
    const int i = i0 + lane;
    const int id = (i < end) ? ids[i] : -1;
    const bool valid = id >= 0 && id < E;
    uint64_t m = __ballot(valid);
    for (int b = 0; b < nbits; ++b) {
      const bool bit = valid && ((id >> b) & 1);
      uint64_t bb = __ballot(bit);
      m &= bit ? bb : ~bb;
    }
    int row = -1;
    if (valid) row = hist[wave * E + id] + __popcll(m & below);
    __builtin_amdgcn_wave_barrier();
    if (valid && lane == 63 - __clzll(m)) hist[wave * E + id] += __popcll(m);
    __builtin_amdgcn_wave_barrier();
    if (i < end) row_of_slot[i] = row;
  }
}

// One workgroup; writes the plan header and the tile list.
__global__ void __launch_bounds__(256)
plan_kernel(const int32_t* __restrict__ offsets, int E, int N, int32_t* __restrict__ plan,
            int max_tiles) {
  __shared__ int s_off[MAX_EXPERTS + 1];
  __shared__ int s_wave[16];
  const int tid = threadIdx.x;
  for (int i = tid; i <= E; i += blockDim.x) s_off[i] = offsets[i];
  __syncthreads();
  int bad = 0;
  for (int i = tid; i < E; i += blockDim.x) bad |= (s_off[i + 1] < s_off[i]);
  if (tid == 0) bad |= (s_off[0] != 0);
  bad = __syncthreads_or(bad);
  if (bad) {
    if (tid < PLAN_HEADER_WORDS) plan[tid] = tid == 0 ? PLAN_BAD_OFFSETS : 0;
    return;
  }
  const int per = (E + blockDim.x - 1) / blockDim.x;
  const int e0 = tid * per;
  int ls = 0, lm = 0, lp = 0;
  for (int j = 0; j < per; ++j) {
    int e = e0 + j;
    if (e < E) {
      int rows = s_off[e + 1] - s_off[e];
      TileChoice t = tile_rule(rows);
      if (t.cls == CLASS_STREAM) ls += t.n_m;
      if (t.cls == CLASS_MFMA) lm += t.n_m;
      lp += t.n_m * t.tile_m - rows;
    }
  }
  int ns, nm, padded;
  int bs = block_exclusive_scan(ls, s_wave, &ns);
  int bm = block_exclusive_scan(lm, s_wave, &nm);
  block_exclusive_scan(lp, s_wave, &padded);
  const int total = ns + nm;
  if (tid == 0) {
    plan[0] = total > max_tiles ? PLAN_CAPACITY : PLAN_OK;
    plan[1] = total;
    plan[2] = ns;
    plan[3] = nm;
    plan[4] = ns * ((N + TN_STREAM - 1) / TN_STREAM);
    plan[5] = nm * ((N + TN_MFMA - 1) / TN_MFMA);
    plan[6] = padded;
    plan[7] = s_off[E];
  }
  int32_t* body = plan + PLAN_HEADER_WORDS;
  for (int j = 0; j < per; ++j) {
    int e = e0 + j;
    if (e >= E) break;
    int rows = s_off[e + 1] - s_off[e];
    TileChoice t = tile_rule(rows);
    if (t.cls == CLASS_NONE) continue;
    int first = t.cls == CLASS_STREAM ? bs : ns + bm;
    for (int i = 0; i < t.n_m; ++i) {
      int idx = first + i;
      if (idx < max_tiles) {
        int r0 = i * t.tile_m;
        body[idx * 4 + 0] = e;
        body[idx * 4 + 1] = s_off[e] + r0;
        body[idx * 4 + 2] = min(t.tile_m, rows - r0);
        body[idx * 4 + 3] = t.tile_m | (t.cls << 16);
      }
    }
    if (t.cls == CLASS_STREAM) bs += t.n_m; else bm += t.n_m;
  }
}

hipError_t launch_route_prep(const int32_t* ids, int n, int E, int32_t* counts,
                             int32_t* offsets, int32_t* row_of_slot, hipStream_t stream) {
  int W = 8192 / E;
  if (W > 16) W = 16;
  if (W < 1) W = 1;
  int nbits = 0;
  while ((1 << nbits) < E) ++nbits;
  size_t lds = (size_t)(W * E + E + 16) * sizeof(int);
  hipLaunchKernelGGL(route_prep_kernel, dim3(1), dim3(W * 64), lds, stream, ids, n, E, nbits,
                     counts, offsets, row_of_slot);
  return hipGetLastError();
}

hipError_t launch_plan(const int32_t* offsets, int E, int N, int32_t* plan, int max_tiles,
                       hipStream_t stream) {
  hipLaunchKernelGGL(plan_kernel, dim3(1), dim3(256), 0, stream, offsets, E, N, plan, max_tiles);
  return hipGetLastError();
}

}  // namespace w4a8
