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

// B workgroups of W waves; workgroup b owns the contiguous slots
// [b*chunk, (b+1)*chunk) and writes their rows.  Every workgroup histograms
// all n ids (the slots before its chunk, its own chunk per wave, the slots
// after it), so it knows each expert's offset and how many of the expert's
// slots precede its chunk without any exchange between workgroups; workgroup
// 0 also writes counts and offsets.  Reading all ids in every workgroup costs
// L2 bandwidth only (the ids of a 16384-token batch are 512 KB), and the
// result does not depend on the number of workgroups.
// Dynamic LDS: own[W*E] + bef[W*E] + aft[W*E] + s_tot[E] + s_wave[16].
__global__ void __launch_bounds__(1024)
route_prep_kernel(const int32_t* __restrict__ ids, int n, int E, int nbits, int chunk,
                  int32_t* __restrict__ counts, int32_t* __restrict__ offsets,
                  int32_t* __restrict__ row_of_slot) {
  extern __shared__ int smem[];
  const int W = blockDim.x >> 6;
  int* own = smem;                // [W][E]: chunk counts per wave, then running row per (wave, expert)
  int* bef = smem + W * E;        // [W][E]: ids before the chunk
  int* aft = bef + W * E;         // [W][E]: ids after the chunk
  int* s_tot = aft + W * E;       // [E]
  int* s_wave = s_tot + E;        // [16]
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;

  for (int i = tid; i < 3 * W * E; i += blockDim.x) smem[i] = 0;
  __syncthreads();

  const int cbegin = min(n, (int)blockIdx.x * chunk);
  const int cend = min(n, cbegin + chunk);
  // each wave owns one contiguous span of the chunk, a multiple of 64 long
  const int span = (((cend - cbegin + W - 1) / W) + 63) & ~63;
  const int begin = min(cend, cbegin + wave * span);
  const int end = min(cend, begin + span);

  // phase 1: histograms (the order of the LDS atomics does not matter)
  for (int i = tid; i < cbegin; i += blockDim.x) {
    const int id = ids[i];
    if (id >= 0 && id < E) atomicAdd(&bef[wave * E + id], 1);
  }
  for (int i = cend + tid; i < n; i += blockDim.x) {
    const int id = ids[i];
    if (id >= 0 && id < E) atomicAdd(&aft[wave * E + id], 1);
  }
  for (int i = begin + lane; i < end; i += 64) {
    const int id = ids[i];
    if (id >= 0 && id < E) atomicAdd(&own[wave * E + id], 1);
  }
  __syncthreads();

  // phase 2: per expert the slots before the chunk, the prefix of the chunk's
  // waves, the total; exclusive scan of the totals over experts
  const int per = (E + blockDim.x - 1) / blockDim.x;
  const int e0 = tid * per;
  int local = 0;
  for (int j = 0; j < per; ++j) {
    const int e = e0 + j;
    if (e < E) {
      int before = 0, after = 0;
      for (int w = 0; w < W; ++w) {
        before += bef[w * E + e];
        after += aft[w * E + e];
      }
      int run = before;
      for (int w = 0; w < W; ++w) {
        const int c = own[w * E + e];
        own[w * E + e] = run;
        run += c;
      }
      const int tot = run + after;
      s_tot[e] = tot;
      if (blockIdx.x == 0) counts[e] = tot;
      local += tot;
    }
  }
  int total;
  int ex = block_exclusive_scan(local, s_wave, &total);
  for (int j = 0; j < per; ++j) {
    const int e = e0 + j;
    if (e < E) {
      if (blockIdx.x == 0) offsets[e] = ex;
      for (int w = 0; w < W; ++w) own[w * E + e] += ex;
      ex += s_tot[e];
    }
  }
  if (tid == 0 && blockIdx.x == 0) offsets[E] = total;
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
    if (valid) row = own[wave * E + id] + __popcll(m & below);
    __builtin_amdgcn_wave_barrier();
    if (valid && lane == 63 - __clzll(m)) own[wave * E + id] += __popcll(m);
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
  // three [W][E] histograms in at most 48 KB of LDS
  int W = 4096 / E;
  if (W > 16) W = 16;
  if (W < 1) W = 1;
  int nbits = 0;
  while ((1 << nbits) < E) ++nbits;
  // chunks of at least 2048 slots (a multiple of 64), at most 256 workgroups
  constexpr int kMinChunk = 2048, kMaxBlocks = 256;
  int chunk = kMinChunk;
  if ((n + chunk - 1) / chunk > kMaxBlocks) chunk = ((n + kMaxBlocks - 1) / kMaxBlocks + 63) & ~63;
  const int blocks = n > 0 ? (n + chunk - 1) / chunk : 1;
  size_t lds = (size_t)(3 * W * E + E + 16) * sizeof(int);
  hipLaunchKernelGGL(route_prep_kernel, dim3(blocks), dim3(W * 64), lds, stream, ids, n, E, nbits, chunk,
                     counts, offsets, row_of_slot);
  return hipGetLastError();
}

hipError_t launch_plan(const int32_t* offsets, int E, int N, int32_t* plan, int max_tiles,
                       hipStream_t stream) {
  hipLaunchKernelGGL(plan_kernel, dim3(1), dim3(256), 0, stream, offsets, E, N, plan, max_tiles);
  return hipGetLastError();
}

}  // namespace w4a8
