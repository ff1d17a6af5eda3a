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
// with an independent reference).  The LDS need grows with W * E, so the
// host picks the number of waves W to fit the device's per-workgroup LDS
// (MoonEP PR #38, change section: drop one wave at a time from the largest
// workgroup, report resource overflow when even one wave does not fit), which
// carries the prep to thousands of experts.
#include <algorithm>

#include "w4a8_device.h"
#include "w4a8_launch.h"

namespace w4a8 {

// B workgroups of up to ROUTE_MAX_WAVES waves; workgroup b owns the contiguous
// slots [b*chunk, (b+1)*chunk) and writes their rows.  The first wr waves
// rank (each one span of the chunk, with its own copy of the chunk's
// counts); all waves histogram and scan.  Every workgroup histograms
// all n ids (the slots before its chunk, its own chunk per wave, the slots
// after it), so it knows each expert's offset and how many of the expert's
// slots precede its chunk without any exchange between workgroups; workgroup
// 0 also writes counts and offsets.  Reading all ids in every workgroup costs
// L2 bandwidth only (the ids of a 16384-token batch are 512 KB), and the
// result does not depend on the number of workgroups or waves.
// Dynamic LDS: own[wr*E] + bef[E] + aft[E] + s_wave[16] ints
// (route_prep_lds_bytes); aft holds each expert's total once the counts are
// summed.  Only a ranking wave needs its own copy of the chunk's counts; one
// copy of the outside counts serves all waves, since LDS atomics serialize
// only on equal addresses within one instruction.  So the LDS bounds the
// number of ranking waves, never the workgroup's size.
__global__ void __launch_bounds__(ROUTE_MAX_WAVES * 64)
route_prep_kernel(const int32_t* __restrict__ ids, int n, int E, int nbits, int chunk, int wr,
                  int32_t* __restrict__ counts, int32_t* __restrict__ offsets,
                  int32_t* __restrict__ row_of_slot) {
  extern __shared__ int smem[];
  const int W = wr;               // ranking waves
  int* own = smem;                // [W][E]: chunk counts per ranking wave, then running row per (wave, expert)
  int* bef = smem + W * E;        // [E]: ids before the chunk
  int* aft = bef + E;             // [E]: ids after the chunk; then the totals
  int* s_wave = aft + E;          // [16]
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;

  const int cbegin = min(n, (int)blockIdx.x * chunk);
  const int cend = min(n, cbegin + chunk);
  // each ranking wave owns one contiguous span of the chunk, a multiple of
  // 64 long; the other waves own none
  const int span = (((cend - cbegin + W - 1) / W) + 63) & ~63;
  const int begin = wave < W ? min(cend, cbegin + wave * span) : cend;
  const int end = wave < W ? min(cend, begin + span) : cend;
  // the first 64 ids of the span, loaded before the LDS is cleared and kept
  // in a register for the ranks (a small batch is all first ids)
  const int id_first = begin + lane < end ? ids[begin + lane] : -1;

  for (int i = tid; i < (W + 2) * E; i += blockDim.x) smem[i] = 0;
  __syncthreads();

  // phase 1: histograms (the order of the LDS atomics does not matter).  The
  // ids outside the chunk are read 16 bytes per lane with ROUTE_LOADS loads in
  // flight (a workgroup of few waves would otherwise wait on one load at a
  // time) and counted by position; the chunk's own ids per wave span.
  auto count_outside = [&](unsigned i, int id) {
    if (id >= 0 && id < E && (i < (unsigned)cbegin || i >= (unsigned)cend))
      atomicAdd(&(i < (unsigned)cbegin ? bef : aft)[id], 1);
  };
  const int head = min(n, (int)((4 - ((reinterpret_cast<uintptr_t>(ids) >> 2) & 3)) & 3));
  if (tid < head) count_outside(tid, ids[tid]);
  const int nv = (n - head) >> 2;  // whole 16-byte units from ids + head
  const int4* vec = reinterpret_cast<const int4*>(ids + head);
  // units [0, ub) reach before the chunk, units [ua, nv) after it; the loop
  // runs over both ranges as one index space and skips the units inside
  const int ub = min(nv, cbegin > head ? (cbegin - head + 3) >> 2 : 0);
  const int ua = max(ub, min(nv, cend > head ? (cend - head) >> 2 : 0));
  const int nvis = ub + (nv - ua);
  auto unit = [&](int v) { return v < ub ? v : v - ub + ua; };
  for (int v0 = tid; v0 < nvis; v0 += ROUTE_LOADS * blockDim.x) {
    int4 q[ROUTE_LOADS];
#pragma unroll
    for (int j = 0; j < ROUTE_LOADS; ++j) {
      const int v = v0 + j * blockDim.x;
      q[j] = v < nvis ? vec[unit(v)] : make_int4(-1, -1, -1, -1);
    }
#pragma unroll
    for (int j = 0; j < ROUTE_LOADS; ++j) {
      const int v = v0 + j * blockDim.x;
      const unsigned i = (unsigned)head + 4u * (unsigned)(v < nvis ? unit(v) : 0);
      count_outside(i, q[j].x);
      count_outside(i + 1, q[j].y);
      count_outside(i + 2, q[j].z);
      count_outside(i + 3, q[j].w);
    }
  }
  for (int i = head + 4 * nv + tid; i < n; i += blockDim.x) count_outside(i, ids[i]);
  if (id_first >= 0 && id_first < E) atomicAdd(&own[wave * E + id_first], 1);
  for (int i = begin + 64 + lane; i < end; i += 64) {
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
      const int after = aft[e];
      int run = bef[e];
      for (int w = 0; w < W; ++w) {
        const int c = own[w * E + e];
        own[w * E + e] = run;
        run += c;
      }
      const int tot = run + after;
      aft[e] = tot;  // only this thread reads or writes column e
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
      ex += aft[e];
    }
  }
  if (tid == 0 && blockIdx.x == 0) offsets[E] = total;
  __syncthreads();

  // phase 3: stable ranks.  Lanes holding the same expert find each other with
  // one ballot per id bit; rank = number of such lanes below this one.
  const uint64_t below = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  for (int i0 = begin; i0 < end; i0 += 64) {
    const int i = i0 + lane;
    const int id = i0 == begin ? id_first : (i < end) ? ids[i] : -1;
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
  // offsets are read from global memory (a few reads per expert, cached), so
  // the plan has no LDS bound on E
  const int32_t* s_off = offsets;
  __shared__ int s_wave[16];
  const int tid = threadIdx.x;
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

size_t route_prep_lds_bytes(int E, int waves) {
  return ((size_t)(waves + 2) * E + 16) * sizeof(int);
}

int route_prep_waves(int E, size_t lds_limit) {
  for (int w = ROUTE_MAX_WAVES; w >= 1; --w)
    if (route_prep_lds_bytes(E, w) <= lds_limit) return w;
  return 0;
}

hipError_t launch_route_prep(const int32_t* ids, int n, int E, int W, int32_t* counts,
                             int32_t* offsets, int32_t* row_of_slot, hipStream_t stream) {
  int nbits = 0;
  while ((1 << nbits) < E) ++nbits;
  // chunks of at least 2048 slots (a multiple of 64), at most 256 workgroups
  constexpr int kMinChunk = 2048, kMaxBlocks = 256;
  int chunk = kMinChunk;
  if ((n + chunk - 1) / chunk > kMaxBlocks) chunk = ((n + kMaxBlocks - 1) / kMaxBlocks + 63) & ~63;
  const int blocks = n > 0 ? (n + chunk - 1) / chunk : 1;
  // a small batch: no more ranking waves than its 64-id spans (the per-expert
  // prefix over waves is serial in W), and no more waves in all than those
  // and one per 64 experts (phase 2's threads), so the workgroup's barriers
  // and scans are short; the row map does not depend on either
  W = std::min(W, std::max(1, (std::min(n, chunk) + 63) / 64));
  const int threads = 64 * std::max(W, std::min(ROUTE_MAX_WAVES, (E + 63) / 64));
  hipLaunchKernelGGL(route_prep_kernel, dim3(blocks), dim3(threads), route_prep_lds_bytes(E, W),
                     stream, ids, n, E, nbits, chunk, W, counts, offsets, row_of_slot);
  return hipGetLastError();
}

hipError_t launch_plan(const int32_t* offsets, int E, int N, int32_t* plan, int max_tiles,
                       hipStream_t stream) {
  hipLaunchKernelGGL(plan_kernel, dim3(1), dim3(256), 0, stream, offsets, E, N, plan, max_tiles);
  return hipGetLastError();
}

}  // namespace w4a8
