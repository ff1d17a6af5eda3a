// Device helpers shared by the two phases of the GEMM kernel of libw4a8
// (stream_phase.h, the weight-streaming class; mfma_phase.h, the MFMA-tile
// class): inline-asm vector
// memory operations with explicit waits, the scaled MFMA of one 128-K group,
// the per-128 promotion, bf16 stores and the LDS swizzle keys.  gfx950 only.
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
#pragma once

#include "w4a8_device.h"
#include "w4a8_launch.h"

namespace w4a8 {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef float v2f __attribute__((ext_vector_type(2)));

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

// Four fp32 -> bf16, round to nearest even, with gfx950's packed conversion
// (v_cvt_pk_bf16_f32: two values per instruction; denormals are kept, as
// the kernels run with fp32 denormals preserved; NaN stays NaN).
typedef __bf16 v2bf __attribute__((ext_vector_type(2)));
__device__ __forceinline__ void store_bf16x4(uint16_t* dst, v4f v) {
  const v2bf lo = __builtin_convertvector((v2f){v[0], v[1]}, v2bf);
  const v2bf hi = __builtin_convertvector((v2f){v[2], v[3]}, v2bf);
  uint2 o;
  o.x = __builtin_bit_cast(uint32_t, lo);
  o.y = __builtin_bit_cast(uint32_t, hi);
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

}  // namespace w4a8
