// Host-side launch interface between the C ABI layer (api.cpp) and the kernel
// translation units (prep.hip, gemm.hip).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace w4a8 {

struct GemmArgs {
  const uint8_t* A;        // [R][K] E4M3 codes
  const float* SA;         // per (row, 128-K group), layout below
  const uint8_t* B;        // [E][N][K/2] packed E2M1
  const uint8_t* SB;       // [E][N][K/32] E8M0
  const int32_t* offsets;  // [E+1]
  uint16_t* C;             // [R][N] bf16 bits (the plain GEMM)
  int E, N, K, layout;     // layout 0 row-major, 1 M-major
  // fused SwiGLU epilogue (N = 2 I weight columns: gate 0 .. I-1, up I .. 2I-1)
  uint8_t* A2;             // [R][I] E4M3 codes of silu(gate) * up
  float* SA2;              // per (row, 128 columns of A2), layout2
  int I, layout2;
  // planned GEMM: a tile list in w4a8_plan's format holding at most max_tiles tiles
  const int32_t* plan;
  int max_tiles;
};

// Route prep: the workgroup holds up to ROUTE_MAX_WAVES waves, W of which
// rank (1..ROUTE_MAX_WAVES), and route_prep_lds_bytes(E, W) bytes of LDS;
// route_prep_waves picks the largest W that fits lds_limit bytes, 0 if none
// does, and the launch lowers W (and the waves) for batches of few ids.
constexpr int ROUTE_MAX_WAVES = 16;
constexpr int ROUTE_LOADS = 16;  // 16-byte id loads in flight per lane
size_t route_prep_lds_bytes(int E, int waves);
int route_prep_waves(int E, size_t lds_limit);
hipError_t launch_route_prep(const int32_t* ids, int n, int E, int W, int32_t* counts, int32_t* offsets,
                             int32_t* row_of_slot, hipStream_t stream);
hipError_t launch_plan(const int32_t* offsets, int E, int N, int32_t* plan, int max_tiles,
                       hipStream_t stream);
hipError_t launch_grouped_gemm(const GemmArgs& args, int grid, hipStream_t stream);
hipError_t launch_grouped_gemm_swiglu(const GemmArgs& args, int grid, hipStream_t stream);
hipError_t launch_grouped_gemm_planned(const GemmArgs& args, int grid, hipStream_t stream);
hipError_t grouped_gemm_occupancy(int* blocks);
hipError_t launch_combine(const uint16_t* C, int R, int N, const int32_t* row_of_slot, const float* weights, int T,
                          int top_k, uint16_t* out, hipStream_t stream);
hipError_t launch_swiglu_quant(const uint16_t* C, int R, int I, uint8_t* A, float* SA, int layout,
                               hipStream_t stream);
hipError_t launch_grouped_gemm_a16(const uint16_t* A, const uint8_t* B, const uint8_t* SB, int fmt, const float* GS,
                                   const int32_t* offsets, int E, int N, int K, uint16_t* C, int grid,
                                   hipStream_t stream);
hipError_t launch_quant_gather(const uint16_t* x, int T, int K, const int32_t* row_of_slot, int top_k, int R,
                               uint8_t* A, float* SA, int layout, hipStream_t stream);

}  // namespace w4a8
