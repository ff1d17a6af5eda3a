// C ABI of libw4a8: argument validation, per-device set-up, kernel dispatch.
// Declarations and contracts: include/w4a8.h.
#include "../../include/w4a8.h"

#include <hip/hip_runtime.h>

#include <cstdarg>
#include <cstdio>
#include <algorithm>
#include <cstring>
#include <mutex>

#include "w4a8_device.h"
#include "w4a8_launch.h"

namespace {

thread_local char g_last_error[512] = "";

int fail(int status, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_last_error, sizeof(g_last_error), fmt, ap);
  va_end(ap);
  return status;
}

int ok() {
  g_last_error[0] = '\0';
  return W4A8_OK;
}

// Device memory of the allocation-free planned GEMM: the plan of one call
// (header + 4 int32 per m-tile) lives here instead of in a caller buffer.
// Each device holds its own copy for the life of the process; host code
// reaches it only through the address hipGetSymbolAddress gives (kept per
// device in DeviceInfo::scratch), never through the array's name.
constexpr size_t kScratchBytes = (size_t)4 << 20;
static __device__ __align__(256) int32_t scratch[kScratchBytes / sizeof(int32_t)];

struct DeviceInfo {
  bool ready = false;
  bool supported = false;
  int cus = 0;
  int grid = 0;  // workgroups of the persistent GEMM launch (one per CU)
  size_t lds_limit = 0;  // LDS bytes one workgroup may hold
  int32_t* scratch = nullptr;  // this device's copy of `scratch`
};

constexpr int kMaxDevices = 64;
DeviceInfo g_dev[kMaxDevices];
std::mutex g_dev_mu;

// Per-device set-up on first use: architecture check, CU count, occupancy.
int device_info(const DeviceInfo** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail(W4A8_ERR_DEVICE, "hipGetDevice: %s", hipGetErrorString(e));
  if (dev < 0 || dev >= kMaxDevices) return fail(W4A8_ERR_DEVICE, "device index %d out of range", dev);
  std::lock_guard<std::mutex> lock(g_dev_mu);
  DeviceInfo& d = g_dev[dev];
  if (!d.ready) {
    hipDeviceProp_t prop;
    e = hipGetDeviceProperties(&prop, dev);
    if (e != hipSuccess) return fail(W4A8_ERR_DEVICE, "hipGetDeviceProperties: %s", hipGetErrorString(e));
    d.supported = std::strncmp(prop.gcnArchName, "gfx950", 6) == 0;
    d.cus = prop.multiProcessorCount;
    d.lds_limit = prop.sharedMemPerBlock;
    if (d.supported) {
      int blocks = 0;
      e = w4a8::grouped_gemm_occupancy(&blocks);
      if (e != hipSuccess) return fail(W4A8_ERR_HIP, "occupancy query: %s", hipGetErrorString(e));
      d.grid = d.cus * (blocks > 0 ? blocks : 1);
      void* ptr = nullptr;
      e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
      if (e != hipSuccess || ptr == nullptr)
        return fail(W4A8_ERR_HIP, "hipGetSymbolAddress(scratch): %s", hipGetErrorString(e));
      d.scratch = static_cast<int32_t*>(ptr);
    }
    d.ready = true;
  }
  if (!d.supported) return fail(W4A8_ERR_DEVICE, "device %d is not gfx950", dev);
  *out = &d;
  return W4A8_OK;
}

bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

int check_gemm_shape(int E, int N, int K, int max_experts = W4A8_MAX_EXPERTS) {
  if (E < 1 || E > max_experts) return fail(W4A8_ERR_SHAPE, "E=%d outside [1, %d]", E, max_experts);
  if (K < 128 || K % 128 || K > W4A8_MAX_K)
    return fail(W4A8_ERR_SHAPE, "K=%d must be a multiple of 128 in [128, %d]", K, W4A8_MAX_K);
  if (N < 32 || N % 32 || N > W4A8_MAX_N)
    return fail(W4A8_ERR_SHAPE, "N=%d must be a multiple of 32 in [32, %d]", N, W4A8_MAX_N);
  return W4A8_OK;
}

}  // namespace

extern "C" {

const char* w4a8_status_string(int status) {
  switch (status) {
    case W4A8_OK: return "W4A8_OK";
    case W4A8_ERR_NULL: return "W4A8_ERR_NULL";
    case W4A8_ERR_SHAPE: return "W4A8_ERR_SHAPE";
    case W4A8_ERR_LAYOUT: return "W4A8_ERR_LAYOUT";
    case W4A8_ERR_ALIGN: return "W4A8_ERR_ALIGN";
    case W4A8_ERR_CAPACITY: return "W4A8_ERR_CAPACITY";
    case W4A8_ERR_DEVICE: return "W4A8_ERR_DEVICE";
    case W4A8_ERR_HIP: return "W4A8_ERR_HIP";
    default: return "W4A8_UNKNOWN_STATUS";
  }
}

const char* w4a8_last_error(void) { return g_last_error; }

int w4a8_plan_params(int32_t* out_host, int n) {
  if (!out_host) return -W4A8_ERR_NULL;
  const int32_t v[7] = {w4a8::GRAN, w4a8::S_MAX, w4a8::T_MAX, w4a8::TN_STREAM, w4a8::TN_MFMA,
                        w4a8::PLAN_HEADER_WORDS, w4a8::PLAN_TILE_WORDS};
  for (int i = 0; i < n && i < 7; ++i) out_host[i] = v[i];
  return 7;
}

size_t w4a8_plan_bytes(int E, int64_t max_total_rows) {
  if (E < 1 || E > W4A8_MAX_PREP_EXPERTS || max_total_rows < 0) return 0;
  // every expert contributes at most floor(rows/T_MAX) + 1 tiles, and only
  // experts with rows contribute
  int64_t tiles = max_total_rows / w4a8::T_MAX + (max_total_rows < E ? max_total_rows : E);
  return (size_t)(w4a8::PLAN_HEADER_WORDS + w4a8::PLAN_TILE_WORDS * tiles) * sizeof(int32_t);
}

int w4a8_route_prep_waves(int E, size_t lds_limit_bytes) {
  if (E < 1 || E > W4A8_MAX_PREP_EXPERTS) return 0;
  return w4a8::route_prep_waves(E, lds_limit_bytes);
}

int w4a8_route_prep(const int32_t* topk_ids_dev, int T, int top_k, int E, int32_t* counts_dev,
                    int32_t* expert_offsets_dev, int32_t* row_of_slot_dev, void* stream) {
  if (E < 1 || E > W4A8_MAX_PREP_EXPERTS)
    return fail(W4A8_ERR_SHAPE, "E=%d outside [1, %d]", E, W4A8_MAX_PREP_EXPERTS);
  if (T < 0 || top_k < 1) return fail(W4A8_ERR_SHAPE, "T=%d top_k=%d", T, top_k);
  if ((int64_t)T * top_k >= (int64_t)1 << 31) return fail(W4A8_ERR_SHAPE, "T*top_k too large");
  const int n = T * top_k;
  if (!counts_dev || !expert_offsets_dev || (n > 0 && (!topk_ids_dev || !row_of_slot_dev)))
    return fail(W4A8_ERR_NULL, "null pointer argument");
  if (!aligned(topk_ids_dev, 4) || !aligned(counts_dev, 4) || !aligned(expert_offsets_dev, 4) ||
      !aligned(row_of_slot_dev, 4))
    return fail(W4A8_ERR_ALIGN, "pointers must be 4-byte aligned");
  const DeviceInfo* d = nullptr;
  int st = device_info(&d);
  if (st != W4A8_OK) return st;
  const int waves = w4a8::route_prep_waves(E, d->lds_limit);
  if (waves == 0)
    return fail(W4A8_ERR_CAPACITY, "E=%d needs %zu bytes of LDS with one wave; the device allows %zu", E,
                w4a8::route_prep_lds_bytes(E, 1), d->lds_limit);
  hipError_t e = w4a8::launch_route_prep(topk_ids_dev, n, E, waves, counts_dev, expert_offsets_dev,
                                          row_of_slot_dev, (hipStream_t)stream);
  if (e != hipSuccess) return fail(W4A8_ERR_HIP, "route_prep launch: %s", hipGetErrorString(e));
  return ok();
}

int w4a8_plan(const int32_t* expert_offsets_dev, int E, int N, int K, void* plan_dev,
              size_t plan_bytes, void* stream) {
  // the plan serves every E the route prep serves; N and K as for the GEMM
  int st = check_gemm_shape(E, N, K, W4A8_MAX_PREP_EXPERTS);
  if (st != W4A8_OK) return st;
  if (!expert_offsets_dev || !plan_dev) return fail(W4A8_ERR_NULL, "null pointer argument");
  if (!aligned(expert_offsets_dev, 4) || !aligned(plan_dev, 4))
    return fail(W4A8_ERR_ALIGN, "pointers must be 4-byte aligned");
  const size_t words = plan_bytes / sizeof(int32_t);
  if (words < (size_t)w4a8::PLAN_HEADER_WORDS)
    return fail(W4A8_ERR_CAPACITY, "plan buffer of %zu bytes cannot hold the header", plan_bytes);
  size_t max_tiles = (words - w4a8::PLAN_HEADER_WORDS) / w4a8::PLAN_TILE_WORDS;
  if (max_tiles > (size_t)0x7fffffff) max_tiles = 0x7fffffff;
  const DeviceInfo* d = nullptr;
  st = device_info(&d);
  if (st != W4A8_OK) return st;
  hipError_t e = w4a8::launch_plan(expert_offsets_dev, E, N, (int32_t*)plan_dev, (int)max_tiles,
                                   (hipStream_t)stream);
  if (e != hipSuccess) return fail(W4A8_ERR_HIP, "plan launch: %s", hipGetErrorString(e));
  return ok();
}

int w4a8_grouped_gemm(const uint8_t* A_fp8_dev, const float* a_scales_dev, int a_scale_layout,
                      const uint8_t* B_fp4_dev, const uint8_t* b_scales_e8m0_dev,
                      const int32_t* expert_offsets_dev, int E, int N, int K, uint16_t* C_bf16_dev,
                      void* stream) {
  int st = check_gemm_shape(E, N, K);
  if (st != W4A8_OK) return st;
  if (a_scale_layout != W4A8_SCALE_ROW_MAJOR && a_scale_layout != W4A8_SCALE_M_MAJOR)
    return fail(W4A8_ERR_LAYOUT, "a_scale_layout=%d is neither row-major (0) nor M-major (1)", a_scale_layout);
  if (!A_fp8_dev || !a_scales_dev || !B_fp4_dev || !b_scales_e8m0_dev || !expert_offsets_dev || !C_bf16_dev)
    return fail(W4A8_ERR_NULL, "null pointer argument");
  if (!aligned(A_fp8_dev, 16) || !aligned(B_fp4_dev, 16) || !aligned(C_bf16_dev, 16) ||
      !aligned(a_scales_dev, 4) || !aligned(b_scales_e8m0_dev, 4) || !aligned(expert_offsets_dev, 4))
    return fail(W4A8_ERR_ALIGN, "A, B, C need 16-byte and scales/offsets 4-byte alignment");
  const DeviceInfo* d = nullptr;
  st = device_info(&d);
  if (st != W4A8_OK) return st;
  w4a8::GemmArgs args{A_fp8_dev, a_scales_dev, B_fp4_dev, b_scales_e8m0_dev, expert_offsets_dev,
                      C_bf16_dev, E, N, K, a_scale_layout, nullptr, nullptr, 0, 0, nullptr, 0};
  hipError_t e = w4a8::launch_grouped_gemm(args, d->grid, (hipStream_t)stream);
  if (e != hipSuccess) return fail(W4A8_ERR_HIP, "grouped_gemm launch: %s", hipGetErrorString(e));
  return ok();
}

int w4a8_grouped_gemm_planned(const uint8_t* A_fp8_dev, const float* a_scales_dev, int a_scale_layout,
                              const uint8_t* B_fp4_dev, const uint8_t* b_scales_e8m0_dev,
                              const int32_t* expert_offsets_dev, int E, int N, int K, const void* plan_dev,
                              size_t plan_bytes, uint16_t* C_bf16_dev, void* stream) {
  int st = check_gemm_shape(E, N, K, W4A8_MAX_PREP_EXPERTS);
  if (st != W4A8_OK) return st;
  if (a_scale_layout != W4A8_SCALE_ROW_MAJOR && a_scale_layout != W4A8_SCALE_M_MAJOR)
    return fail(W4A8_ERR_LAYOUT, "a_scale_layout=%d is neither row-major (0) nor M-major (1)", a_scale_layout);
  if (!A_fp8_dev || !a_scales_dev || !B_fp4_dev || !b_scales_e8m0_dev || !expert_offsets_dev || !plan_dev ||
      !C_bf16_dev)
    return fail(W4A8_ERR_NULL, "null pointer argument");
  if (!aligned(A_fp8_dev, 16) || !aligned(B_fp4_dev, 16) || !aligned(C_bf16_dev, 16) ||
      !aligned(a_scales_dev, 4) || !aligned(b_scales_e8m0_dev, 4) || !aligned(expert_offsets_dev, 4) ||
      !aligned(plan_dev, 4))
    return fail(W4A8_ERR_ALIGN, "A, B, C need 16-byte and scales/offsets/plan 4-byte alignment");
  const size_t words = plan_bytes / sizeof(int32_t);
  if (words < (size_t)w4a8::PLAN_HEADER_WORDS)
    return fail(W4A8_ERR_CAPACITY, "plan buffer of %zu bytes cannot hold the header", plan_bytes);
  size_t max_tiles = (words - w4a8::PLAN_HEADER_WORDS) / w4a8::PLAN_TILE_WORDS;
  if (max_tiles > (size_t)0x7fffffff) max_tiles = 0x7fffffff;
  const DeviceInfo* d = nullptr;
  st = device_info(&d);
  if (st != W4A8_OK) return st;
  w4a8::GemmArgs args{A_fp8_dev, a_scales_dev, B_fp4_dev, b_scales_e8m0_dev, expert_offsets_dev, C_bf16_dev,
                      E, N, K, a_scale_layout, nullptr, nullptr, 0, 0, (const int32_t*)plan_dev, (int)max_tiles};
  hipError_t e = w4a8::launch_grouped_gemm_planned(args, d->grid, (hipStream_t)stream);
  if (e != hipSuccess) return fail(W4A8_ERR_HIP, "grouped_gemm_planned launch: %s", hipGetErrorString(e));
  return ok();
}

int w4a8_grouped_gemm_planned_noalloc(const uint8_t* A_fp8_dev, const float* a_scales_dev, int a_scale_layout,
                                      const uint8_t* B_fp4_dev, const uint8_t* b_scales_e8m0_dev,
                                      const int32_t* expert_offsets_dev, int E, int N, int K, int64_t max_total_rows,
                                      uint16_t* C_bf16_dev, void* stream) {
  int st = check_gemm_shape(E, N, K, W4A8_MAX_PREP_EXPERTS);
  if (st != W4A8_OK) return st;
  if (a_scale_layout != W4A8_SCALE_ROW_MAJOR && a_scale_layout != W4A8_SCALE_M_MAJOR)
    return fail(W4A8_ERR_LAYOUT, "a_scale_layout=%d is neither row-major (0) nor M-major (1)", a_scale_layout);
  if (!A_fp8_dev || !a_scales_dev || !B_fp4_dev || !b_scales_e8m0_dev || !expert_offsets_dev || !C_bf16_dev)
    return fail(W4A8_ERR_NULL, "null pointer argument");
  if (!aligned(A_fp8_dev, 16) || !aligned(B_fp4_dev, 16) || !aligned(C_bf16_dev, 16) ||
      !aligned(a_scales_dev, 4) || !aligned(b_scales_e8m0_dev, 4) || !aligned(expert_offsets_dev, 4))
    return fail(W4A8_ERR_ALIGN, "A, B, C need 16-byte and scales/offsets 4-byte alignment");
  if (max_total_rows < 0) return fail(W4A8_ERR_SHAPE, "max_total_rows=%lld", (long long)max_total_rows);
  const size_t need = w4a8_plan_bytes(E, max_total_rows);
  if (need > kScratchBytes)
    return fail(W4A8_ERR_CAPACITY, "a plan for E=%d and %lld rows needs %zu bytes; the library's device scratch "
                "holds %zu", E, (long long)max_total_rows, need, kScratchBytes);
  const DeviceInfo* d = nullptr;
  st = device_info(&d);
  if (st != W4A8_OK) return st;
  const int max_tiles = (int)((kScratchBytes / sizeof(int32_t) - w4a8::PLAN_HEADER_WORDS) / w4a8::PLAN_TILE_WORDS);
  hipError_t e = w4a8::launch_plan(expert_offsets_dev, E, N, d->scratch, max_tiles, (hipStream_t)stream);
  if (e != hipSuccess) return fail(W4A8_ERR_HIP, "plan launch: %s", hipGetErrorString(e));
  w4a8::GemmArgs args{A_fp8_dev, a_scales_dev, B_fp4_dev, b_scales_e8m0_dev, expert_offsets_dev, C_bf16_dev,
                      E, N, K, a_scale_layout, nullptr, nullptr, 0, 0, d->scratch, max_tiles};
  e = w4a8::launch_grouped_gemm_planned(args, d->grid, (hipStream_t)stream);
  if (e != hipSuccess) return fail(W4A8_ERR_HIP, "grouped_gemm_planned launch: %s", hipGetErrorString(e));
  return ok();
}

int w4a8_grouped_gemm_swiglu(const uint8_t* A_fp8_dev, const float* a_scales_dev, int a_scale_layout,
                             const uint8_t* B13_fp4_dev, const uint8_t* b13_scales_e8m0_dev,
                             const int32_t* expert_offsets_dev, int E, int I, int K, uint8_t* A2_fp8_dev,
                             float* a2_scales_dev, int a2_scale_layout, void* stream) {
  if (I < 128 || I % 128 || (int64_t)I > W4A8_MAX_N / 2)
    return fail(W4A8_ERR_SHAPE, "I=%d must be a multiple of 128 in [128, %d]", I, W4A8_MAX_N / 2);
  int st = check_gemm_shape(E, 2 * I, K);
  if (st != W4A8_OK) return st;
  if ((int64_t)2 * I * (K / 2) >= ((int64_t)1 << 31))
    return fail(W4A8_ERR_SHAPE, "2I * K/2 = %lld bytes of one expert's weights must stay below 2^31",
                (long long)2 * I * (K / 2));
  if ((a_scale_layout != W4A8_SCALE_ROW_MAJOR && a_scale_layout != W4A8_SCALE_M_MAJOR) ||
      (a2_scale_layout != W4A8_SCALE_ROW_MAJOR && a2_scale_layout != W4A8_SCALE_M_MAJOR))
    return fail(W4A8_ERR_LAYOUT, "scale layouts %d, %d must be row-major (0) or M-major (1)", a_scale_layout,
                a2_scale_layout);
  if (!A_fp8_dev || !a_scales_dev || !B13_fp4_dev || !b13_scales_e8m0_dev || !expert_offsets_dev || !A2_fp8_dev ||
      !a2_scales_dev)
    return fail(W4A8_ERR_NULL, "null pointer argument");
  if (!aligned(A_fp8_dev, 16) || !aligned(B13_fp4_dev, 16) || !aligned(A2_fp8_dev, 16) ||
      !aligned(a_scales_dev, 4) || !aligned(b13_scales_e8m0_dev, 4) || !aligned(expert_offsets_dev, 4) ||
      !aligned(a2_scales_dev, 4))
    return fail(W4A8_ERR_ALIGN, "A, B13, A2 need 16-byte and scales/offsets 4-byte alignment");
  const DeviceInfo* d = nullptr;
  st = device_info(&d);
  if (st != W4A8_OK) return st;
  w4a8::GemmArgs args{A_fp8_dev, a_scales_dev, B13_fp4_dev, b13_scales_e8m0_dev, expert_offsets_dev, nullptr,
                      E, 2 * I, K, a_scale_layout, A2_fp8_dev, a2_scales_dev, I, a2_scale_layout, nullptr, 0};
  hipError_t e = w4a8::launch_grouped_gemm_swiglu(args, d->grid, (hipStream_t)stream);
  if (e != hipSuccess) return fail(W4A8_ERR_HIP, "grouped_gemm_swiglu launch: %s", hipGetErrorString(e));
  return ok();
}

int w4a8_quantize_gather(const uint16_t* x_bf16_dev, int T, int K, const int32_t* row_of_slot_dev, int top_k,
                         int R, uint8_t* A_fp8_dev, float* a_scales_dev, int a_scale_layout, void* stream) {
  if (T < 0 || top_k < 1 || R < 0) return fail(W4A8_ERR_SHAPE, "T=%d top_k=%d R=%d", T, top_k, R);
  if ((int64_t)T * top_k >= (int64_t)1 << 31) return fail(W4A8_ERR_SHAPE, "T*top_k too large");
  if (K < 128 || K % 128 || K > W4A8_MAX_K)
    return fail(W4A8_ERR_SHAPE, "K=%d must be a multiple of 128 in [128, %d]", K, W4A8_MAX_K);
  if (a_scale_layout != W4A8_SCALE_ROW_MAJOR && a_scale_layout != W4A8_SCALE_M_MAJOR)
    return fail(W4A8_ERR_LAYOUT, "a_scale_layout=%d is neither row-major (0) nor M-major (1)", a_scale_layout);
  if (T > 0 && (!x_bf16_dev || !row_of_slot_dev || (R > 0 && (!A_fp8_dev || !a_scales_dev))))
    return fail(W4A8_ERR_NULL, "null pointer argument");
  if (!aligned(x_bf16_dev, 16) || !aligned(A_fp8_dev, 16) || !aligned(row_of_slot_dev, 4) ||
      !aligned(a_scales_dev, 4))
    return fail(W4A8_ERR_ALIGN, "x and A need 16-byte, row_of_slot and scales 4-byte alignment");
  const DeviceInfo* d = nullptr;
  int st = device_info(&d);
  if (st != W4A8_OK) return st;
  if (T == 0 || R == 0) return ok();
  hipError_t e = w4a8::launch_quant_gather(x_bf16_dev, T, K, row_of_slot_dev, top_k, R, A_fp8_dev, a_scales_dev,
                                           a_scale_layout, (hipStream_t)stream);
  if (e != hipSuccess) return fail(W4A8_ERR_HIP, "quantize_gather launch: %s", hipGetErrorString(e));
  return ok();
}

int w4a8_combine(const uint16_t* C_bf16_dev, int R, int N, const int32_t* row_of_slot_dev,
                 const float* weights_dev, int T, int top_k, uint16_t* out_bf16_dev, void* stream) {
  if (T < 0 || top_k < 1 || R < 0) return fail(W4A8_ERR_SHAPE, "T=%d top_k=%d R=%d", T, top_k, R);
  if ((int64_t)T * top_k >= (int64_t)1 << 31) return fail(W4A8_ERR_SHAPE, "T*top_k too large");
  if (N < 8 || N % 8 || N > W4A8_MAX_N) return fail(W4A8_ERR_SHAPE, "N=%d must be a multiple of 8 in [8, %d]", N, W4A8_MAX_N);
  if (T > 0 && (!row_of_slot_dev || !weights_dev || !out_bf16_dev || (R > 0 && !C_bf16_dev)))
    return fail(W4A8_ERR_NULL, "null pointer argument");
  if (!aligned(C_bf16_dev, 16) || !aligned(out_bf16_dev, 16) || !aligned(row_of_slot_dev, 4) ||
      !aligned(weights_dev, 4))
    return fail(W4A8_ERR_ALIGN, "C and out need 16-byte, row_of_slot and weights 4-byte alignment");
  const DeviceInfo* d = nullptr;
  int st = device_info(&d);
  if (st != W4A8_OK) return st;
  if (T == 0) return ok();
  hipError_t e = w4a8::launch_combine(C_bf16_dev, R, N, row_of_slot_dev, weights_dev, T, top_k, out_bf16_dev,
                                      (hipStream_t)stream);
  if (e != hipSuccess) return fail(W4A8_ERR_HIP, "combine launch: %s", hipGetErrorString(e));
  return ok();
}

int w4a8_grouped_gemm_a16(const uint16_t* A_bf16_dev, const uint8_t* B_fp4_dev, const uint8_t* b_scales_dev,
                          int b_scale_format, const float* expert_scales_dev, const int32_t* expert_offsets_dev,
                          int E, int N, int K, uint16_t* C_bf16_dev, void* stream) {
  if (E < 1 || E > W4A8_MAX_PREP_EXPERTS)
    return fail(W4A8_ERR_SHAPE, "E=%d outside [1, %d]", E, W4A8_MAX_PREP_EXPERTS);
  if (K < 128 || K % 128 || K > W4A8_MAX_K)
    return fail(W4A8_ERR_SHAPE, "K=%d must be a multiple of 128 in [128, %d]", K, W4A8_MAX_K);
  if (N < 16 || N % 16 || N > W4A8_MAX_N)
    return fail(W4A8_ERR_SHAPE, "N=%d must be a multiple of 16 in [16, %d]", N, W4A8_MAX_N);
  if ((int64_t)E * ((N + 63) / 64) >= ((int64_t)1 << 31)) return fail(W4A8_ERR_SHAPE, "E * ceil(N/64) too large");
  if (b_scale_format != W4A8_WSCALE_MX && b_scale_format != W4A8_WSCALE_NV)
    return fail(W4A8_ERR_LAYOUT, "b_scale_format=%d is neither MXFP4 (0) nor NVFP4 (1)", b_scale_format);
  if (!A_bf16_dev || !B_fp4_dev || !b_scales_dev || !expert_offsets_dev || !C_bf16_dev)
    return fail(W4A8_ERR_NULL, "null pointer argument");
  if (!aligned(A_bf16_dev, 16) || !aligned(B_fp4_dev, 16) || !aligned(C_bf16_dev, 16) ||
      !aligned(b_scales_dev, 4) || !aligned(expert_scales_dev, 4) || !aligned(expert_offsets_dev, 4))
    return fail(W4A8_ERR_ALIGN, "A, B, C need 16-byte and scales/offsets 4-byte alignment");
  const DeviceInfo* d = nullptr;
  int st = device_info(&d);
  if (st != W4A8_OK) return st;
  // items of (expert, 64 columns), about four workgroups of four waves per CU
  const int64_t items = (int64_t)E * ((N + 63) / 64);
  const int grid = (int)std::min<int64_t>(items, (int64_t)4 * d->cus);
  hipError_t e = w4a8::launch_grouped_gemm_a16(A_bf16_dev, B_fp4_dev, b_scales_dev, b_scale_format,
                                               expert_scales_dev, expert_offsets_dev, E, N, K, C_bf16_dev, grid,
                                               (hipStream_t)stream);
  if (e != hipSuccess) return fail(W4A8_ERR_HIP, "grouped_gemm_a16 launch: %s", hipGetErrorString(e));
  return ok();
}

int w4a8_swiglu_quant(const uint16_t* C_bf16_dev, int R, int I, uint8_t* A_fp8_dev, float* a_scales_dev,
                      int a_scale_layout, void* stream) {
  if (R < 0) return fail(W4A8_ERR_SHAPE, "R=%d", R);
  if (I < 128 || I % 128 || I > W4A8_MAX_K)
    return fail(W4A8_ERR_SHAPE, "I=%d must be a multiple of 128 in [128, %d]", I, W4A8_MAX_K);
  if (a_scale_layout != W4A8_SCALE_ROW_MAJOR && a_scale_layout != W4A8_SCALE_M_MAJOR)
    return fail(W4A8_ERR_LAYOUT, "a_scale_layout=%d is neither row-major (0) nor M-major (1)", a_scale_layout);
  if (R > 0 && (!C_bf16_dev || !A_fp8_dev || !a_scales_dev)) return fail(W4A8_ERR_NULL, "null pointer argument");
  if (!aligned(C_bf16_dev, 16) || !aligned(A_fp8_dev, 16) || !aligned(a_scales_dev, 4))
    return fail(W4A8_ERR_ALIGN, "C and A need 16-byte, scales 4-byte alignment");
  const DeviceInfo* d = nullptr;
  int st = device_info(&d);
  if (st != W4A8_OK) return st;
  if (R == 0) return ok();
  hipError_t e = w4a8::launch_swiglu_quant(C_bf16_dev, R, I, A_fp8_dev, a_scales_dev, a_scale_layout,
                                           (hipStream_t)stream);
  if (e != hipSuccess) return fail(W4A8_ERR_HIP, "swiglu_quant launch: %s", hipGetErrorString(e));
  return ok();
}

}  // extern "C"
