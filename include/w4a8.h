/*
 * w4a8.h -- C ABI of the grouped-contiguous W4A8 MoE expert GEMM for MI355X (gfx950).
 *
 * The operation (humming PR #129, title, intro and the "Results" benchmark
 * command): a grouped GEMM over experts whose routed rows are stored
 * contiguously by expert, with
 *   A  FP8 E4M3 activations, one fp32 scale per (row, 128-K group), the scales
 *      stored row-major or M-major ("--input_scale_group_size 128",
 *      "--use_m_major_input_scale");
 *   B  MXFP4 E2M1 expert weights, one E8M0 scale per 32 K
 *      ("--b_dtype float4e2m1 --bs_dtype float8e8m0 --weight_scale_group_size 32");
 *   C  bf16 output ("--c_dtype bfloat16");
 * and the M tile of every expert chosen from that expert's own row count
 * (same page, commit 1 "Row-major tile model" and commit 2 "Small-expert seed
 * tile").  The routing prep that produces the contiguous grouping keeps a
 * per-expert histogram and prefix arrays, as the MoE planning kernel of
 * MoonEP PR #38 (background section) does.
 *
 *   C[r, n] = bf16_rne( sum_k e4m3(A[r,k]) * SA(r, k/128)
 *                             * e2m1(B[e,n,k]) * 2^(SB[e,n,k/32] - 127) ),
 *   e = the expert with offsets[e] <= r < offsets[e+1].
 *
 * Conventions shared by every entry point
 *   - Pointers named *_dev are device pointers (hipMalloc / torch CUDA memory);
 *     pointers named *_host are host pointers.  The caller owns every buffer;
 *     the library keeps no pointer after the call's stream work completes and
 *     never allocates or frees memory on the call path.
 *   - `stream` is a hipStream_t passed as void* (NULL = the legacy default
 *     stream).  All device work is enqueued on it asynchronously; no entry
 *     point synchronises the host, so calls may be captured in a HIP graph.
 *   - Return value: a w4a8_status.  Argument errors the host can see are
 *     reported before anything is launched; a HIP launch failure returns
 *     W4A8_ERR_HIP.  w4a8_last_error() gives a per-thread text for the last
 *     non-OK return.
 *   - Conditions only the device can see (offsets not starting at 0 or
 *     decreasing) make the kernels write nothing; w4a8_plan reports them in
 *     its header's status word.
 *   - Only gfx950 devices are supported (W4A8_ERR_DEVICE otherwise).
 */
#ifndef W4A8_H
#define W4A8_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  W4A8_OK = 0,
  W4A8_ERR_NULL = 1,      /* a required pointer is NULL */
  W4A8_ERR_SHAPE = 2,     /* E, N, K, T or top_k outside the supported range */
  W4A8_ERR_LAYOUT = 3,    /* unknown a_scale_layout */
  W4A8_ERR_ALIGN = 4,     /* a pointer is not aligned as documented */
  W4A8_ERR_CAPACITY = 5,  /* a caller buffer is too small */
  W4A8_ERR_DEVICE = 6,    /* current device is not gfx950 or cannot be queried */
  W4A8_ERR_HIP = 7        /* a HIP runtime call failed */
} w4a8_status;

/* Input-scale layouts (humming PR #129: row-major and M-major input scales). */
enum {
  W4A8_SCALE_ROW_MAJOR = 0, /* a_scales fp32 [R][K/128]: SA(r,g) at r*(K/128)+g */
  W4A8_SCALE_M_MAJOR = 1    /* a_scales fp32 [K/128][R]: SA(r,g) at g*R+r, R = offsets[E] */
};

/* Weight-scale formats of w4a8_grouped_gemm_a16. */
enum {
  W4A8_WSCALE_MX = 0,  /* MXFP4: E8M0 code per (expert, column, 32 K), value 2^(code-127) */
  W4A8_WSCALE_NV = 1   /* NVFP4: E4M3FN code per (expert, column, 16 K) */
};

/* Limits of this version. */
#define W4A8_MAX_EXPERTS 2048        /* grouped GEMM: per-expert tables live in LDS */
#define W4A8_MAX_PREP_EXPERTS 65536  /* route prep and plan; the route prep's LDS fit
                                        may lower it on a device (W4A8_ERR_CAPACITY) */
#define W4A8_MAX_K 1048576     /* keeps every in-tile byte offset within 32 bits */
#define W4A8_MAX_N 16777216    /* keeps work-item counts within 32 bits */

/*
 * w4a8_route_prep -- routing histogram, exclusive-scan offsets and row map.
 *
 * topk_ids_dev       int32 [T*top_k], row-major [T][top_k]: expert of each
 *                    (token, slot).  Ids outside [0, E) are ignored.
 * counts_dev         out int32 [E]: slots routed to each expert.
 * expert_offsets_dev out int32 [E+1]: offsets[0] = 0, offsets[e+1] =
 *                    offsets[e] + counts[e]; offsets[E] = R, the routed rows.
 * row_of_slot_dev    out int32 [T*top_k]: the grouped row of each slot; rows
 *                    of one expert keep the flat (token, slot) order (a stable
 *                    counting sort), so the result is unique.  -1 for an
 *                    ignored id.
 * Limits: 1 <= E <= W4A8_MAX_PREP_EXPERTS, 0 <= T, 1 <= top_k,
 * T*top_k < 2^31.  Large E (MoonEP PR #38, background section: shared expert
 * pools of thousands of experts): a workgroup of 16 waves holds
 * (W + 2) * E + 16 int32 of LDS, where W waves rank the slots of the
 * workgroup's chunk, each with its own copy of per-expert counts; W is the
 * largest of 16, 15, ..., 1 that fits the device's per-workgroup LDS (the
 * fit of MoonEP PR #38, change section, applied to the ranking copies: the
 * other waves need no LDS, so the workgroup keeps all 16).  A batch of fewer
 * than 1024 slots uses at most one ranking wave per 64 slots, and the
 * workgroup then holds only those waves and one per 64 experts (at most 16).
 * When not even one copy fits (E above 13648 on a 160 KB device) the call
 * returns W4A8_ERR_CAPACITY before any launch.  The result does not depend on
 * W or on the number of waves.
 * Alignment: 4 bytes for every pointer.
 */
int w4a8_route_prep(const int32_t* topk_ids_dev, int T, int top_k, int E,
                    int32_t* counts_dev, int32_t* expert_offsets_dev,
                    int32_t* row_of_slot_dev, void* stream);

/*
 * w4a8_route_prep_waves -- host only, no device work: the ranking waves per
 * workgroup w4a8_route_prep uses for E experts on a device whose workgroups
 * may hold lds_limit_bytes of LDS, for batches of at least 1024 slots (the
 * largest W in 16..1 with
 * 4 * ((W + 2) * E + 16) <= lds_limit_bytes).  Returns 0 when no W fits (the
 * route prep then returns W4A8_ERR_CAPACITY) or E is outside
 * [1, W4A8_MAX_PREP_EXPERTS].
 */
int w4a8_route_prep_waves(int E, size_t lds_limit_bytes);

/*
 * w4a8_plan_bytes -- bytes a plan buffer needs for E experts and at most
 * max_total_rows routed rows (host only; no device work).  Returns 0 for
 * E outside [1, W4A8_MAX_PREP_EXPERTS] or a negative row count.
 */
size_t w4a8_plan_bytes(int E, int64_t max_total_rows);

/*
 * w4a8_plan -- per-expert tile list built on the device from expert offsets
 * (the tile rule that the GEMM kernels apply in their own prologue, exposed
 * for inspection and for callers that want the list).
 *
 * expert_offsets_dev int32 [E+1] (as produced by w4a8_route_prep).
 * plan_dev           out int32 buffer of plan_bytes bytes:
 *   header [8]: status (0 ok, 1 offsets invalid, 2 buffer too small),
 *               m-tiles, streaming-class m-tiles, MFMA-class m-tiles,
 *               streaming work items, MFMA work items, padded rows, rows R
 *   then 4 int32 per m-tile: expert, first row, rows, tile_m | class << 16
 *   (class 1 = weight-streaming small-M kernel, 2 = MFMA kernel); streaming
 *   tiles first, then MFMA tiles, each in (expert, row) order.
 * Rule for an expert with rows r (integer only; constants by w4a8_plan_params):
 *   r == 0 -> no tile; r <= S_MAX -> one streaming tile, tile_m = ceil16(r);
 *   r > S_MAX -> n = ceil(r / T_MAX) MFMA tiles, tile_m = ceil16(ceil(r / n)).
 * Limits: 1 <= E <= W4A8_MAX_PREP_EXPERTS (offsets are read from global
 * memory, no LDS bound); N and K as w4a8_grouped_gemm.  plan_bytes must hold
 * at least the header (W4A8_ERR_CAPACITY otherwise); a plan with more tiles
 * than fit sets status 2 and writes the tiles that fit.  Alignment: 4 bytes.
 */
int w4a8_plan(const int32_t* expert_offsets_dev, int E, int N, int K,
              void* plan_dev, size_t plan_bytes, void* stream);

/*
 * w4a8_quantize_gather -- the producer of the GEMM's A and a_scales: bf16
 * tokens quantized to E4M3 codes with one fp32 scale per (row, 128-K group)
 * (humming PR #129, "Results" command: float8e4m3 activations, input-scale
 * group size 128), written to the grouped row of every (token, slot).
 *
 * x_bf16_dev       uint16 (bf16 bits) [T][K], row-major.  16-byte aligned.
 * row_of_slot_dev  int32 [T*top_k] (as produced by w4a8_route_prep): the
 *                  grouped row of slot (t, j) at t*top_k + j.  Slots whose
 *                  row is outside [0, R) are skipped.  4-byte aligned.
 * A_fp8_dev        out uint8 [R][K] E4M3FN codes.  16-byte aligned.
 * a_scales_dev     out fp32 per (row, group) in a_scale_layout
 *                  (W4A8_SCALE_ROW_MAJOR [R][K/128] or W4A8_SCALE_M_MAJOR
 *                  [K/128][R]).  4-byte aligned.
 * Per token t and group g: s = amax|x[t, 128g .. 128g+127]| / 448 (1 if the
 * group is all zero), code = E4M3FN round-to-nearest-even of clip(x / s,
 * +-448), fp32 divisions rounded to nearest; sign kept (-0 -> 0x80).  Every
 * named row gets the codes and scales of its token; other rows are left as
 * they were.  NaN or infinite inputs are outside the definition.
 * Limits: T >= 0, 1 <= top_k, T*top_k < 2^31, K % 128 == 0,
 * 128 <= K <= W4A8_MAX_K, R >= 0.  T == 0 or R == 0 does nothing.
 */
int w4a8_quantize_gather(const uint16_t* x_bf16_dev, int T, int K,
                         const int32_t* row_of_slot_dev, int top_k, int R,
                         uint8_t* A_fp8_dev, float* a_scales_dev, int a_scale_layout,
                         void* stream);

/*
 * w4a8_combine -- the step after the grouped GEMM: every token's top_k
 * expert rows summed back, each weighted by its router weight (the
 * single-GPU half of an expert-parallel combine; the routing it inverts is
 * the MoE planning of MoonEP PR #38, background section).
 *
 * C_bf16_dev       uint16 (bf16 bits) [R][N], grouped rows.  16-byte aligned.
 * row_of_slot_dev  int32 [T*top_k]: the row of slot (t, j) at t*top_k + j
 *                  (as produced by w4a8_route_prep); rows outside [0, R)
 *                  contribute nothing.  4-byte aligned.
 * weights_dev      fp32 [T*top_k]: the weight of each slot.  4-byte aligned.
 * out_bf16_dev     out uint16 (bf16 bits) [T][N].  16-byte aligned.
 * out[t, :] = bf16_rne(sum over j = 0, 1, ..., top_k-1 of w[t, j] *
 * C[row(t, j), :]), summed in fp32 in that order with one rounded product
 * and one rounded addition per term (no fused multiply-add), from 0; a token
 * with no valid slot gets zeros.  The result is unique.
 * Limits: T >= 0, 1 <= top_k, T*top_k < 2^31, N % 8 == 0,
 * 8 <= N <= W4A8_MAX_N, R >= 0.  T == 0 does nothing.
 */
int w4a8_combine(const uint16_t* C_bf16_dev, int R, int N, const int32_t* row_of_slot_dev,
                 const float* weights_dev, int T, int top_k, uint16_t* out_bf16_dev, void* stream);

/*
 * w4a8_swiglu_quant -- the step between the two projections (humming PR
 * #129 and PR #58 benchmark gate/up and down as a pair): SwiGLU of the
 * gate/up output, requantized to E4M3 with one fp32 scale per (row, 128) for
 * the down projection's A and a_scales.
 *
 * C_bf16_dev    uint16 (bf16 bits) [R][2I]: gate in columns 0 .. I-1, up in
 *               columns I .. 2I-1.  16-byte aligned.
 * A_fp8_dev     out uint8 [R][I] E4M3FN codes.  16-byte aligned.
 * a_scales_dev  out fp32 per (row, 128-column group) in a_scale_layout
 *               (row-major [R][I/128] or M-major [I/128][R]).  4-byte aligned.
 * h = silu(g) * u = (g / (1 + e^-g)) * u, evaluated in fp32 with the
 * hardware exponential and reciprocal (within about five fp32 units in the
 * last place of the exact value; where e^-g overflows fp32, g below about
 * -88.7, silu is -0); then per group s = amax|h| / 448 (1 if all zero) and
 * the E4M3FN code of clip(h * (1/s), +-448), round to nearest even.  Near an
 * E4M3 rounding midpoint the fp32 evaluation may pick either neighbour: the
 * result is the definition's for values within 2^-20 relative of the exact
 * ones, not bit-reproducible by another evaluation order.  Deterministic:
 * the same input gives the same bytes.
 * Limits: R >= 0, I % 128 == 0, 128 <= I <= W4A8_MAX_K.  R == 0 does nothing.
 */
int w4a8_swiglu_quant(const uint16_t* C_bf16_dev, int R, int I, uint8_t* A_fp8_dev, float* a_scales_dev,
                      int a_scale_layout, void* stream);

/*
 * w4a8_grouped_gemm -- the grouped W4A8 GEMM.
 *
 * A_fp8_dev          uint8 [R][K] E4M3 codes; rows offsets[e]..offsets[e+1]-1
 *                    belong to expert e.  16-byte aligned.
 * a_scales_dev       fp32 per (row, 128-K group) in the given layout
 *                    (W4A8_SCALE_ROW_MAJOR or W4A8_SCALE_M_MAJOR; for M-major
 *                    the leading dimension is R = offsets[E], read on the
 *                    device).  4-byte aligned.
 * B_fp4_dev          uint8 [E][N][K/2] E2M1 codes, K-contiguous per output
 *                    column; element 2j in bits 3:0, element 2j+1 in bits 7:4.
 *                    16-byte aligned.
 * b_scales_e8m0_dev  uint8 [E][N][K/32] E8M0 codes.  4-byte aligned.
 * expert_offsets_dev int32 [E+1], offsets[0] = 0, nondecreasing.
 * C_bf16_dev         out uint16 (bf16 bits) [R][N]; only rows < R are written.
 *                    16-byte aligned.
 * Limits: 1 <= E <= W4A8_MAX_EXPERTS; K % 128 == 0, 128 <= K <= W4A8_MAX_K;
 * N % 32 == 0, 32 <= N <= W4A8_MAX_N; R*K and R*N below 2^62.  A, a_scales and C must hold R rows.
 * Numerics: each 128-K group is reduced by a scaled MFMA in fp32 (E8M0 weight
 * scales applied inside it), multiplied by its fp32 activation scale and
 * accumulated in fp32; one RNE rounding to bf16 at the end.  NaN codes
 * (E4M3 S.1111.111, E8M0 0xFF) propagate to the rows/columns they touch.
 */
int w4a8_grouped_gemm(const uint8_t* A_fp8_dev, const float* a_scales_dev, int a_scale_layout,
                      const uint8_t* B_fp4_dev, const uint8_t* b_scales_e8m0_dev,
                      const int32_t* expert_offsets_dev, int E, int N, int K,
                      uint16_t* C_bf16_dev, void* stream);

/*
 * w4a8_grouped_gemm_planned -- the grouped W4A8 GEMM of w4a8_grouped_gemm,
 * run over a tile list built beforehand instead of one the kernel derives
 * from the offsets.  The per-expert tables of w4a8_grouped_gemm live in LDS
 * and stop at W4A8_MAX_EXPERTS; this entry point keeps none, so it serves
 * the shared expert pools of thousands of experts that MoonEP PR #38
 * (background section) plans for, up to W4A8_MAX_PREP_EXPERTS.  One plan
 * serves every GEMM over the same offsets (gate/up and down of a layer).
 *
 * plan_dev, plan_bytes  a plan in w4a8_plan's format (header, then
 *                    {expert, first row, rows, tile_m | class << 16} per
 *                    m-tile, streaming tiles first), normally w4a8_plan's
 *                    output for the same offsets, E and N; caller-owned,
 *                    read only.  4-byte aligned.  Other rules may be run
 *                    through it as long as every streaming tile (class 1)
 *                    holds 1 .. S_MAX rows and every MFMA tile (class 2)
 *                    1 .. T_MAX rows (w4a8_plan_params).
 * Every tile is checked against the offsets before use: a tile whose rows
 * are not inside its expert's rows and inside [0, R) is skipped (its rows
 * are then not written), so no plan makes the kernel touch memory outside
 * A, a_scales, B, b_scales and C.  A plan whose status word is not 0 makes
 * the kernel write nothing.  Streaming tiles are dealt as items of up to
 * 512 columns (split further where the tile's rows leave fewer registers
 * per column), MFMA tiles as 512-column items.  The other
 * arguments, layouts, numerics and limits are those of w4a8_grouped_gemm,
 * except 1 <= E <= W4A8_MAX_PREP_EXPERTS.  plan_bytes below the header ->
 * W4A8_ERR_CAPACITY.
 */
int w4a8_grouped_gemm_planned(const uint8_t* A_fp8_dev, const float* a_scales_dev, int a_scale_layout,
                              const uint8_t* B_fp4_dev, const uint8_t* b_scales_e8m0_dev,
                              const int32_t* expert_offsets_dev, int E, int N, int K, const void* plan_dev,
                              size_t plan_bytes, uint16_t* C_bf16_dev, void* stream);

/*
 * w4a8_grouped_gemm_planned_noalloc -- w4a8_grouped_gemm_planned for callers
 * that cannot allocate device memory (code under HIP graph capture, tight
 * serving loops, harnesses that forbid hipMalloc): the plan is built by
 * w4a8_plan's kernel into the library's own device scratch and the planned
 * GEMM runs from it, so the caller passes only inputs and outputs.
 *
 * max_total_rows     an upper bound on offsets[E] (host value), as for
 *                    w4a8_plan_bytes.
 * The scratch is a fixed 4 MiB per device (a plan of up to 262,142 m-tiles),
 * held from the first call on that device until the process ends; a call
 * whose w4a8_plan_bytes(E, max_total_rows) exceeds it returns
 * W4A8_ERR_CAPACITY before any launch.  If the device's offsets[E] exceeds
 * max_total_rows and the plan then does not fit, its status word says so
 * and the GEMM writes nothing.  Every call on one device uses the same
 * scratch, which keeps the last call's plan: calls that overlap on one
 * device (different streams, or host threads) race and must be ordered by
 * the caller.  No allocation, no host synchronisation.  Other arguments,
 * numerics and limits as w4a8_grouped_gemm_planned.
 */
int w4a8_grouped_gemm_planned_noalloc(const uint8_t* A_fp8_dev, const float* a_scales_dev, int a_scale_layout,
                                      const uint8_t* B_fp4_dev, const uint8_t* b_scales_e8m0_dev,
                                      const int32_t* expert_offsets_dev, int E, int N, int K, int64_t max_total_rows,
                                      uint16_t* C_bf16_dev, void* stream);

/*
 * w4a8_grouped_gemm_swiglu -- the gate/up projection with the step between
 * the two projections fused into its epilogue (humming PR #129 "Results"
 * and PR #58 "H200 performance" time gate/up and down as a pair): the
 * grouped W4A8 GEMM of w4a8_grouped_gemm with N = 2I weight columns, then
 * h = silu(gate) * up and its E4M3 requantization exactly as
 * w4a8_swiglu_quant, but from the fp32 accumulators (no bf16 rounding of the
 * gate/up output, which is never written).
 *
 * A_fp8_dev, a_scales_dev, a_scale_layout, expert_offsets_dev, E, K: as
 *                    w4a8_grouped_gemm.
 * B13_fp4_dev        uint8 [E][2I][K/2] packed E2M1: columns 0 .. I-1 the
 *                    gate projection (w1), I .. 2I-1 the up projection (w3),
 *                    the concatenated [w1; w3] layout.  16-byte aligned.
 * b13_scales_e8m0_dev uint8 [E][2I][K/32] E8M0.  4-byte aligned.
 * A2_fp8_dev         out uint8 [R][I] E4M3FN codes of h.  16-byte aligned.
 * a2_scales_dev      out fp32 per (row, 128 columns of A2) in a2_scale_layout
 *                    (row-major [R][I/128] or M-major [I/128][R], R =
 *                    offsets[E]).  4-byte aligned.
 * Per row and 128-column group: s = amax|h| / 448 (1 if all zero), codes =
 * E4M3 round-to-nearest-even of clip(h * (1/s), +-448).  gate and up carry
 * the GEMM's fp32 accumulation error; h is evaluated as in
 * w4a8_swiglu_quant.  Only rows < R are written.  Every expert with rows
 * runs as MFMA tiles of 256 output columns (the small-M streaming schedule
 * is not used by this entry point).
 * Limits: as w4a8_grouped_gemm with N = 2I; I % 128 == 0; 2I * K/2 < 2^31.
 */
int w4a8_grouped_gemm_swiglu(const uint8_t* A_fp8_dev, const float* a_scales_dev, int a_scale_layout,
                             const uint8_t* B13_fp4_dev, const uint8_t* b13_scales_e8m0_dev,
                             const int32_t* expert_offsets_dev, int E, int I, int K, uint8_t* A2_fp8_dev,
                             float* a2_scales_dev, int a2_scale_layout, void* stream);

/*
 * w4a8_grouped_gemm_a16 -- the grouped-contiguous expert GEMM with 16-bit
 * activations and FP4 weights: the MXFP4 / NVFP4 A16 paths (humming PR #58,
 * "Summary": small-M FP4 paths exercised by MXFP4/NVFP4 A16; "H200
 * performance": BF16 FP4 expert-GEMM sweeps, gate/up and down):
 *
 *   C[r, n] = bf16_rne( gs[e] * sum_k A[r, k] * e2m1(B[e, n, k]) * s(e, n, k) )
 *
 * A_bf16_dev         bf16 [R][K] activations, rows grouped by expert as for
 *                    w4a8_grouped_gemm.  16-byte aligned.
 * B_fp4_dev          uint8 [E][N][K/2] packed E2M1 (element 2j in the low
 *                    nibble).  16-byte aligned.
 * b_scales_dev       W4A8_WSCALE_MX: uint8 [E][N][K/32] E8M0 codes, s =
 *                    2^(code-127) (0xFF NaN); W4A8_WSCALE_NV: uint8
 *                    [E][N][K/16] E4M3FN codes, s their value (0x7F/0xFF
 *                    NaN).  4-byte aligned.
 * b_scale_format     W4A8_WSCALE_MX or W4A8_WSCALE_NV (W4A8_ERR_LAYOUT
 *                    otherwise).
 * expert_scales_dev  fp32 [E] per-expert scales gs (the NVFP4 tensor scale of
 *                    each expert's weights), or NULL for all ones.  4-byte
 *                    aligned.
 * expert_offsets_dev int32 [E+1] as for w4a8_grouped_gemm; offsets that do
 *                    not start at 0 or decrease make the kernel write nothing.
 * C_bf16_dev         out bf16 [R][N]; only rows < R are written.  16-byte
 *                    aligned.
 * Numerics: the FP4 weights are converted to bf16 times their scale (exact
 * for scales whose products stay inside fp32's normal range) and summed on
 * the matrix core in fp32 (one rounding per 16 K); the result is multiplied
 * by gs[e] in fp32 and rounded once to bf16 (round to nearest even).  NaN
 * scale codes make their columns NaN for the expert's rows.
 * Limits: 1 <= E <= W4A8_MAX_PREP_EXPERTS; K % 128 == 0, 128 <= K <=
 * W4A8_MAX_K; N % 16 == 0, 16 <= N <= W4A8_MAX_N; E * ceil(N/64) < 2^31.
 * Every expert with rows is served, in passes of 64 rows over its weights
 * (the schedule is tuned for small M: larger experts re-read their weights
 * once per 64 rows).  No allocation, no host synchronisation.
 */
int w4a8_grouped_gemm_a16(const uint16_t* A_bf16_dev, const uint8_t* B_fp4_dev, const uint8_t* b_scales_dev,
                          int b_scale_format, const float* expert_scales_dev, const int32_t* expert_offsets_dev,
                          int E, int N, int K, uint16_t* C_bf16_dev, void* stream);

/*
 * w4a8_plan_params -- the plan rule's constants, written to out_host[0..n-1]
 * in this order: GRAN (m granularity), S_MAX, T_MAX, TN_STREAM (n granularity
 * of streaming work), TN_MFMA (n width of an MFMA work item), plan header
 * words, words per tile.  Returns the number of constants available (7) or
 * -W4A8_ERR_NULL if out_host is NULL.
 */
int w4a8_plan_params(int32_t* out_host, int n);

/* Human-readable name of a status code (static string). */
const char* w4a8_status_string(int status);

/* Per-thread detail of the last non-OK return of this thread ("" if none). */
const char* w4a8_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* W4A8_H */
