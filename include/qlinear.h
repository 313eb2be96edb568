/*
 * libqlinear -- weight-quantized linear layer out = x @ dequant(W)^T on AMD
 * Instinct MI355X (gfx950), as hand-written HIP kernels behind a C ABI.
 *
 * Conventions shared by every call
 * --------------------------------
 * - Tensors are dense, row-major and contiguous; every pointer is a DEVICE
 *   pointer on the device that is current in the calling thread, unless the
 *   comment says otherwise.  Activations x are [M, K], weights W are [N, K]
 *   (the output feature n owns row n, K contiguous), outputs are [M, N].
 * - Storage formats: float8_e4m3fn = OCP E4M3 "FN" (bias 7, max 448, NaN only
 *   at 0x7F/0xFF, no inf); bfloat16 = upper half of an IEEE binary32; NVFP4 =
 *   two E2M1 codes per byte (even k in the low nibble) plus one E4M3 scale per
 *   16 consecutive k of a row.
 * - `stream` is a hipStream_t passed as an opaque pointer (NULL = the null
 *   stream).  Every call only enqueues work on it and returns; nothing
 *   synchronises.  Outputs are valid once the stream has reached the work.
 * - Ownership: the caller owns every buffer, including the optional
 *   float32 workspace of the *_ws calls (split-K partial sums; size from
 *   qlinear_gemm_workspace_size).  The library allocates and frees nothing
 *   and keeps no pointer past the call; its state is a per-device cache of
 *   the device's properties (architecture, CU count) and the fixed 8 MiB
 *   device buffer that only qlinear_fp8_gemm_noalloc uses.  A call's kernel choice, and so its summation order and
 *   output bits, depends only on its arguments (shapes, operand alignment,
 *   the workspace size given) and the device's CU count, never on earlier
 *   calls.  Calls without a workspace run whole-K tiles.
 * - Errors: the return value (a qlinear_status) is the only error channel.
 *   Arguments are validated before anything is enqueued; on an error nothing
 *   is written.  Device-side contents (offsets, ids) are not validated by the
 *   host; the kernels guard them as documented per call.
 * - Inputs and outputs must not alias.  Calls are stateless and
 *   thread-safe; two calls that run at once (different streams) need
 *   different output buffers and, if they take one, different workspaces.
 * - Accumulation is float32 (int32 for int8 x int8); float outputs are
 *   rounded once, to nearest even.
 *
 * The operations follow the documentation pages of the Mojo `linalg.matmul.
 * gpu.apple` kernels: "fp8_gemv", "fp4_matmul", "Matmul2dFp8" and
 * "int8_matmul".  Those pages describe Apple-M5 kernels; only what they
 * compute is taken from them, not how.
 */
#ifndef QLINEAR_H
#define QLINEAR_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define QLINEAR_ABI_VERSION 2

typedef enum qlinear_status {
  QLINEAR_OK = 0,
  QLINEAR_ERR_INVALID_ARG = 1,  /* null pointer, size <= 0, bad dtype, bad layout */
  QLINEAR_ERR_UNSUPPORTED = 2,  /* device is not gfx950, or a forced kernel family cannot run the call */
  QLINEAR_ERR_DEVICE = 3,       /* no usable HIP device / device query failed */
  QLINEAR_ERR_LAUNCH = 4,       /* a kernel launch reported an error */
  QLINEAR_ERR_SCRATCH_LIMIT = 5 /* qlinear_fp8_gemm_noalloc: the shape needs more split-K
                                   scratch than the library's fixed buffer holds */
} qlinear_status;

typedef enum qlinear_dtype {
  QLINEAR_F32 = 0,
  QLINEAR_BF16 = 1,
  QLINEAR_I32 = 2
} qlinear_dtype;

/* Kernel family for the *_path calls; AUTO is what the plain call does. */
typedef enum qlinear_path {
  QLINEAR_PATH_AUTO = 0,
  QLINEAR_PATH_GEMV = 1,    /* vector-ALU GEMV, 1 <= M <= 4                         */
  QLINEAR_PATH_SKINNY = 2,  /* matrix-core skinny GEMM, 1 <= M <= 16                */
  QLINEAR_PATH_TILED = 3,   /* LDS-tiled matrix-core GEMM, any M                     */
  QLINEAR_PATH_SPLITK = 4   /* split-K skinny GEMM, M <= 16, K % 64 == 0, aligned    */
} qlinear_path;

/* Weight format of qlinear_gemm_workspace_size. */
typedef enum qlinear_weight_format {
  QLINEAR_WEIGHT_FP8 = 0,    /* qlinear_fp8_gemm_ws   */
  QLINEAR_WEIGHT_NVFP4 = 1,  /* qlinear_nvfp4_gemm_ws */
  QLINEAR_WEIGHT_BF16 = 2    /* qlinear_bf16_gemm_ws  */
} qlinear_weight_format;

/* Activation of a fused epilogue. */
typedef enum qlinear_activation {
  QLINEAR_ACT_NONE = 0,
  QLINEAR_ACT_RELU = 1,       /* max(v, 0)                                           */
  QLINEAR_ACT_SILU = 2,       /* v / (1 + exp(-v))                                   */
  QLINEAR_ACT_GELU_TANH = 3   /* 0.5 v (1 + tanh(sqrt(2/pi) (v + 0.044715 v^3)))     */
} qlinear_activation;

/*
 * Fused epilogue of the *_epilogue calls: page "Matmul2dFp8" ("Parameters",
 * elementwise_lambda_fn: an optional element-wise function of the output
 * element's (row, col) coordinates and value, fused into the store).  A C
 * ABI cannot take a lambda, so this is a fixed menu of element-wise steps,
 * applied in float32 to output element (m, n) after alpha and before the
 * single rounding to the output type:
 *     v = alpha * acc
 *     v = v * row_scale[m]            (row_scale: float32 [M], or NULL)
 *     v = v * col_scale[n]            (col_scale: float32 [N], or NULL)
 *     v = v + bias[n]                 (bias: bfloat16 [N], or NULL)
 *     v = activation(v)
 *     v = v + residual[m * residual_ld + n]   (residual: [M, residual_ld] of
 *                                      residual_dtype F32 or BF16, or NULL)
 * The residual may be the output buffer itself (same type, residual_ld = N):
 * each element is read before it is written, by the same thread.  All
 * pointers are device pointers, read only, owned by the caller.  An invalid
 * activation, a residual_ld below N or a misaligned pointer gives
 * QLINEAR_ERR_INVALID_ARG.  A NULL descriptor (or one with every pointer
 * NULL and no activation) is the plain call.
 */
typedef struct qlinear_epilogue {
  const float* row_scale;
  const float* col_scale;
  const void* bias;
  const void* residual;
  int64_t residual_ld;
  int residual_dtype;
  int activation;
} qlinear_epilogue;

/* Version of this ABI (QLINEAR_ABI_VERSION of the build). */
int qlinear_abi_version(void);

/* Static, human-readable name of a status code ("unknown status" otherwise). */
const char* qlinear_status_string(int status);

/*
 * W8A16 GEMV (batch-1 decode), page "fp8_gemv" (summary, "Structure",
 * "Scale contract"; enqueue_apple_fp8_gemv):
 *     out[n] = alpha * sum_k x[k] * dec_e4m3(w[n, k])
 * w: float8_e4m3fn [N, K]; x: bfloat16 [K]; out: [N] of out_dtype (F32 or
 * BF16).  alpha = 1 returns the raw product; any other alpha is the
 * per-tensor weight_scale folded in float32 before the single output
 * rounding.  Any K >= 1 and any alignment are accepted.  With x 16-byte
 * aligned the weight is read with 16-byte loads at any K and weight
 * alignment (rows that start off a 16-byte boundary, e.g. K = 2050, are
 * shifted into place in registers; the loads stay inside the 16-byte blocks
 * that hold the weight's bytes); an unaligned x takes a byte-load kernel.
 */
int qlinear_fp8_gemv(const void* w, const void* x, void* out, int out_dtype,
                     int64_t N, int64_t K, float alpha, void* stream);

/*
 * W8A16 matmul at any M >= 1, page "fp8_gemv" (enqueue_apple_fp8_matmul) and
 * page "Matmul2dFp8" (W8A16 GEMM, c_type = fp32/bf16, fp32 accumulation):
 *     out[m, n] = alpha * sum_k x[m, k] * dec_e4m3(w[n, k])
 * w: float8_e4m3fn [N, K]; x: bfloat16 [M, K]; out: [M, N] of out_dtype (F32
 * or BF16).  Chooses the GEMV (M = 1), skinny (M <= 16) or tiled kernel.
 */
int qlinear_fp8_gemm(const void* w, const void* x, void* out, int out_dtype,
                     int64_t M, int64_t N, int64_t K, float alpha, void* stream);

/*
 * As qlinear_fp8_gemm, with the kernel family forced (tests compare the
 * families with each other).  A family that cannot take the given M returns
 * QLINEAR_ERR_INVALID_ARG.  QLINEAR_PATH_SPLITK (K split over blocks, float32
 * partial planes added by a second kernel in a fixed order) needs a
 * workspace, so through this call (which has none) it returns
 * QLINEAR_ERR_UNSUPPORTED and launches nothing; see qlinear_fp8_gemm_ws.
 */
int qlinear_fp8_gemm_path(const void* w, const void* x, void* out, int out_dtype,
                          int64_t M, int64_t N, int64_t K, float alpha, int path,
                          void* stream);

/*
 * FP8 weight materialisation, page "fp8_gemv" (enqueue_fp8_materialize):
 *     out[n, k] = dec_e4m3(w[n, k])     (exact in F32 and in BF16)
 * w: float8_e4m3fn [N, K]; out: [N, K] of out_dtype (F32 or BF16).  NaN codes
 * give a quiet NaN.  Uses the same decoder as the matmul kernels.
 */
int qlinear_fp8_materialize(const void* w, void* out, int out_dtype,
                            int64_t N, int64_t K, void* stream);

/*
 * Grouped (MoE) W8A16 matmul, page "Matmul2dFp8" (run_grouped): for every
 * group z in 0 .. num_groups-1, with start = a_offsets[z] and
 * end = a_offsets[z+1],
 *     out[r, n] = sum_k x[r, k] * dec_e4m3(w[expert_ids[z], n, k])
 * for rows r in [start, end).  The result is raw (the per-expert scale is
 * applied by the caller, as on the page).  expert_ids[z] == -1 marks an
 * inactive group, whose rows are written as zeros; an empty group writes
 * nothing; rows that no group covers are left untouched.
 * w: float8_e4m3fn [num_experts, N, K]; x: bfloat16 [T, K]; out: [T, N] of
 * out_dtype (F32 or BF16); a_offsets: uint32 [num_groups + 1] and
 * expert_ids: int32 [num_groups], both in DEVICE memory and not read by the
 * host.  Offsets must be non-decreasing for the result to be defined
 * (overlapping groups race); the kernel still never reads or writes out of
 * bounds: offsets are clipped to T, a group whose end does not exceed its
 * start is empty, and any id outside 0 .. num_experts-1 is treated as -1.
 * max_tokens_per_group (>= 0) only sizes the launch grid; groups larger
 * than it are still computed in full.  1 <= num_groups <= 65535.
 */
int qlinear_fp8_grouped_gemm(const void* w, const void* x, const uint32_t* a_offsets,
                             const int32_t* expert_ids, void* out, int out_dtype,
                             int64_t num_groups, int64_t max_tokens_per_group,
                             int64_t num_experts, int64_t T, int64_t N, int64_t K,
                             void* stream);

/*
 * W4A16 NVFP4 matmul, page "fp4_matmul" (enqueue_apple_fp4_matmul):
 *     out[m, n] = alpha * sum_k x[m, k] * D[n, k],
 *     D[n, k] = e2m1(code(n, k)) * dec_e4m3(w_scale[n, k / 16])
 * w_packed: uint8 [N, K/2], code(n, 2j) in the low nibble of byte j and
 * code(n, 2j+1) in the high nibble; w_scale: float8_e4m3fn [N, K/16];
 * x: bfloat16 [M, K]; out: [M, N] of out_dtype (F32 or BF16).  K % 16 == 0.
 * alpha is the per-tensor global scale (weight_scale_2; 1 = raw), applied in
 * float32 before the single output rounding.  M <= 4 runs on the vector ALU;
 * larger M stages the packed codes and block scales in LDS, and each lane
 * decodes its own matrix-core operand fragment to bfloat16 in registers.
 */
int qlinear_nvfp4_gemm(const void* w_packed, const void* w_scale, const void* x, void* out,
                       int out_dtype, int64_t M, int64_t N, int64_t K, float alpha,
                       void* stream);

/*
 * FP8 activation quantisation for W8A8, page "fp8_gemv" ("Scale contract":
 * the checkpoint's per-tensor input_scale cancels only while the activation
 * stays bf16; with fp8 activations it is the quantisation step):
 *     q[m, k] = E4M3(clamp(x[m, k] / input_scale, -448, 448))
 * one IEEE float32 division, round to nearest even, float8_e4m3fn codes.
 * x: bfloat16 [M, K] (2-byte aligned); q: uint8 [M, K]; input_scale: finite
 * and > 0, else QLINEAR_ERR_INVALID_ARG.  Non-finite activations are outside
 * the contract.
 */
int qlinear_fp8_quantize_act(const void* x, void* q, float input_scale, int64_t M, int64_t K,
                             void* stream);

/*
 * FP8 W8A8 matmul, page "fp8_gemv" with fp8 activations:
 *     out[m, n] = alpha * sum_k dec_e4m3(xq[m, k]) * dec_e4m3(w[n, k])
 * alpha = input_scale * weight_scale, applied in float32 before the single
 * output rounding; every product is exact and accumulation is float32.
 * xq: float8_e4m3fn [M, K] (as made by qlinear_fp8_quantize_act); w:
 * float8_e4m3fn [N, K]; out: [M, N] of out_dtype (F32 or BF16).  K % 64 == 0
 * with 16-byte aligned operands under 4 GiB runs on the gfx950 fp8 matrix
 * cores; any other shape takes a slow element-wise kernel.
 */
int qlinear_fp8_w8a8_gemm(const void* xq, const void* w, void* out, int out_dtype,
                          int64_t M, int64_t N, int64_t K, float alpha, void* stream);

/*
 * Grouped (MoE) W4A16 NVFP4 matmul: the ragged addressing of page
 * "Matmul2dFp8" (run_grouped) with the weight format of page "fp4_matmul".
 * For every group z, rows r in [a_offsets[z], a_offsets[z+1]):
 *     out[r, n] = sum_k x[r, k] * D_e[n, k],   e = expert_ids[z],
 *     D_e[n, k] = e2m1(code_e(n, k)) * dec_e4m3(w_scale[e, n, k / 16])
 * w_packed: uint8 [num_experts, N, K/2] (nibble order as qlinear_nvfp4_gemm);
 * w_scale: float8_e4m3fn [num_experts, N, K/16]; x: bfloat16 [T, K];
 * out: [T, N] of out_dtype (F32 or BF16); K % 16 == 0.  The result is raw:
 * each expert's global scale (weight_scale_2) is applied by the caller.
 * a_offsets, expert_ids, num_groups, max_tokens_per_group, inactive / empty
 * groups, untouched rows, precondition and bounds behaviour: exactly as
 * qlinear_fp8_grouped_gemm.  Returns QLINEAR_ERR_INVALID_ARG for a null
 * pointer, a non-positive size, K % 16 != 0 or a misaligned x / out /
 * a_offsets / expert_ids; nothing is written then.
 */
int qlinear_nvfp4_grouped_gemm(const void* w_packed, const void* w_scale, const void* x,
                               const uint32_t* a_offsets, const int32_t* expert_ids, void* out,
                               int out_dtype, int64_t num_groups, int64_t max_tokens_per_group,
                               int64_t num_experts, int64_t T, int64_t N, int64_t K,
                               void* stream);

/* As qlinear_nvfp4_gemm with the kernel family forced: QLINEAR_PATH_GEMV
 * (M <= 4) or QLINEAR_PATH_TILED (any M); others are QLINEAR_ERR_INVALID_ARG. */
int qlinear_nvfp4_gemm_path(const void* w_packed, const void* w_scale, const void* x,
                            void* out, int out_dtype, int64_t M, int64_t N, int64_t K,
                            float alpha, int path, void* stream);

/*
 * NVFP4 dequantisation, page "fp4_matmul" (summary: the packed weight is
 * dequantised to bf16): out[n, k] = D[n, k] as above, exact in BF16 and F32.
 * Uses the same decoders as the matmul kernels (BF16: the matrix-core tile
 * decoder, F32: the vector-ALU decoder).  K % 16 == 0.
 */
int qlinear_nvfp4_dequant(const void* w_packed, const void* w_scale, void* out, int out_dtype,
                          int64_t N, int64_t K, void* stream);

/*
 * Per-row symmetric int8 quantisation of a bfloat16 activation, page
 * "int8_matmul" ("Quantization (W8A8)"; enqueue_apple_int8_quantize_activation):
 *     a_scale[m] = absmax_k |x[m, k]| / 127      (IEEE float32 division)
 *     q[m, k]    = clamp(round_half_even(x[m, k] / a_scale[m]), -127, 127)
 * with IEEE float32 division per element; an all-zero row gives a_scale 0
 * and zero codes; -128 is never produced.  Non-finite inputs follow the
 * same formulas: a row holding a NaN gets a_scale NaN, one holding an
 * infinity (and no NaN) a_scale +inf, and either gets zero codes, so its
 * dequantised outputs are NaN.  x: bfloat16 [M, K]; q: int8 [M, K];
 * a_scale: float32 [M].  Reads x once per row when K <= 4096.
 */
int qlinear_int8_quantize_act(const void* x, void* q, float* a_scale, int64_t M, int64_t K,
                              void* stream);

/*
 * W8A8 int8 matmul with the dequantising epilogue, page "int8_matmul"
 * (enqueue_apple_int8_matmul, Int8DequantWriter):
 *     acc[m, n] = sum_k a[m, k] * b[n, k]                       (exact int32)
 *     out[m, n] = acc[m, n] * a_scale[m] * b_scale[n] + bias[n]   (float32, one rounding to out)
 * a: int8 [M, K]; b: int8 [N, K] (row n = output channel n); a_scale: float32
 * [M]; b_scale: float32 [N]; bias: bfloat16 [N] or NULL (no bias).
 * out_dtype BF16 or F32 gives the dequantised result; I32 stores the raw
 * accumulators (a_scale, b_scale and bias are then ignored and may be NULL).
 * K <= 133144 so that no int32 accumulator can overflow.
 */
int qlinear_int8_gemm(const void* a, const void* b, const float* a_scale, const float* b_scale,
                      const void* bias, void* out, int out_dtype, int64_t M, int64_t N,
                      int64_t K, void* stream);

/*
 * Dense bf16 control matmul: the bf16 weight path that page "fp8_gemv"
 * ("WHY it wins at decode") compares W8A16 against (2 bytes per weight
 * against 1) and the dense GEMM that page "Matmul2dFp8" (summary) mirrors:
 *     out[m, n] = alpha * sum_k x[m, k] * w[n, k]
 * w: bfloat16 [N, K]; x: bfloat16 [M, K]; out: [M, N] of out_dtype (F32 or
 * BF16); alpha applied in float32 before the single output rounding;
 * float32 accumulation of exact products.  Any K >= 1 and alignment (both
 * operands 2-byte aligned); K % 8 == 0 with 16-byte aligned operands takes
 * the wide-load kernels.  The kernel families are those of
 * qlinear_fp8_gemm: GEMV (M <= 4), skinny (M <= 16), tiled (any M; with a
 * workspace, qlinear_bf16_gemm_ws, small-M tiles split K).
 */
int qlinear_bf16_gemm(const void* w, const void* x, void* out, int out_dtype,
                      int64_t M, int64_t N, int64_t K, float alpha, void* stream);

/* As qlinear_bf16_gemm with the kernel family forced (see qlinear_fp8_gemm_path). */
int qlinear_bf16_gemm_path(const void* w, const void* x, void* out, int out_dtype,
                           int64_t M, int64_t N, int64_t K, float alpha, int path,
                           void* stream);

/*
 * qlinear_fp8_gemm / qlinear_nvfp4_gemm / qlinear_bf16_gemm with a fused
 * epilogue (qlinear_epilogue; NULL = the plain call).  Same operands, kernel
 * choice (no workspace) and errors as the plain calls; the _path variant
 * forces the kernel family as qlinear_fp8_gemm_path does.
 */
int qlinear_fp8_gemm_epilogue(const void* w, const void* x, void* out, int out_dtype,
                              int64_t M, int64_t N, int64_t K, float alpha,
                              const qlinear_epilogue* epilogue, void* stream);
int qlinear_fp8_gemm_epilogue_path(const void* w, const void* x, void* out, int out_dtype,
                                   int64_t M, int64_t N, int64_t K, float alpha,
                                   const qlinear_epilogue* epilogue, int path, void* stream);
int qlinear_nvfp4_gemm_epilogue(const void* w_packed, const void* w_scale, const void* x,
                                void* out, int out_dtype, int64_t M, int64_t N, int64_t K,
                                float alpha, const qlinear_epilogue* epilogue, void* stream);
int qlinear_bf16_gemm_epilogue(const void* w, const void* x, void* out, int out_dtype,
                               int64_t M, int64_t N, int64_t K, float alpha,
                               const qlinear_epilogue* epilogue, void* stream);

/*
 * Split-K workspace size, pages "Matmul2dFp8" (the tiled W8A16 GEMM) and
 * "fp4_matmul" (the NVFP4 GEMM): with few output tiles (small M) the tiled
 * and skinny matrix-core kernels split K over several blocks, each writing
 * a float32 partial-sum plane [M, N] into a caller-provided workspace, and a
 * second kernel adds the planes in a fixed order.  This only changes the
 * order of the float32 additions, never what is computed.
 * *bytes receives the workspace size with which the *_ws call of
 * `weight_format` (a qlinear_weight_format) and `path` (a qlinear_path)
 * takes its fastest kernel for (M, N, K) on the current device, assuming
 * 16-byte aligned operands; 0 means the call takes no workspace there.  A
 * smaller workspace is not an error: the call then uses fewer K slices or
 * whole-K tiles.  Reads no device memory and launches nothing.  Returns
 * QLINEAR_ERR_INVALID_ARG for a null `bytes`, a non-positive size, an unknown
 * format or path, or NVFP4 K % 16 != 0.
 */
int qlinear_gemm_workspace_size(int weight_format, int path, int64_t M, int64_t N, int64_t K,
                                int64_t* bytes);

/*
 * The W8A16, NVFP4 and bf16 matmuls with every option: a fused epilogue
 * (NULL = none), a kernel family (`path`, QLINEAR_PATH_AUTO = the automatic
 * choice) and a caller-owned split-K workspace: `workspace` is device memory
 * on the current device, 16-byte aligned, of `workspace_bytes` bytes (NULL
 * with 0 = none).  Its contents on entry do not matter and on return are
 * unspecified; it must not be in use by another call that runs at the same
 * time.  Operands, results and errors otherwise exactly as
 * qlinear_fp8_gemm(_epilogue_path), qlinear_nvfp4_gemm(_epilogue) and
 * qlinear_bf16_gemm(_epilogue); the result bits depend only on the
 * arguments.  A misaligned workspace, workspace_bytes < 0, or a NULL
 * workspace with workspace_bytes > 0 gives QLINEAR_ERR_INVALID_ARG.
 * QLINEAR_PATH_SPLITK (qlinear_fp8_gemm_ws only) returns
 * QLINEAR_ERR_UNSUPPORTED, launching nothing, when the shape leaves fewer
 * than two K slices of 256 values or the partial planes exceed the
 * workspace.
 */
int qlinear_fp8_gemm_ws(const void* w, const void* x, void* out, int out_dtype,
                        int64_t M, int64_t N, int64_t K, float alpha,
                        const qlinear_epilogue* epilogue, int path, void* workspace,
                        int64_t workspace_bytes, void* stream);
int qlinear_nvfp4_gemm_ws(const void* w_packed, const void* w_scale, const void* x, void* out,
                          int out_dtype, int64_t M, int64_t N, int64_t K, float alpha,
                          const qlinear_epilogue* epilogue, int path, void* workspace,
                          int64_t workspace_bytes, void* stream);
int qlinear_bf16_gemm_ws(const void* w, const void* x, void* out, int out_dtype,
                         int64_t M, int64_t N, int64_t K, float alpha,
                         const qlinear_epilogue* epilogue, int path, void* workspace,
                         int64_t workspace_bytes, void* stream);

/*
 * qlinear_fp8_gemm_ws for callers that cannot allocate device memory (code
 * under graph capture, tight serving loops, hosts that forbid allocation):
 * the split-K partial sums go to a fixed 8 MiB buffer of the library on the
 * current device (each device has its own copy, held from the library's load
 * until the process ends) instead of a caller-given workspace.  The call
 * allocates nothing; the caller still passes inputs and outputs.  Kernels,
 * results and errors are those of qlinear_fp8_gemm_ws with a workspace of
 * the size qlinear_gemm_workspace_size gives (bit-identical output).  A
 * shape whose workspace size exceeds 8 MiB returns QLINEAR_ERR_SCRATCH_LIMIT
 * and launches nothing.  The buffer is shared by every call on a device and
 * keeps the last call's partial sums: two calls of this function that can
 * run at the same time on one device (different streams, host threads
 * without stream ordering) race on it and give undefined results.
 */
int qlinear_fp8_gemm_noalloc(const void* w, const void* x, void* out, int out_dtype,
                             int64_t M, int64_t N, int64_t K, float alpha,
                             const qlinear_epilogue* epilogue, int path, void* stream);

/*
 * Grouped matmuls with the per-expert weight scale folded in: page
 * "Matmul2dFp8" (run_grouped produces the raw product; the graph then
 * multiplies each expert's rows by that expert's weight_scale).  Rows of
 * group z are multiplied by expert_scale[expert_ids[z]] (float32
 * [num_experts], device memory; NULL = raw) in float32 before the single
 * output rounding; inactive groups still write zeros.  Everything else is
 * exactly qlinear_fp8_grouped_gemm / qlinear_nvfp4_grouped_gemm.
 */
int qlinear_fp8_grouped_gemm_scaled(const void* w, const void* x, const uint32_t* a_offsets,
                                    const int32_t* expert_ids, const float* expert_scale,
                                    void* out, int out_dtype, int64_t num_groups,
                                    int64_t max_tokens_per_group, int64_t num_experts,
                                    int64_t T, int64_t N, int64_t K, void* stream);
int qlinear_nvfp4_grouped_gemm_scaled(const void* w_packed, const void* w_scale, const void* x,
                                      const uint32_t* a_offsets, const int32_t* expert_ids,
                                      const float* expert_scale, void* out, int out_dtype,
                                      int64_t num_groups, int64_t max_tokens_per_group,
                                      int64_t num_experts, int64_t T, int64_t N, int64_t K,
                                      void* stream);

/*
 * Grouped (MoE) W8A8 int8 matmul: the ragged addressing of page
 * "Matmul2dFp8" (run_grouped) over the body of page "int8_matmul"
 * ("Quantization (W8A8)"; Int8DequantWriter).  For every group z, rows r in
 * [a_offsets[z], a_offsets[z+1]) and e = expert_ids[z]:
 *     acc[r, n] = sum_k a[r, k] * b[e, n, k]                     (exact int32)
 *     out[r, n] = acc[r, n] * a_scale[r] * b_scale[e, n] + bias[e, n]
 * a: int8 [T, K] and a_scale: float32 [T] (qlinear_int8_quantize_act over the
 * T rows); b: int8 [num_experts, N, K]; b_scale: float32 [num_experts, N];
 * bias: bfloat16 [num_experts, N] or NULL; out: [T, N] of out_dtype (BF16,
 * F32, or I32 for the raw accumulators, which ignores the scales and bias).
 * a_offsets, expert_ids, num_groups, max_tokens_per_group, inactive / empty
 * groups (zeros / nothing), untouched rows, preconditions and bounds
 * behaviour: exactly as qlinear_fp8_grouped_gemm.  K <= 133144 (no int32
 * overflow).  K % 64 == 0 with 16-byte aligned a and b runs the LDS-tiled
 * matrix-core kernel; anything else a register-staged one.  Returns
 * QLINEAR_ERR_INVALID_ARG for a null pointer, a non-positive size, a bad
 * out_dtype or a misaligned pointer; nothing is written then.
 */
int qlinear_int8_grouped_gemm(const void* a, const void* b, const float* a_scale,
                              const float* b_scale, const void* bias, const uint32_t* a_offsets,
                              const int32_t* expert_ids, void* out, int out_dtype,
                              int64_t num_groups, int64_t max_tokens_per_group,
                              int64_t num_experts, int64_t T, int64_t N, int64_t K, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* QLINEAR_H */
