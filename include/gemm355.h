/*
 * gemm355 -- dense GEMM for AMD Instinct MI355X (gfx950), C ABI.
 *
 *   C = act( alpha * (scale_a[m] * scale_b[n]) * sum_k A[m,k] B[k,n] + beta * C + bias[n] )
 *
 * The operation is the general matrix multiply C = alpha*A*B + beta*C of the
 * first DeepGEMM page (sec. 1.1: A is MxK, B is KxN, C is MxN), with 16-bit
 * inputs accumulated in FP32 (same page, sec. 3.1), and the epilogue fused
 * before the store: bias, then activation, then the output cast (same page,
 * sec. 6.1). The FP8 entry point takes E4M3 inputs with one FP32 scale per
 * row of A (per token) and one per column of B (per channel), applied after
 * accumulation and before the store (DeepGEMM: FP8 precision Tensor Core GEMM
 * optimisation, sec. 1.2 and 3.2). Like that page's interface (sec. 5.1) the
 * calls take device pointers, sizes, a scale description, an optional
 * workspace with a size query, and a stream.
 *
 * Conventions common to every entry point
 * ---------------------------------------
 * - All matrix, vector and workspace pointers are DEVICE pointers owned by the
 *   caller. The library never allocates, frees or synchronises, and apart
 *   from the scratch array of gemm_bf16_noalloc keeps no mutable global
 *   state: the other calls are reentrant and may run on any stream.
 * - Operand layouts (per operand, gemm_layout):
 *     A ROW: a(m,k) = A[m*lda + k], lda >= K      A COL: a(m,k) = A[k*lda + m], lda >= M
 *     B ROW: b(k,n) = B[k*ldb + n], ldb >= N      B COL: b(k,n) = B[n*ldb + k], ldb >= K
 *   "K-major" means A ROW and B COL. C is always row-major: C[m*ldc + n],
 *   ldc >= N. C is read (when beta != 0) and written with dtype c_dtype.
 * - Element types: BF16 (1-8-7, stored as uint16), OCP FP8 E4M3FN (1-4-3,
 *   bias 7, max 448, stored as uint8), FP32. bias is BF16[N] (NULL for none).
 *   scale_a is FP32[M] and scale_b FP32[N], contiguous (stride 1).
 * - Rounding: FP32 accumulation; epilogue arithmetic in FP32; the BF16 output
 *   cast rounds to nearest even.
 * - Activations: ReLU max(z,0); GELU_ERF z*Phi(z) = 0.5 z (1 + erf(z/sqrt 2));
 *   GELU_TANH 0.5 z (1 + tanh(sqrt(2/pi) (z + 0.044715 z^3))). Both GELUs are
 *   evaluated in forms without cancellation, so they keep their relative
 *   accuracy for large negative z: within 2^-19 relative (+1 ulp) of the exact
 *   value for FP32 output, within one BF16 ulp for BF16 output.
 * - Quick returns: M == 0 or N == 0 returns GEMM_OK and launches nothing.
 *   K == 0 gives C = act(beta*C + bias). beta == 0 means C is not read (NaN in
 *   C is ignored).
 * - Errors: every argument check happens before anything is enqueued; on a
 *   status other than GEMM_OK and GEMM_ERR_HIP nothing was launched and no
 *   memory was touched. GEMM_ERR_HIP means the HIP runtime rejected one of the
 *   call's launches; a call of two launches (a split-K GEMM and its
 *   reduction) whose second launch fails has already enqueued the first, which
 *   writes only the workspace. Before launching, the call consumes any HIP
 *   error that an earlier call on the same thread left pending (hipGetLastError),
 *   so GEMM_ERR_HIP never reports someone else's error. Faults inside a kernel
 *   surface at the caller's next synchronisation. Nothing is printed and
 *   nothing aborts.
 * - Aliasing: C must not overlap A, B, bias, the scales or the workspace.
 * - Asynchrony: work is enqueued on `stream` (a hipStream_t; NULL = the null
 *   stream) and the call returns without waiting.
 * - Determinism: for a given (shape, layouts, dtype) the result is bitwise
 *   reproducible run to run (the split-K reduction sums partials in a fixed
 *   order; no floating-point atomics).
 */
#ifndef GEMM355_H
#define GEMM355_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  GEMM_OK = 0,
  GEMM_ERR_NULL_POINTER = 1,       /* a required pointer is NULL */
  GEMM_ERR_BAD_DIM = 2,            /* M, N or K negative, or too large for 32-bit tile indexing */
  GEMM_ERR_BAD_LD = 3,             /* a leading dimension is smaller than its operand's row extent */
  GEMM_ERR_BAD_ENUM = 4,           /* unknown layout, output dtype or activation */
  GEMM_ERR_UNSUPPORTED = 5,        /* a valid combination this library does not implement */
  GEMM_ERR_WORKSPACE_TOO_SMALL = 6,/* workspace_bytes < gemm_workspace_size(...) */
  GEMM_ERR_HIP = 7                 /* the HIP runtime rejected the launch */
} gemm_status;

typedef enum { GEMM_ROW_MAJOR = 0, GEMM_COL_MAJOR = 1 } gemm_layout;
typedef enum { GEMM_OUT_F32 = 0, GEMM_OUT_BF16 = 1 } gemm_out_dtype;
typedef enum {
  GEMM_ACT_NONE = 0,
  GEMM_ACT_RELU = 1,
  GEMM_ACT_GELU_ERF = 2,
  GEMM_ACT_GELU_TANH = 3
} gemm_act;

/*
 * BF16 x BF16 -> FP32 accumulate -> epilogue -> FP32 or BF16 C.
 * A: BF16, logical MxK, layout_a / lda as above. B: BF16, logical KxN.
 * All four layout combinations are accepted.
 * workspace: device scratch of at least gemm_workspace_size(M, N, K, 0) bytes
 * (may be NULL when that size is 0). Its contents on entry do not matter.
 */
gemm_status gemm_bf16(int64_t M, int64_t N, int64_t K, float alpha,
                      const void* A, int64_t lda, gemm_layout layout_a,
                      const void* B, int64_t ldb, gemm_layout layout_b,
                      float beta, void* C, int64_t ldc, gemm_out_dtype c_dtype,
                      const void* bias, gemm_act act,
                      void* workspace, size_t workspace_bytes, void* stream);

/*
 * gemm_bf16 for callers that cannot allocate device memory (code under HIP
 * graph capture, tight serving loops, harnesses that forbid hipMalloc): the
 * same operation, arguments and kernels, without a workspace argument. Split-K
 * partials go to a scratch array of 32 MiB that the library holds in every
 * GPU's memory from the module load until the process ends; the call
 * allocates and frees nothing. A shape whose plan needs more workspace than
 * that returns GEMM_ERR_WORKSPACE_TOO_SMALL (gemm_workspace_size(M, N, K, 0)
 * tells in advance) before anything is launched. The scratch of the calling
 * thread's current device is used, so that device must be the one the
 * stream and pointers belong to. All calls on one GPU share its array: calls
 * that overlap in time (on different streams, or from several threads) race
 * and give undefined results; calls ordered on one stream are safe. The first
 * call on each device looks up the array's device address
 * (hipGetSymbolAddress); a failure there returns GEMM_ERR_HIP.
 */
gemm_status gemm_bf16_noalloc(int64_t M, int64_t N, int64_t K, float alpha,
                              const void* A, int64_t lda, gemm_layout layout_a,
                              const void* B, int64_t ldb, gemm_layout layout_b,
                              float beta, void* C, int64_t ldc, gemm_out_dtype c_dtype,
                              const void* bias, gemm_act act, void* stream);

/*
 * OCP FP8 E4M3 x E4M3 -> FP32 accumulate -> x scale_a[m]*scale_b[n] -> epilogue.
 * A must be ROW (K-major, per-token rows) and B COL (K-major, per-channel
 * rows); other layouts return GEMM_ERR_UNSUPPORTED. scale_a (FP32[M]) and
 * scale_b (FP32[N]) are required. Codes 0x7F/0xFF (NaN) give undefined results.
 * workspace: at least gemm_workspace_size(M, N, K, 1) bytes.
 */
gemm_status gemm_fp8_scaled(int64_t M, int64_t N, int64_t K, float alpha,
                            const void* A, int64_t lda, gemm_layout layout_a,
                            const void* B, int64_t ldb, gemm_layout layout_b,
                            const float* scale_a, const float* scale_b,
                            float beta, void* C, int64_t ldc, gemm_out_dtype c_dtype,
                            const void* bias, gemm_act act,
                            void* workspace, size_t workspace_bytes, void* stream);

/*
 * MX FP8 GEMM: E4M3 x E4M3 with one power-of-two (E8M0) scale per 32
 * consecutive K elements of each row of A and of each column of B, i.e. the
 * per-group scaling the FP8 DeepGEMM page (sec. 3.2) names next to the
 * per-token x per-channel form, in the block layout of the OCP
 * Microscaling (MX) formats, which gfx950's scaled MFMA applies in hardware:
 *
 *   C = act( alpha * sum_k a(m,k) 2^(SA[m][k/32]-127) * b(k,n) 2^(SB[n][k/32]-127)
 *            + beta * C + bias[n] )
 *
 * A: E4M3 codes, ROW (K-major), lda >= K. B: E4M3 codes, COL (K-major, N rows
 * of ldb), ldb >= K. Other layouts: GEMM_ERR_UNSUPPORTED.
 * scale_a: E8M0 codes (uint8), M rows of ldsa bytes; byte k/32 of row m
 * scales a(m, k). scale_b: N rows of ldsb bytes; byte k/32 of row n scales
 * b(k, n). Code c means 2^(c-127); code 255 (NaN) gives undefined results.
 * ldsa, ldsb: >= ceil(K/32), multiples of 4, >= 4; the arrays must span
 * M * ldsa and N * ldsb bytes, 4-byte aligned. Bytes past ceil(K/32) in a
 * row are never used.
 * A, B: any byte alignment and any K; the path reads its operands by DMA
 * only, with 32-bit offsets, so an operand spanning 2^31 bytes or more
 * ((rows - 1) * ld + K) gives GEMM_ERR_UNSUPPORTED.
 * There are no FP32 per-token / per-channel scales on this call. Epilogue,
 * C, bias, act, beta, workspace (size: gemm_workspace_size(M, N, K, 1)) and
 * stream as for gemm_fp8_scaled. Errors as for gemm_fp8_scaled, plus
 * GEMM_ERR_BAD_LD for ldsa / ldsb, GEMM_ERR_NULL_POINTER for NULL scales when
 * K > 0, GEMM_ERR_BAD_DIM when (M + 256) * ldsa or (N + 256) * ldsb reaches 2^31.
 */
gemm_status gemm_mxfp8(int64_t M, int64_t N, int64_t K, float alpha,
                       const void* A, int64_t lda, gemm_layout layout_a,
                       const void* B, int64_t ldb, gemm_layout layout_b,
                       const void* scale_a, int64_t ldsa, const void* scale_b, int64_t ldsb,
                       float beta, void* C, int64_t ldc, gemm_out_dtype c_dtype,
                       const void* bias, gemm_act act,
                       void* workspace, size_t workspace_bytes, void* stream);

/* Element type of a quantised output (gemm_*_quant). */
typedef enum { GEMM_QOUT_INT8 = 0, GEMM_QOUT_E4M3 = 1 } gemm_qout_dtype;

/*
 * GEMM with a quantising epilogue: the FP32 epilogue value is quantised per
 * token (row) and written as one byte per element, so the next layer reads a
 * quarter of the FP32 bytes and no separate quantisation pass over C is
 * needed (first DeepGEMM page, sec. 6.2: the quantisation
 * round(x * scale + zero_point) applied to each output fragment inside the
 * epilogue, with one scale per row looked up by the row index). For output
 * element (m, n):
 *
 *   z = alpha * (scale_a[m] * scale_b[n]) * sum_k a(m,k) b(k,n) + bias[n]
 *       (scale_a, scale_b only in gemm_fp8_scaled_quant)
 *   y = act(z)                                     (FP32, as in gemm_bf16)
 *   GEMM_QOUT_INT8: v = fp32(y * out_scale[m] + zp[m]) (fused multiply-add,
 *                   one rounding; zp = out_zero[m], or 0 when out_zero is NULL)
 *                   Q[m*ldq+n] = int8 of round-to-nearest-even(v), saturated
 *                   to [-128, 127]
 *   GEMM_QOUT_E4M3: w = fp32(y * out_scale[m])
 *                   Q[m*ldq+n] = OCP E4M3FN code of w, round to nearest even,
 *                   saturating at +-448 (out_zero must be NULL)
 *
 * out_scale multiplies (it is the inverse of the dequantisation step); the
 * next layer recovers y ~ (q - zp) / out_scale. There is no beta and no C_in:
 * Q is only written. A, B, layouts, bias, act, scale_a / scale_b, workspace
 * and stream are as in gemm_bf16 / gemm_fp8_scaled (same layout rules, same
 * workspace size query with is_fp8 = 0 / 1).
 * Q: device, M x N bytes, row-major, ldq >= N (int8 or E4M3 codes).
 * out_scale: device FP32[M], finite; out_zero: device INT32[M] with values of
 * magnitude below 2^24, or NULL. NaN or infinite y give undefined codes.
 * Errors (before anything is enqueued): GEMM_ERR_BAD_ENUM (q_dtype, layout
 * or act), GEMM_ERR_UNSUPPORTED (out_zero given with GEMM_QOUT_E4M3, or a
 * layout the dtype does not support), GEMM_ERR_NULL_POINTER (out_scale, Q,
 * A / B when K > 0, the FP8 scales), and the other codes as for the plain calls.
 */
gemm_status gemm_bf16_quant(int64_t M, int64_t N, int64_t K, float alpha,
                            const void* A, int64_t lda, gemm_layout layout_a,
                            const void* B, int64_t ldb, gemm_layout layout_b,
                            const void* bias, gemm_act act,
                            const float* out_scale, const int32_t* out_zero,
                            void* Q, int64_t ldq, gemm_qout_dtype q_dtype,
                            void* workspace, size_t workspace_bytes, void* stream);

gemm_status gemm_fp8_scaled_quant(int64_t M, int64_t N, int64_t K, float alpha,
                                  const void* A, int64_t lda, gemm_layout layout_a,
                                  const void* B, int64_t ldb, gemm_layout layout_b,
                                  const float* scale_a, const float* scale_b,
                                  const void* bias, gemm_act act,
                                  const float* out_scale, const int32_t* out_zero,
                                  void* Q, int64_t ldq, gemm_qout_dtype q_dtype,
                                  void* workspace, size_t workspace_bytes, void* stream);

/*
 * Per-token FP8 quantisation of BF16 activations, producing the A operand and
 * scale_a of gemm_fp8_scaled (the per-token scaling of DeepGEMM: FP8 precision
 * Tensor Core GEMM optimisation, sec. 1.2, done in one pass per row instead of
 * separate scale and cast kernels). For each row m of X:
 *   scale[m]   = fp32(max_k |x(m,k)| / 448), or 1 if the row is all zero
 *   Q[m*ldq+k] = OCP E4M3FN code of x(m,k) / scale[m] (IEEE float32 division,
 *                round to nearest even, saturating at +-448)
 * X: BF16, M x K row-major, ldx >= K (device). Q: uint8, M x K row-major,
 * ldq >= K (device). scale: FP32[M] (device). Columns K..ld-1 are neither read
 * nor written. K == 0 writes scale = 1 for every row. NaN or infinite inputs
 * give undefined codes and scales. Errors: GEMM_ERR_BAD_DIM (M or K negative
 * or above 2^30), GEMM_ERR_BAD_LD, GEMM_ERR_NULL_POINTER (scale, or X / Q when
 * K > 0), GEMM_ERR_HIP; all checks run before anything is enqueued.
 */
gemm_status gemm_quantize_fp8_rows(int64_t M, int64_t K, const void* X, int64_t ldx,
                                   void* Q, int64_t ldq, float* scale, void* stream);

/*
 * One-time reorder of a weight matrix B (logical K x N) into the layout the
 * fast path reads: Bp[n*ldbp + k] = b(k, n), i.e. GEMM_COL_MAJOR (K-major)
 * with leading dimension ldbp. The FP8 DeepGEMM page (sec. 3.2) rearranges B
 * once, before the calls that reuse it, so the reorder is paid once per
 * weight. Pass the result to gemm_bf16 / gemm_fp8_scaled / gemm_mxfp8 with
 * layout_b = GEMM_COL_MAJOR and ldb = ldbp: a K-major B (below 2^31 bytes)
 * is copied to on-chip memory by DMA (the fast path) at any alignment, while
 * an N-contiguous B is read through registers, several times slower, unless
 * it is BF16 with 16-byte aligned rows and N a multiple of 8. With ldbp *
 * elem_bytes and K * elem_bytes multiples of 16 and Bp 16-byte aligned, the
 * DMA reads are aligned and decode-sized M can use the skinny kernel.
 * B: device, elements of elem_bytes (2: BF16, 1: E4M3; moved as bits), in
 * layout_b (ROW: b(k,n) = B[k*ldb + n], ldb >= N; COL: B[n*ldb + k],
 * ldb >= K). Bp: device, N rows of ldbp >= K elements; the elements k >= K of
 * each row are not written. Bp must not overlap B.
 * Errors (before anything is enqueued): GEMM_ERR_BAD_ENUM (layout_b,
 * elem_bytes), GEMM_ERR_BAD_DIM (K or N negative or above 2^30),
 * GEMM_ERR_BAD_LD, GEMM_ERR_NULL_POINTER (B or Bp when K, N > 0),
 * GEMM_ERR_HIP. K == 0 or N == 0 does nothing.
 */
gemm_status gemm_pack_b(int64_t K, int64_t N, const void* B, int64_t ldb, gemm_layout layout_b,
                        int elem_bytes, void* Bp, int64_t ldbp, void* stream);

/*
 * Bytes of device workspace a call with these sizes needs (0 when the chosen
 * kernel needs none). Pure host arithmetic; callable without a GPU. Query
 * once and allocate up front (the FP8 page's interface, sec. 5.1, separates
 * the size query from the call for the same reason). is_fp8: 0 for
 * gemm_bf16, 1 for gemm_fp8_scaled. Negative sizes return 0.
 */
size_t gemm_workspace_size(int64_t M, int64_t N, int64_t K, int is_fp8);

/*
 * The launch plan the library would use (host arithmetic only, no GPU
 * needed): tile sizes, split-K factor and grid. Returns GEMM_OK or
 * GEMM_ERR_BAD_DIM / GEMM_ERR_NULL_POINTER. Intended for tests and tuning.
 */
typedef struct {
  int32_t kernel;       /* 0 = tiled MFMA kernel, 1 = skinny weight-streaming kernel
                           (M <= 16; K split over the waves of a workgroup) */
  int32_t tile_m, tile_n, tile_k;
  int32_t split_k;      /* number of K partitions (1 = none) */
  int32_t waves;        /* wavefronts per workgroup */
  int64_t grid;         /* workgroups launched by the main kernel */
  size_t workspace_bytes;
} gemm_plan_info;

gemm_status gemm_plan(int64_t M, int64_t N, int64_t K, int is_fp8, gemm_plan_info* out);

/* Static, NUL-terminated name of a status code ("GEMM_OK", ...). */
const char* gemm_status_string(gemm_status s);

#ifdef __cplusplus
}
#endif

#endif /* GEMM355_H */
