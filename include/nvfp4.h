/*
 * nvfp4.h -- C ABI of libnvfp4.so: NVFP4 quantization, expansion, the NVFP4-weight GEMM and
 * percentile-amax calibration, as hand-written HIP kernels for AMD Instinct MI355X (gfx950).
 *
 * The format ("Qwen-Image NVFP4 on a 16 GB Ada GPU: NVFP4 vs NF4, weight error, speed and the
 * NF4 grain", section "What NVFP4 is and how it differs from NF4"):
 *   - each element is an E2M1 code: sign bit, 2 exponent bits, 1 mantissa bit, magnitudes
 *     {0, 0.5, 1, 1.5, 2, 3, 4, 6};
 *   - each run of 16 consecutive elements along a row carries one FP8 E4M3 (OCP e4m3fn) scale;
 *   - each tensor carries one fp32 global scale;
 *   - value = E2M1 x block scale x global scale; two codes per byte, element 2j in the low
 *     nibble of byte j (the stored-block figure "First NVFP4 block, as stored in the file");
 *   - storage is 4.5 bits per element.
 *
 * Conventions for every entry point:
 *   - all pointers are device memory owned by the caller; the library never allocates, frees
 *     or retains them;
 *   - work is enqueued on `stream` and the call returns without synchronizing;
 *   - arguments are validated before anything is enqueued: on any error nothing runs and the
 *     status says why; a failed kernel launch returns NVFP4_ERR_LAUNCH;
 *   - data-dependent conditions (a NaN or infinity in the input) do not fail the call: they OR
 *     bit 0 into the optional device int `flags`, which the caller clears;
 *   - matrices are row-major with a row stride (`ld*`, in elements); every pointer and every
 *     row start must be 16-byte aligned, except the fp32 GEMM output C, whose rows need 4 bytes
 *     (NVFP4_ERR_ALIGN otherwise);
 *   - the library checks once per device that it runs on gfx950 (NVFP4_ERR_DEVICE otherwise);
 *   - the calls are thread-safe; calls that share a workspace buffer must be ordered by the
 *     caller (same stream, or events);
 *   - every call may be captured in a HIP graph and replayed: the library enqueues kernels only
 *     (no allocation, memset, copy or host synchronization), and no per-call value is frozen into
 *     the kernel arguments.
 */
#ifndef NVFP4_H
#define NVFP4_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    NVFP4_OK = 0,
    NVFP4_ERR_NULL = 1,      /* a required pointer is NULL                                       */
    NVFP4_ERR_SHAPE = 2,     /* negative size, cols % 16 != 0, ld < cols, or operands disagree   */
    NVFP4_ERR_ALIGN = 3,     /* a pointer or a row start is not 16-byte aligned                  */
    NVFP4_ERR_DTYPE = 4,     /* dtype not accepted by this entry point                          */
    NVFP4_ERR_WORKSPACE = 5, /* workspace NULL or smaller than nvfp4_workspace_size()            */
    NVFP4_ERR_ARG = 6,       /* p outside (0, 100], a bad mode flag, both/neither GEMM operand   */
    NVFP4_ERR_DEVICE = 7,    /* the current device is not gfx950                                 */
    NVFP4_ERR_LAUNCH = 8     /* the HIP runtime refused a launch                                 */
} nvfp4_status;

typedef enum {
    NVFP4_F32 = 0,  /* IEEE binary32                                                           */
    NVFP4_BF16 = 1, /* bfloat16                                                                */
    NVFP4_F16 = 2,  /* IEEE binary16                                                           */
    NVFP4_E4M3 = 3  /* OCP FP8 e4m3fn bytes (bias 7, no infinity, 0x7F / 0xFF are NaN)          */
} nvfp4_dtype;

/* An NVFP4 tensor of logical shape [rows x cols], cols % 16 == 0, dense:
 *   codes        rows * cols/2 bytes, row-major; element 2j of a row in the low nibble of byte j
 *   scales       rows * cols/16 bytes, row-major; E4M3 bit patterns, sign bit always 0
 *   global_scale one float; element value = e2m1(code) * e4m3(scale) * (*global_scale)       */
typedef struct {
    uint8_t *codes;
    uint8_t *scales;
    float *global_scale;
    int64_t rows, cols;
} nvfp4_tensor;

/* Operation selectors for nvfp4_workspace_size. */
enum {
    NVFP4_OP_QUANTIZE = 0,
    NVFP4_OP_DEQUANTIZE = 1,
    NVFP4_OP_GEMM = 2,
    NVFP4_OP_PERCENTILE = 3,
    NVFP4_OP_STATS = 4,
    NVFP4_OP_LOWRANK = 5,
    NVFP4_OP_GEMM_QA = 6,
    NVFP4_OP_AMAX = 7
};

/*
 * nvfp4_quantize -- x [out->rows x out->cols] (row stride ld_x elements) -> NVFP4 `out`.
 *
 * Steps (the passage each follows):
 *   1. widen to fp32; for an E4M3 source, v = fl(e4m3(b) * *src_scale), a NULL src_scale meaning
 *      1.0 ("Qwen-Rapid-AIO-NVFP4", section "Why This Exists": FP8 weights are upcast to FP32
 *      before re-quantizing, and some layers come without weight_scale);
 *   2. amax = max |v| over the tensor, or *amax_in when given (a static, calibrated amax; values
 *      beyond it clip to +-6 x 448 x g) -- activations use the run-time form
 *      ("Qwen3-VL-8B-Instruct-heretic-NVFP4", "Quantization Details": per-tensor amax at run time);
 *   3. g = fl(amax / 2688), 2688 = 6 x 448, written to *out->global_scale;
 *   4. per 16-element block: scale byte = E4M3 round-to-nearest-even, saturating at 448, of
 *      fl(bamax / fl(6 g)); 0 when g = 0;
 *   5. per element: d = fl(s g), r = fl(1 / d), code = nearest E2M1 of fl(|v| r) (ties to the
 *      even code, saturating at 6), sign bit = sign bit of v; s = 0 gives magnitude 0;
 *   6. pack two codes per byte, low nibble first.
 * Arguments: x_dtype any of nvfp4_dtype; src_scale only for NVFP4_E4M3 (must be > 0 if given);
 * amax_in NULL for the run-time amax; flags nullable (bit 0 = non-finite input seen; bit 1 = the
 * run-time amax could not be agreed within a bounded wait; bit 2 = the workspace was not in the
 * state the previous call left it in; outputs are unspecified when any is set); workspace of
 * nvfp4_workspace_size(NVFP4_OP_QUANTIZE, rows, cols, 0) bytes (run-time amax only).
 * Run-time amax in one launch: every workgroup keeps its part of the input on chip while the grid
 * agrees on amax through the workspace, so the input crosses HBM once.  Preconditions:
 *   - the workspace holds zeros before its first use (it then carries a call counter from one call
 *     to the next and needs no further clearing; the call may be captured in a HIP graph and
 *     replayed); a workspace that was not zeroed, or is used by overlapping calls, sets bit 2;
 *   - no kernel of another stream holds compute units while the call runs: the launch uses as
 *     many workgroups as the GPU holds at once, and each waits for all the others.  Work that keeps
 *     some of them off the GPU for the bounded wait sets bit 1.  Callers that overlap streams use
 *     the two-launch form instead: nvfp4_tensor_amax, then this call with amax_in = its output
 *     (identical codes, scale bytes and global scale, no co-residency needed).
 * src_scale, amax_in, flags and workspace are device pointers.
 */
nvfp4_status nvfp4_quantize(const void *x, nvfp4_dtype x_dtype, int64_t ld_x, const float *src_scale,
                            const float *amax_in, const nvfp4_tensor *out, int32_t *flags, void *workspace,
                            size_t workspace_bytes, hipStream_t stream);

/*
 * nvfp4_quantize_batch -- count (0 .. 8) tensors of one source dtype quantized to NVFP4, each with
 * its own run-time amax: exactly what count calls of nvfp4_quantize (amax_in NULL) on the same
 * stream produce, in one launch when the tensors together stay resident on chip (a layer's four
 * 3072 x 3072 FP8 projection weights do; "Qwen-Rapid-AIO-NVFP4", section "Why This Exists": every
 * FP8 weight of the model is requantized to NVFP4), else one launch per tensor.  Steps 1-6 of
 * nvfp4_quantize per tensor.  x[i], ld_x[i], src_scale[i] and out[i] are the arguments of tensor
 * i's call; the arrays x, ld_x, src_scale and out are host memory (src_scale may be NULL: no source
 * scale for any tensor; an element may be NULL), the pointers in them device memory.  One flags
 * word (nullable) collects the bits of every tensor.  The workspace and its preconditions are
 * those of nvfp4_quantize (the same workspace may serve both); in one launch every workgroup waits
 * for all the others, as in nvfp4_quantize.  NVFP4_ERR_ARG for count outside 0 .. 8.
 */
nvfp4_status nvfp4_quantize_batch(int count, const void *const *x, nvfp4_dtype x_dtype, const int64_t *ld_x,
                                  const float *const *src_scale, const nvfp4_tensor *out, int32_t *flags,
                                  void *workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * nvfp4_quantize_noalloc -- nvfp4_quantize without a workspace argument, for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc).  Same arguments, steps, results and flags as nvfp4_quantize; the run-time amax
 * agreement uses a scratch array inside the library instead of the caller's workspace: 16 KiB of
 * device memory per GPU the library runs on, held until the process ends, zeroed when the library
 * is loaded and left consistent by every call.  Every tensor size fits it.  The call allocates
 * nothing (no hipMalloc, no library routine that allocates).  All calls on one GPU share that GPU's
 * scratch: calls that overlap on one GPU (different streams with no ordering between them) race on
 * it; such a race is reported in flags bit 2 when it is seen, and the outputs are then invalid.
 * The static-amax form (amax_in not NULL) uses no scratch.  NVFP4_ERR_DEVICE also when the scratch
 * address cannot be obtained.
 */
nvfp4_status nvfp4_quantize_noalloc(const void *x, nvfp4_dtype x_dtype, int64_t ld_x, const float *src_scale,
                                    const float *amax_in, const nvfp4_tensor *out, int32_t *flags,
                                    hipStream_t stream);

/*
 * nvfp4_tensor_amax -- *amax_out = max |v| over x [rows x cols] (row stride ld_x elements), v the
 * source value widened as nvfp4_quantize step 1 does (E4M3 source: times *src_scale, NULL meaning
 * 1.0; "Qwen3-VL-8B-Instruct-heretic-NVFP4", "Quantization Details": a per-tensor amax taken at
 * run time).  The first launch of the two-launch run-time quantize: passing amax_out as amax_in to
 * nvfp4_quantize or nvfp4_quantize_fp8 gives exactly the outputs of their one-launch run-time form,
 * without its requirement that the whole grid be resident at once.  Two kernels: per-workgroup
 * maxima into the workspace, then one workgroup reduces them.  A non-finite value ORs bit 0 into
 * the optional *flags.  cols % 16 == 0; rows == 0 gives 0.  workspace of
 * nvfp4_workspace_size(NVFP4_OP_AMAX, rows, cols, 0) bytes (needs no initialization; not the
 * workspace of a run-time-amax quantize, whose contents carry from call to call).
 * src_scale, amax_out, flags and workspace are device pointers.
 */
nvfp4_status nvfp4_tensor_amax(const void *x, nvfp4_dtype x_dtype, int64_t rows, int64_t cols, int64_t ld_x,
                               const float *src_scale, float *amax_out, int32_t *flags, void *workspace,
                               size_t workspace_bytes, hipStream_t stream);

/*
 * nvfp4_quantize_fp8 -- x [rows x cols] (row stride ld_x elements) -> FP8 E4M3 bytes out [rows x
 * cols] (dense, row-major) and one fp32 tensor scale, for the layers kept in FP8 and for the FP8
 * activations of nvfp4_gemm_fp8a ("Qwen3-VL-8B-Instruct-heretic-NVFP4", "Quantization Details":
 * float8_e4m3fn, tensorwise, round to nearest, for embed_tokens and lm_head; "Runtime /
 * hardware": FP4 weights against dynamically quantized FP8 activations):
 *   1. widen to fp32 as nvfp4_quantize does (E4M3 source: times *src_scale, NULL meaning 1.0);
 *   2. amax = max |v| over the tensor, or *amax_in (static; values beyond it saturate);
 *   3. *out_scale = fl(amax / 448), 448 the largest E4M3 value; 1.0 when amax = 0;
 *   4. byte = sign bit of v | E4M3 round-to-nearest-even of fl(|v| / scale), saturating at 448
 *      (0x7E); value = e4m3(byte) x scale.
 * cols % 16 == 0.  flags, workspace and the preconditions of the one-launch run-time amax as for
 * nvfp4_quantize (workspace of nvfp4_workspace_size(NVFP4_OP_QUANTIZE, rows, cols, 0) bytes, zeroed
 * before first use, when amax_in is NULL).
 * src_scale, amax_in, out_scale, flags and workspace are device pointers.
 */
nvfp4_status nvfp4_quantize_fp8(const void *x, nvfp4_dtype x_dtype, int64_t rows, int64_t cols, int64_t ld_x,
                                const float *src_scale, const float *amax_in, uint8_t *out, float *out_scale,
                                int32_t *flags, void *workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * nvfp4_dequantize -- the expander: NVFP4 `in` -> out [in->rows x in->cols] (row stride ld_out),
 * w = fl(e2m1 x s x g) in fp32 ("Qwen-Image NVFP4 on a 16 GB Ada GPU", section "Running the NVFP4
 * weights on Ada": each byte gives its two E2M1 values, each block's scale multiplies its 16
 * values, then the global scale); bf16 output is the round-to-nearest-even of that fp32 value.
 * out_dtype: NVFP4_F32 or NVFP4_BF16.  No workspace.
 */
nvfp4_status nvfp4_dequantize(const nvfp4_tensor *in, void *out, nvfp4_dtype out_dtype, int64_t ld_out,
                              hipStream_t stream);

/*
 * nvfp4_gemm -- C [M x N] fp32 (row stride ldc) = A . W_hat^T, with W an NVFP4 tensor [N x K]
 * (a PyTorch Linear weight, out-features x in-features):
 *   - W4A16: a_bf16 [M x K] bf16 (row stride lda), a_q NULL: the weights are expanded exactly
 *     to bf16 (e2m1 x s has at most 6 significant bits) inside the kernel, activations stay
 *     bf16 ("Qwen-Image NVFP4 on a 16 GB Ada GPU", section "Running the NVFP4 weights on Ada");
 *   - W4A4: a_q an NVFP4 tensor [M x K] (from nvfp4_quantize, run-time or static amax), a_bf16
 *     NULL: both operands expanded exactly ("What NVFP4 is and how it differs from NF4": on
 *     Blackwell weights and activations are both 4-bit; "Qwen3-VL-8B-Instruct-heretic-NVFP4",
 *     "Runtime / hardware");
 * products are summed in fp32 and the sum is multiplied by the global scale(s) at the end.
 * Exactly one of a_bf16 / a_q must be non-NULL (NVFP4_ERR_ARG otherwise).  lda is ignored for
 * W4A4.  workspace (16-byte aligned, or NULL): with nvfp4_workspace_size(NVFP4_OP_GEMM, M, N, K)
 * bytes, problems with few output tiles and a long K are split along K (fp32 partial sums per
 * slice in the workspace, then summed in slice order); with less, or NULL, the unsplit kernel runs.
 * Up to 16 rows of A (M <= 5, or M <= 16 with K a multiple of 32 up to 4096) take the GEMV forms,
 * which stream W once and need no workspace.
 */
nvfp4_status nvfp4_gemm(const void *a_bf16, const nvfp4_tensor *a_q, int64_t M, int64_t lda,
                        const nvfp4_tensor *w, float *c, int64_t ldc, void *workspace, size_t workspace_bytes,
                        hipStream_t stream);

/*
 * nvfp4_gemm_qa -- C [M x N] fp32 (row stride ldc) = A_hat . W_hat^T, the W4A4 product with the
 * activations quantized inside the GEMM: A_hat is the NVFP4 form of a_bf16 [M x K] (bf16, row stride
 * lda) under the static (calibrated) amax *a_amax -- exactly what nvfp4_quantize(amax_in = a_amax)
 * would store -- so no activation-quantize launch precedes the product ("Qwen3-VL-8B-Instruct-
 * heretic-NVFP4", "Quantization Details": NVFP4 activations with a per-tensor amax;
 * "Qwen-Rapid-AIO-NVFP4", "Recommended Model": static per-layer amax from p99.9 calibration; with
 * a static amax the quantization of a tile needs nothing outside the tile).  Values above the amax
 * saturate.  One launch in the usual case; three forms, chosen per problem:
 *   - staged: when all of the W4A4 product's workgroups run in one round on the device (as at
 *     4096 x 3072 x 3072, 512 x 12288 x 4096 and 512 x 4096 x 12288), the workgroups that share an
 *     A row block (and K slice) each quantize a share of its 16-element blocks into the workspace,
 *     wait for one another on a counter in the workspace, then run the W4A4 main loop on them --
 *     each block is quantized once, and the result is bit-identical to nvfp4_quantize(amax_in =
 *     a_amax) followed by nvfp4_gemm (W4A4).  Needs the full workspace; its first 4096 bytes are
 *     the group counters, which must be zero before the first call that uses this workspace and
 *     which every call leaves zero (allocate it zeroed once and reuse it; calls that share it must
 *     not overlap).  The wait assumes the product's workgroups can all be resident together (no
 *     kernel on another stream holding the CUs for long); a workgroup whose wait runs out quantizes
 *     its whole row block itself, so results never depend on it.
 *   - fused (K % 64 == 0, M > 4, N <= 512, when staged does not apply): each workgroup quantizes
 *     the A rows of its tile in its staging path (the block scale, the codes and their exact f16
 *     values; see nvfp4_quantize for the steps);
 *   - otherwise a quantize pass into the workspace followed by the W4A4 kernel (NVFP4_ERR_WORKSPACE
 *     if the workspace is NULL or smaller than the quantized activations).
 * a_amax: device pointer to one float (>= 0; 0 gives C = 0).  Inputs must be finite (no flag).
 * workspace (16-byte aligned): nvfp4_workspace_size(NVFP4_OP_GEMM_QA, M, N, K) bytes covers every
 * form.
 */
nvfp4_status nvfp4_gemm_qa(const void *a_bf16, const float *a_amax, int64_t M, int64_t lda, const nvfp4_tensor *w,
                           float *c, int64_t ldc, void *workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * nvfp4_gemm_lowrank -- C [M x N] fp32 (row stride ldc) = A_hat . W_hat^T + (A . V^T) . U^T: the
 * NVFP4 product of nvfp4_gemm plus a bf16 low-rank branch of the weight, W ~ W_hat + U . V
 * ("Qwen Image 2.1: INT4 + FP4", section "What I quantized": FP4 weights with BF16 rank-128
 * branches).
 *   a_bf16  [M x K] bf16, row stride lda: the activations of the branch, and of the main product
 *           when a_q is NULL (W4A16); required (may be NULL only when M == 0 or K == 0);
 *   a_q     NULL, or the NVFP4 activations [M x K] of a W4A4 main product;
 *   lr_down V [rank x K] bf16, dense; lr_up U [N x rank] bf16, dense; 16 <= rank <= 256,
 *           rank % 16 == 0 (NVFP4_ERR_SHAPE otherwise).
 * T = A . V^T is summed in fp32 and carried as two bf16 planes (T_hi + T_lo, about 2^-17 relative);
 * the up-projection runs in the GEMM's epilogue on the matrix cores when the product takes the
 * unsplit tiled kernel, otherwise as a second pass that adds into C.
 * workspace (device, 16-byte aligned): at least nvfp4_workspace_size(NVFP4_OP_LOWRANK, M, N, K)
 * bytes -- T (M * 1 KiB) then the product's split-K planes; NVFP4_ERR_WORKSPACE when smaller than
 * the T part (with less than the full size the product runs unsplit).  M == 0 or K == 0 needs no
 * workspace (C = 0 when K == 0).
 */
nvfp4_status nvfp4_gemm_lowrank(const void *a_bf16, const nvfp4_tensor *a_q, int64_t M, int64_t lda,
                                const nvfp4_tensor *w, const void *lr_down, const void *lr_up, int64_t rank, float *c,
                                int64_t ldc, void *workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * nvfp4_gemm_fp8a -- C [M x N] fp32 (row stride ldc) = A_hat . W_hat^T with FP8 activations: a_fp8
 * [M x K] E4M3 bytes (row stride lda bytes, from nvfp4_quantize_fp8) with tensor scale *a_scale,
 * and W an NVFP4 tensor [N x K] ("Qwen3-VL-8B-Instruct-heretic-NVFP4", "Runtime / hardware": FP4
 * weight x dynamically quantized FP8 activation).  Both operands are expanded exactly to f16
 * inside the kernel (e4m3 values and e2m1 x s both fit f16 exactly; bf16 in the GEMV forms for
 * M <= 16); products are summed in fp32 and the sum is multiplied by *a_scale and the weight's
 * global scale at the end.  workspace as for nvfp4_gemm (split-K partial sums; NULL runs the
 * unsplit kernel; none needed where the GEMV forms run: M <= 5 with M x K x 2 <= 64 KiB, and
 * M <= 16 with K a multiple of 32 up to 4096).
 */
nvfp4_status nvfp4_gemm_fp8a(const uint8_t *a_fp8, const float *a_scale, int64_t M, int64_t lda,
                             const nvfp4_tensor *w, float *c, int64_t ldc, void *workspace, size_t workspace_bytes,
                             hipStream_t stream);

/*
 * amax_percentile -- calibration statistic: for each column c of x [rows x cols] (per_channel
 * = 1, out_pct/out_max hold cols floats) or for the whole tensor (per_channel = 0, one float),
 * the nearest-rank p-th percentile of |x| (k = clamp(ceil(p n / 100), 1, n), the k-th smallest)
 * and the maximum of |x| ("Qwen-Rapid-AIO-NVFP4", section "Recommended Model": p99.9 calibration
 * instead of max aggregation; "Qwen-Image NVFP4 on a 16 GB Ada GPU", section "Quality: the error
 * of each matrix": percentiles by nearest rank).  The selection is exact on the bit patterns.
 * x_dtype: NVFP4_F32, NVFP4_BF16 or NVFP4_F16.  out_max and flags may be NULL.  workspace of
 * nvfp4_workspace_size(NVFP4_OP_PERCENTILE, rows, cols, per_channel) bytes; per channel that size
 * holds candidate lists (8 KB per channel) for ranks 17 .. about 250 from an end over at least
 * 32768 rows (one pass over x after a threshold from every 16th row; the exact passes only for
 * channels the candidates cannot settle), and with less, down to 1036 bytes per channel, two or
 * four radix passes over x run instead: the results are the same.  -0 counts as +0.  rows must be
 * >= 1.
 */
nvfp4_status amax_percentile(const void *x, nvfp4_dtype x_dtype, int64_t rows, int64_t cols, int64_t ld_x,
                             double p, int per_channel, float *out_pct, float *out_max, int32_t *flags,
                             void *workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * nvfp4_matrix_stats -- quality statistics of one weight matrix w [rows x cols] (row stride ld_w
 * elements) and, when q is not NULL, of its NVFP4 form q ("Qwen-Image NVFP4 on a 16 GB Ada GPU",
 * section "Quality: the error of each matrix": the relative error of each matrix, its kurtosis,
 * the ratio of the maximum to the standard deviation in blocks of 64).  Writes 7 doubles to out:
 *   out[0] ||w - w_hat||_F / ||w||_F, w_hat the exact expansion of q (NaN when q is NULL);
 *   out[1] excess kurtosis m4 / m2^2 - 3, population central moments (from power sums in double);
 *   out[2] mean over blocks of 64 consecutive elements in row-major order (the last one may be
 *          shorter) of max |w| / population std of the block, blocks with std 0 left out (NaN if
 *          none);
 *   out[3] mean; out[4] population std; out[5] max |w|; out[6] number of blocks in out[2].
 * w_dtype: NVFP4_F32, NVFP4_BF16 or NVFP4_F16; cols % 16 == 0 (and cols <= 2^30 when the rows are
 * not contiguous, ld_w != cols); q, when given, has w's shape.
 * out (8-byte aligned) and workspace (nvfp4_workspace_size(NVFP4_OP_STATS, 0, 0, 0) bytes) are
 * device pointers.  The sums are reduced in a fixed order, so results repeat exactly on one device.
 */
nvfp4_status nvfp4_matrix_stats(const void *w, nvfp4_dtype w_dtype, int64_t rows, int64_t cols, int64_t ld_w,
                                const nvfp4_tensor *q, double *out, void *workspace, size_t workspace_bytes,
                                hipStream_t stream);

/* Workspace bytes an entry point needs (0 when none).  For NVFP4_OP_PERCENTILE the last argument
 * is per_channel; for NVFP4_OP_GEMM the arguments are (M, N, K), and the size is planned for the
 * current device (an MI355X's 256 CUs when none can be queried). */
size_t nvfp4_workspace_size(int op, int64_t rows, int64_t cols, int64_t k);

/* A static, human-readable name for a status code. */
const char *nvfp4_status_string(nvfp4_status s);

#ifdef __cplusplus
}
#endif

#endif /* NVFP4_H */
