// Host-side launchers behind the C ABI (one per entry point).  Each enqueues its kernels on
// `stream` and returns the HIP error of the launches; argument validation happens in api.hip.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "nvfp4.h"

namespace nvfp4 {

// Quantize workspace: a few words plus one 64-bit slot per workgroup of the single-pass kernel
// (2040 slots: four workgroups per CU on parts with up to 510 CUs, two on larger ones).
constexpr size_t kQuantizeWsBytes = 16384;

hipError_t launch_quantize(const void *x, nvfp4_dtype dt, int64_t ld_x, const float *src_scale, const float *amax_in,
                           const nvfp4_tensor *out, int32_t *flags, void *workspace, int num_cus, hipStream_t stream);

// Run-time amax quantizes of up to kQuantizeMaxBatch tensors of one source dtype in one launch of the
// single-pass kernel, each tensor with its own amax, when every tensor stays resident on chip;
// otherwise nothing is launched and *batched is false.
constexpr int kQuantizeMaxBatch = 8;
hipError_t launch_quantize_batch(int count, const void *const *x, nvfp4_dtype dt, const int64_t *ld_x,
                                 const float *const *src_scale, const nvfp4_tensor *out, int32_t *flags,
                                 void *workspace, int num_cus, hipStream_t stream, bool *batched);

// Run-time amax as a pass of its own: *amax_out = max |v| (fp32; E4M3 source: the largest byte's
// value times *src_scale), from per-workgroup partial maxima in the workspace (kAmaxWsBytes).
constexpr int kAmaxMaxParts = 2048;
constexpr size_t kAmaxWsBytes = kAmaxMaxParts * 4;
hipError_t launch_amax(const void *x, nvfp4_dtype dt, int64_t ld_x, int64_t rows, int64_t cols, const float *src_scale,
                       float *amax_out, int32_t *flags, void *workspace, int num_cus, hipStream_t stream);

// FP8 E4M3 tensorwise: out [rows x cols] bytes (dense), *out_scale = the tensor scale.
hipError_t launch_quantize_fp8(const void *x, nvfp4_dtype dt, int64_t ld_x, int64_t rows, int64_t cols,
                               const float *src_scale, const float *amax_in, uint8_t *out, float *out_scale,
                               int32_t *flags, void *workspace, int num_cus, hipStream_t stream);

hipError_t launch_dequantize(const nvfp4_tensor *in, void *out, nvfp4_dtype out_dtype, int64_t ld_out, int num_cus,
                             hipStream_t stream);

// GEMM execution plan: tile shape (index into the shape table), number of K slices (split-K when
// > 1: each slice writes an fp32 partial plane, then an ordered sum) and K steps of 64 per slice.
struct GemmPlan {
    int cfg;
    int splits;
    int slice_steps;
};
// first_cfg: the first shape of the table the plan may use (the quantizing A path starts at the
// 128-row shapes, kFirstQuantTileCfg).
constexpr int kFirstQuantTileCfg = 2;
GemmPlan plan_gemm(int64_t M, int64_t N, int64_t K, int num_cus, int first_cfg = 0);
// Workspace bytes the plan for this problem uses (its split-K partial planes), 0 if none.
size_t gemm_ws_bytes(int64_t M, int64_t N, int64_t K, int num_cus, int first_cfg = 0);

hipError_t launch_gemm(const void *a_bf16, const nvfp4_tensor *a_q, int64_t M, int64_t lda, const nvfp4_tensor *w,
                       float *c, int64_t ldc, void *workspace, size_t workspace_bytes, int num_cus,
                       hipStream_t stream);

// The GEMM with E4M3 activations [M x K] (row stride lda bytes) and one tensor scale.
hipError_t launch_gemm_fp8(const uint8_t *a_fp8, const float *a_scale, int64_t M, int64_t lda, const nvfp4_tensor *w,
                           float *c, int64_t ldc, void *workspace, size_t workspace_bytes, int num_cus,
                           hipStream_t stream);

// The GEMM with a bf16 low-rank branch: C = A_hat . W_hat^T + (A . V^T) . U^T, V [r x K] and
// U [N x r] bf16 (dense).  The workspace holds T = A . V^T as a bf16 pair (lowrank_t_bytes(M)
// bytes), then the product's split-K planes (gemm_ws_bytes).
size_t lowrank_t_bytes(int64_t M);
hipError_t launch_gemm_lowrank(const void *a_bf16, const nvfp4_tensor *a_q, int64_t M, int64_t lda,
                               const nvfp4_tensor *w, const void *v, const void *u, int r, float *c, int64_t ldc,
                               void *workspace, size_t workspace_bytes, int num_cus, hipStream_t stream);
hipError_t launch_lowrank_down(const void *a_bf16, int64_t lda, const void *v, int64_t M, int64_t K, int r,
                               void *t, hipStream_t stream);
hipError_t launch_lowrank_up_add(const void *t, const void *u, int r, int64_t M, int64_t N, float *c, int64_t ldc,
                                 hipStream_t stream);

// W4A4 with the activations quantized in the GEMM (static amax): whether the fused kernel applies,
// and its launch (C = A_hat . W_hat^T, A_hat the NVFP4 quantization of A with amax *amax).
bool gemm_qa_fusable(int64_t M, int64_t K, int64_t lda);
hipError_t launch_gemm_qa_fused(const void *a_bf16, const float *amax, int64_t M, int64_t lda, const nvfp4_tensor *w,
                                float *c, int64_t ldc, void *workspace, size_t workspace_bytes, int num_cus,
                                hipStream_t stream);

// The staged one-launch form: every workgroup quantizes a share of its A row block (and K slice)
// into the workspace and waits for the other workgroups of that row block, then runs the W4A4 main
// loop on the quantized activations.  The workspace starts with kQaSyncBytes of group counters that
// must be zero before the first call and that every call leaves zero; the NVFP4 activations
// ([M][K/2] codes, [M][K/16] scales, each 256-byte aligned) and the split-K planes follow.  Applies
// when the product's plan runs all its workgroups in one round on the device (every group
// co-resident) with at most kQaMaxGroups groups; returns false (nothing launched) otherwise.
constexpr int kQaMaxGroups = 512;
constexpr size_t kQaSyncBytes = 2 * kQaMaxGroups * 4;
bool gemm_qa_staged_applies(int64_t M, int64_t N, int64_t K, int64_t lda, int num_cus);
size_t gemm_qa_staged_ws_bytes(int64_t M, int64_t N, int64_t K, int num_cus);
hipError_t launch_gemm_qa_staged(const void *a_bf16, const float *amax, int64_t M, int64_t lda, const nvfp4_tensor *w,
                                 float *c, int64_t ldc, void *workspace, size_t workspace_bytes, int num_cus,
                                 hipStream_t stream);

// Workspace of amax_percentile: the full size (with the candidate lists of the per-channel
// candidate path), and the least that runs (the radix passes only).
size_t percentile_ws_bytes(int64_t cols, int per_channel);
size_t percentile_ws_min_bytes(int64_t cols, int per_channel);

hipError_t launch_percentile(const void *x, nvfp4_dtype dt, int64_t rows, int64_t cols, int64_t ld_x, uint32_t k,
                             int per_channel, float *out_pct, float *out_max, int32_t *flags, void *workspace,
                             size_t workspace_bytes, int num_cus, hipStream_t stream);

// Matrix statistics: partial sums of at most kStatsMaxGroups workgroups in the workspace.
constexpr int kStatsMaxGroups = 2048;
size_t stats_ws_bytes();
hipError_t launch_stats(const void *x, nvfp4_dtype dt, int64_t rows, int64_t cols, int64_t ld_x,
                        const nvfp4_tensor *q, double *out, void *workspace, int num_cus, hipStream_t stream);

hipError_t launch_fill_zero_f32(float *c, int64_t rows, int64_t cols, int64_t ld, hipStream_t stream);

}  // namespace nvfp4
