// The bf16 low-rank branch next to an NVFP4 weight ("Qwen Image 2.1: INT4 + FP4", section "What I
// quantized": FP4 weights with BF16 rank-128 branches): the weight is W_hat + U . V with U [N x r]
// and V [r x K] in bf16, and the layer adds (A . V^T) . U^T to the NVFP4 product.
//
// T = A . V^T [M x r] is formed once per call (fp32 sums of exact bf16 products) and kept as two
// bf16 planes, T_hi = bf16(T) and T_lo = bf16(T - T_hi): T_hi + T_lo carries T to about 2^-17 of
// its size, so the up-projection runs on the bf16 matrix cores (two products per 16-deep slice)
// and still adds the branch with nearly fp32 accuracy.
#pragma once

#include "common.h"

namespace nvfp4 {

constexpr int kLrMaxRank = 256;
constexpr int kLrChunk = 64;  // ranks per LDS-staged chunk of the fused epilogue

// Branch operands of the up-projection: T_hi / T_lo [M x r] bf16 (dense, plane stride M * r) and
// U [N x r] bf16 (dense).
struct LrArgs {
    const __bf16 *t;  // T_hi; T_lo follows at t + M * r
    const __bf16 *u;
    int r;
};

// A buffer resource over [base, base + bytes): loads at offsets at or past `bytes` return zero.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t lr_rsrc(const void *base, int64_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0, (int)bytes, 0x00020000);
}

// An offset past every resource the branch builds (they stay below 2^31 bytes): the load returns 0.
constexpr uint32_t kLrOob = 0x80000000u;

__device__ __forceinline__ bf16x8 lr_load(__amdgpu_buffer_rsrc_t r, uint32_t off) {
    return __builtin_bit_cast(bf16x8, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0));
}

}  // namespace nvfp4
