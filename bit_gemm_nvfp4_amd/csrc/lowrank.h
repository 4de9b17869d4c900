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

// Branch operands of the up-projection: T_hi / T_lo [M x r] bf16 (dense, plane stride M * r) and
// U [N x r] bf16 (dense).
struct LrArgs {
    const __bf16 *t;  // T_hi; T_lo follows at t + M * r
    const __bf16 *u;
    int r;
};

// acc[i][j] += T . U^T for the 32 x 32 tiles (row0 + 32 i, col0 + 32 j) of one wave, in the operand
// layout of v_mfma_f32_32x32x16_bf16 (lane l: row or column l % 32, the eight k at 8 (l / 32)).
// Rows past M and columns past N read zeros.  The operands of slice k + 16 are loaded before the
// matrix instructions of slice k.
template <int TM, int TN>
__device__ __forceinline__ void lr_branch(f32x16 (&acc)[TM][TN], const LrArgs &lr, int64_t M, int64_t N,
                                          int64_t row0, int64_t col0, int lane) {
    const int l32 = lane & 31, kh = (lane >> 5) * 8;
    const int r = lr.r;
    const __bf16 *tlo = lr.t + M * (int64_t)r;
    const bf16x8 zero = {};
    bf16x8 ah[2][TM], al[2][TM], b[2][TN];
    auto load = [&](int buf, int kc) {
#pragma unroll
        for (int i = 0; i < TM; i++) {
            const int64_t row = row0 + i * 32 + l32;
            const int64_t off = row * r + kc + kh;
            ah[buf][i] = row < M ? *reinterpret_cast<const bf16x8 *>(lr.t + off) : zero;
            al[buf][i] = row < M ? *reinterpret_cast<const bf16x8 *>(tlo + off) : zero;
        }
#pragma unroll
        for (int j = 0; j < TN; j++) {
            const int64_t col = col0 + j * 32 + l32;
            b[buf][j] = col < N ? *reinterpret_cast<const bf16x8 *>(lr.u + col * r + kc + kh) : zero;
        }
    };
    auto mma = [&](int buf) {
#pragma unroll
        for (int i = 0; i < TM; i++)
#pragma unroll
            for (int j = 0; j < TN; j++) {
                acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ah[buf][i], b[buf][j], acc[i][j], 0, 0, 0);
                acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(al[buf][i], b[buf][j], acc[i][j], 0, 0, 0);
            }
    };
    load(0, 0);
    int kc = 0;
    for (; kc + 32 <= r; kc += 32) {
        load(1, kc + 16);
        mma(0);
        if (kc + 32 < r) load(0, kc + 32);
        mma(1);
    }
    if (kc < r) mma(0);  // r % 32 == 16: the last slice
}

}  // namespace nvfp4
