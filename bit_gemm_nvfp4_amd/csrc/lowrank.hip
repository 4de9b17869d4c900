// The two passes of the bf16 low-rank branch that do not live inside the NVFP4 GEMM's epilogue
// ("Qwen Image 2.1: INT4 + FP4", section "What I quantized": FP4 weights with BF16 rank-128
// branches; the branch adds (A . V^T) . U^T to the layer's product).
//
// k_lr_down: T = A . V^T [M x r] on the bf16 matrix cores, written as the bf16 pair T_hi, T_lo.
//   A workgroup takes 32 rows of A and up to 128 columns of T (one 32-wide column block per wave,
//   the waves of a workgroup share the A fragments through L1) over the whole of K, so A streams
//   from HBM once.  Each wave keeps four 16-deep slices of loads in flight ahead of its matrix
//   instructions.
// k_lr_up_add: C += T . U^T for products that do not take the fused epilogue (the GEMV for M <= 4,
//   K % 64 != 0, split-K): a 32 x 128 tile per workgroup, then a read-modify-write of C.
#include <hip/hip_runtime.h>

#include "common.h"
#include "internal.h"
#include "lowrank.h"

namespace nvfp4 {

constexpr int kLrDownSlices = 4;  // 16-deep slices per prefetch group (64 of K)

__global__ __launch_bounds__(256) void k_lr_down(const __bf16 *__restrict__ A, int64_t lda, const __bf16 *__restrict__ V,
                                                 int64_t M, int64_t K, int r, __bf16 *__restrict__ T) {
    const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
    const int l32 = lane & 31, kh = (lane >> 5) * 8;
    const int64_t row = (int64_t)blockIdx.x * 32 + l32;   // A row of this lane's fragments
    const int col = blockIdx.y * 128 + wid * 32 + l32;    // V row (T column) of this lane's fragments
    if (blockIdx.y * 128 + wid * 32 >= r) return;         // wave with no columns (r % 128 != 0)
    const bool row_ok = row < M, col_ok = col < r;
    const __bf16 *pa = A + (row_ok ? row : 0) * lda + kh;
    const __bf16 *pv = V + (int64_t)(col_ok ? col : 0) * K + kh;
    const bf16x8 zero = {};
    f32x16 acc = {};
    bf16x8 fa[2][kLrDownSlices], fv[2][kLrDownSlices];
    auto load = [&](int buf, int64_t k0) {
#pragma unroll
        for (int s = 0; s < kLrDownSlices; s++) {
            const int64_t k = k0 + 16 * s;
            const bool in = k < K;
            fa[buf][s] = row_ok && in ? *reinterpret_cast<const bf16x8 *>(pa + k) : zero;
            fv[buf][s] = col_ok && in ? *reinterpret_cast<const bf16x8 *>(pv + k) : zero;
        }
    };
    auto mma = [&](int buf) {
#pragma unroll
        for (int s = 0; s < kLrDownSlices; s++)
            acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[buf][s], fv[buf][s], acc, 0, 0, 0);
    };
    constexpr int64_t G = 16 * kLrDownSlices;
    load(0, 0);
    for (int64_t k0 = 0; k0 < K; k0 += 2 * G) {
        if (k0 + G < K) load(1, k0 + G);
        mma(0);
        if (k0 + G >= K) break;
        if (k0 + 2 * G < K) load(0, k0 + 2 * G);
        mma(1);
    }
    // acc element e: row 8 (e / 4) + 4 (lane / 32) + e % 4 of the tile, column lane % 32
    const int64_t plane = M * (int64_t)r;
    const int tcol = blockIdx.y * 128 + wid * 32 + l32;
    if (tcol < r) {
#pragma unroll
        for (int e = 0; e < 16; e++) {
            const int64_t trow = (int64_t)blockIdx.x * 32 + 8 * (e / 4) + 4 * (lane >> 5) + (e % 4);
            if (trow < M) {
                const float t = acc[e];
                const __bf16 hi = (__bf16)t;
                T[trow * r + tcol] = hi;
                T[plane + trow * r + tcol] = (__bf16)(t - (float)hi);
            }
        }
    }
}

// C[M x N] += T . U^T; 4 waves, each a 32 x 32 tile of a 32 x 128 block.
__global__ __launch_bounds__(256) void k_lr_up_add(LrArgs lr, int64_t M, int64_t N, float *__restrict__ C,
                                                   int64_t ldc) {
    const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
    const int64_t row0 = (int64_t)blockIdx.x * 32, col0 = (int64_t)blockIdx.y * 128 + wid * 32;
    if (col0 >= N) return;
    f32x16 acc[1][1];
    acc[0][0] = f32x16{};
    lr_branch<1, 1>(acc, lr, M, N, row0, col0, lane);
    const int64_t col = col0 + (lane & 31);
    if (col < N) {
#pragma unroll
        for (int e = 0; e < 16; e++) {
            const int64_t row = row0 + 8 * (e / 4) + 4 * (lane >> 5) + (e % 4);
            if (row < M) C[row * ldc + col] += acc[0][0][e];
        }
    }
}

size_t lowrank_t_bytes(int64_t M) {
    // T_hi and T_lo at the largest rank, rounded up to keep what follows 256-byte aligned
    return ((size_t)M * kLrMaxRank * 2 * sizeof(__bf16) + 255) / 256 * 256;
}

hipError_t launch_lowrank_down(const void *a_bf16, int64_t lda, const void *v, int64_t M, int64_t K, int r,
                               void *t, hipStream_t stream) {
    const dim3 grid((unsigned)((M + 31) / 32), (unsigned)((r + 127) / 128));
    hipLaunchKernelGGL(k_lr_down, grid, dim3(256), 0, stream, (const __bf16 *)a_bf16, lda, (const __bf16 *)v, M, K, r,
                       (__bf16 *)t);
    return hipGetLastError();
}

hipError_t launch_lowrank_up_add(const void *t, const void *u, int r, int64_t M, int64_t N, float *c, int64_t ldc,
                                 hipStream_t stream) {
    const LrArgs lr{(const __bf16 *)t, (const __bf16 *)u, r};
    const dim3 grid((unsigned)((M + 31) / 32), (unsigned)((N + 127) / 128));
    hipLaunchKernelGGL(k_lr_up_add, grid, dim3(256), 0, stream, lr, M, N, c, ldc);
    return hipGetLastError();
}

}  // namespace nvfp4
