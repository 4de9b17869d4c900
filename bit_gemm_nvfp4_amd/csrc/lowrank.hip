// The two passes of the bf16 low-rank branch that do not live inside the NVFP4 GEMM's epilogue
// ("Qwen Image 2.1: INT4 + FP4", section "What I quantized": FP4 weights with BF16 rank-128
// branches; the branch adds (A . V^T) . U^T to the layer's product).
//
// k_lr_down: T = A . V^T [M x r] on the bf16 matrix cores, written as the bf16 pair T_hi, T_lo
//   (64 x 32 blocks of T, operands staged in LDS with contiguous row reads).
// k_lr_up_add: C += T . U^T for products that do not take the fused epilogue (the GEMV for M <= 5,
//   K % 64 != 0, split-K): a 32 x 128 tile per workgroup, then a read-modify-write of C.
#include <hip/hip_runtime.h>

#include "common.h"
#include "internal.h"
#include "lowrank.h"

namespace nvfp4 {

constexpr int kLrDownBM = 64;   // rows of A per workgroup
constexpr int kLrDownBN = 32;   // columns of T per workgroup
constexpr int kLrDownKC = 128;  // K per staged chunk
constexpr int kLrDownRow = kLrDownKC + 8;  // padded LDS row (bf16): fragment reads spread over banks
constexpr int kLrDownSPW = kLrDownKC / 16 / 4;  // 16-deep slices of a chunk per wave

// A workgroup (4 waves) computes a 64 x 32 block of T over the whole of K.  Chunks of 128 of K of
// its A rows and V rows are loaded with whole 16-byte pieces per lane (rows read contiguously),
// staged in LDS (two buffers: the next chunk's loads are in flight while the current one is
// multiplied), and read back as matrix fragments; wave w multiplies its quarter of each chunk's
// 16-deep slices into its own two 32 x 32 accumulators, and the four waves' sums are added in LDS
// in wave order (fixed, so the result does not depend on timing).  Workgroups that share rows of
// A are numbered to land on one XCD at about the same time, so those rows come from its L2.
__global__ __launch_bounds__(256) void k_lr_down(const __bf16 *__restrict__ A, int64_t lda,
                                                 const __bf16 *__restrict__ V, int64_t M, int64_t K, int r,
                                                 __bf16 *__restrict__ T) {
    constexpr int A_UNITS = kLrDownBM * (kLrDownKC / 8) / 256;  // 16-byte pieces per thread per chunk
    constexpr int V_UNITS = kLrDownBN * (kLrDownKC / 8) / 256;
    constexpr int STAGE = (kLrDownBM + kLrDownBN) * kLrDownRow;   // bf16 per LDS buffer
    static_assert(A_UNITS * 256 == kLrDownBM * (kLrDownKC / 8) && V_UNITS * 256 == kLrDownBN * (kLrDownKC / 8),
                  "the pieces of a chunk cover the tile's rows exactly");
    __shared__ __attribute__((aligned(16))) __bf16 lds[2 * STAGE > 4 * 2 * 16 * 64 * 2 ? 2 * STAGE : 4 * 2 * 16 * 64 * 2];
    const int tid = threadIdx.x, lane = tid & 63, wid = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int l32 = lane & 31, kh = (lane >> 5) * 8;
    // workgroup -> (row block, column block): the column blocks of one row block share id % 8
    const int nrb = (int)((M + kLrDownBM - 1) / kLrDownBM), ncb = (r + kLrDownBN - 1) / kLrDownBN;
    const int xcd = blockIdx.x % 8, j = blockIdx.x / 8;
    const int rb = (j / ncb) * 8 + xcd, cbk = j % ncb;
    if (rb >= nrb) return;
    const int64_t m0 = (int64_t)rb * kLrDownBM;
    const int c0 = cbk * kLrDownBN;
    const int64_t mrows = (M - m0) < kLrDownBM ? (M - m0) : kLrDownBM;
    const int vrows = (r - c0) < kLrDownBN ? (r - c0) : kLrDownBN;
    const __amdgpu_buffer_rsrc_t ra = lr_rsrc(A + m0 * lda, ((mrows - 1) * lda + K) * 2);
    const __amdgpu_buffer_rsrc_t rv = lr_rsrc(V + (int64_t)c0 * K, (int64_t)vrows * K * 2);
    // this thread's pieces: piece u = tid + 256 q -> row u / (KC / 8), 8 elements at (u % (KC / 8)) * 8
    uint32_t a_off[A_UNITS], v_off[V_UNITS], a_lds[A_UNITS], v_lds[V_UNITS];
    uint32_t a_k[A_UNITS], v_k[V_UNITS];
#pragma unroll
    for (int q = 0; q < A_UNITS; q++) {
        const int u = tid + 256 * q, row = u / (kLrDownKC / 8), c8 = (u % (kLrDownKC / 8)) * 8;
        a_off[q] = (uint32_t)(row * lda + c8) * 2;
        a_k[q] = (uint32_t)c8;
        a_lds[q] = (uint32_t)(row * kLrDownRow + c8);
    }
#pragma unroll
    for (int q = 0; q < V_UNITS; q++) {
        const int u = tid + 256 * q, row = u / (kLrDownKC / 8), c8 = (u % (kLrDownKC / 8)) * 8;
        v_off[q] = (uint32_t)((int64_t)row * K + c8) * 2;
        v_k[q] = (uint32_t)c8;
        v_lds[q] = (uint32_t)((kLrDownBM + row) * kLrDownRow + c8);
    }
    // four register sets of loads: three chunks stay in flight while one is multiplied (eight
    // sets, or chunks of 256, measured no faster)
    constexpr int NSET = 4;
    bf16x8 ga[NSET][A_UNITS], gv[NSET][V_UNITS];
    // chunks past K load zeros, so the loads carry no branches (and the waits stay exact)
    auto load = [&](int set, int64_t k0) {
#pragma unroll
        for (int q = 0; q < A_UNITS; q++)
            ga[set][q] = lr_load(ra, k0 + a_k[q] < (uint64_t)K ? a_off[q] + (uint32_t)k0 * 2 : kLrOob);
#pragma unroll
        for (int q = 0; q < V_UNITS; q++)
            gv[set][q] = lr_load(rv, k0 + v_k[q] < (uint64_t)K ? v_off[q] + (uint32_t)k0 * 2 : kLrOob);
    };
    auto store = [&](int set, int buf) {
        __bf16 *st = lds + buf * STAGE;
#pragma unroll
        for (int q = 0; q < A_UNITS; q++) *reinterpret_cast<bf16x8 *>(st + a_lds[q]) = ga[set][q];
#pragma unroll
        for (int q = 0; q < V_UNITS; q++) *reinterpret_cast<bf16x8 *>(st + v_lds[q]) = gv[set][q];
    };
    f32x16 acc[2];
    acc[0] = f32x16{};
    acc[1] = f32x16{};
    auto mma = [&](int buf) {
        const __bf16 *st = lds + buf * STAGE;
#pragma unroll
        for (int s = 0; s < kLrDownSPW; s++) {
            const int kk = (kLrDownSPW * wid + s) * 16 + kh;
            const bf16x8 fv = *reinterpret_cast<const bf16x8 *>(st + (kLrDownBM + l32) * kLrDownRow + kk);
#pragma unroll
            for (int i = 0; i < 2; i++) {
                const bf16x8 fa = *reinterpret_cast<const bf16x8 *>(st + (i * 32 + l32) * kLrDownRow + kk);
                acc[i] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa, fv, acc[i], 0, 0, 0);
            }
        }
    };
    // chunk c is multiplied from LDS buffer c % 2 and was loaded into register set c % NSET
    const int64_t nchunks = (K + kLrDownKC - 1) / kLrDownKC;
#pragma unroll
    for (int set = 0; set < NSET; set++) load(set, (int64_t)set * kLrDownKC);
    store(0, 0);
    load(0, (int64_t)NSET * kLrDownKC);
    __syncthreads();
    auto step = [&](int64_t c, int set_next) {  // set_next = (c + 1) % NSET
        mma((int)(c & 1));
        store(set_next, (int)((c + 1) & 1));
        load(set_next, (c + 1 + NSET) * kLrDownKC);
        __syncthreads();
    };
    // whole rounds of NSET: chunks past the end are zeros (no branches, so the waits stay exact)
    for (int64_t c = 0; c < nchunks; c += NSET) {
#pragma unroll
        for (int i = 0; i < NSET; i++) step(c + i, (i + 1) % NSET);
    }
    // the four waves' partial tiles, as [wave][tile][element][lane], summed in wave order
    float *red = reinterpret_cast<float *>(lds);
#pragma unroll
    for (int i = 0; i < 2; i++)
#pragma unroll
        for (int e = 0; e < 16; e++) red[((wid * 2 + i) * 16 + e) * 64 + lane] = acc[i][e];
    __syncthreads();
    const int64_t plane = M * (int64_t)r;
    for (int idx = tid; idx < 2 * 16 * 64; idx += 256) {
        const int i = idx / 1024, e = (idx / 64) % 16, ln = idx % 64;
        const int64_t trow = m0 + i * 32 + 8 * (e / 4) + 4 * (ln >> 5) + (e % 4);
        const int tcol = c0 + (ln & 31);
        if (trow < M && tcol < r) {
            float v = red[idx];
            for (int w = 1; w < 4; w++) v += red[w * 2048 + idx];
            const __bf16 hi = (__bf16)v;
            T[trow * r + tcol] = hi;
            T[plane + trow * r + tcol] = (__bf16)(v - (float)hi);
        }
    }
}

// C[M x N] += T . U^T; 4 waves, each a 32 x 32 tile of a 32 x 128 block, slices of 16 ranks in
// pairs with the next pair's loads in flight.
__global__ __launch_bounds__(256) void k_lr_up_add(LrArgs lr, int64_t M, int64_t N, float *__restrict__ C,
                                                   int64_t ldc) {
    const int lane = threadIdx.x & 63, wid = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int l32 = lane & 31, kh = (lane >> 5) * 8;
    const int r = lr.r;
    const int64_t row0 = (int64_t)blockIdx.x * 32, col0 = (int64_t)blockIdx.y * 128 + wid * 32;
    if (col0 >= N) return;
    const int64_t mrows = (M - row0) < 32 ? (M - row0) : 32;
    const int64_t ncols = (N - col0) < 32 ? (N - col0) : 32;
    const __amdgpu_buffer_rsrc_t rh = lr_rsrc(lr.t + row0 * r, mrows * r * 2);
    const __amdgpu_buffer_rsrc_t rl = lr_rsrc(lr.t + M * (int64_t)r + row0 * r, mrows * r * 2);
    const __amdgpu_buffer_rsrc_t ru = lr_rsrc(lr.u + col0 * r, ncols * r * 2);
    const uint32_t off = (uint32_t)(l32 * r + kh) * 2;
    f32x16 acc = {};
    bf16x8 ah[2], al[2], bu[2];
    auto load = [&](int buf, int kc) {
        const uint32_t o = kc < r ? off + (uint32_t)kc * 2 : kLrOob;
        ah[buf] = lr_load(rh, o);
        al[buf] = lr_load(rl, o);
        bu[buf] = lr_load(ru, o);
    };
    auto mma = [&](int buf) {
        acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ah[buf], bu[buf], acc, 0, 0, 0);
        acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(al[buf], bu[buf], acc, 0, 0, 0);
    };
    load(0, 0);
    for (int kc = 0; kc < r; kc += 32) {
        load(1, kc + 16);
        __builtin_amdgcn_sched_barrier(0);
        mma(0);
        __builtin_amdgcn_sched_barrier(0);
        load(0, kc + 32);
        __builtin_amdgcn_sched_barrier(0);
        mma(1);  // zeros when kc + 16 >= r
        __builtin_amdgcn_sched_barrier(0);
    }
    const int64_t col = col0 + l32;
    if (col < N) {
#pragma unroll
        for (int e = 0; e < 16; e++) {
            const int64_t row = row0 + 8 * (e / 4) + 4 * (lane >> 5) + (e % 4);
            if (row < M) C[row * ldc + col] += acc[e];
        }
    }
}

size_t lowrank_t_bytes(int64_t M) {
    // T_hi and T_lo at the largest rank, rounded up to keep what follows 256-byte aligned
    return ((size_t)M * kLrMaxRank * 2 * sizeof(__bf16) + 255) / 256 * 256;
}

hipError_t launch_lowrank_down(const void *a_bf16, int64_t lda, const void *v, int64_t M, int64_t K, int r,
                               void *t, hipStream_t stream) {
    const int64_t nrb = (M + kLrDownBM - 1) / kLrDownBM, ncb = (r + kLrDownBN - 1) / kLrDownBN;
    const dim3 grid((unsigned)((nrb + 7) / 8 * 8 * ncb));
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
