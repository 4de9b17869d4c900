// Quality statistics of one weight matrix and its NVFP4 form, in one pass over both
// ("Qwen-Image NVFP4 on a 16 GB Ada GPU", section "Quality: the error of each matrix": the relative
// error of each matrix, its kurtosis, and the ratio of the maximum to the standard deviation in
// blocks of 64).
//
//   rel_error  = ||W - W_hat||_F / ||W||_F, W_hat the exact expansion e2m1 x s x g (in double);
//   kurtosis   = m4 / m2^2 - 3 with population central moments, from the power sums S1..S4 of
//                w - c accumulated in double, c = w[0][0] (the shift keeps the cancellation in the
//                central moments small unless the first element is far out in the tail);
//   block ratio = mean over blocks of 64 consecutive elements (row-major order; the last block may
//                be shorter) of max |w| / population std of the block, blocks with std 0 left out;
//   also the mean, the population std and max |w|.
//
// Work unit: one 16-element NVFP4 block per lane (row-major block index u, so its elements are
// 16u .. 16u + 15 of the flattened matrix and its codes are bytes 8u .. 8u + 7 of the dense code
// array).  A wave takes 64 consecutive units per pass, so the four lanes 4k .. 4k + 3 hold one block
// of 64 and finish its mean and spread with two shuffles each.  Each workgroup writes its partial
// sums to the workspace; one workgroup then adds them in a fixed order (deterministic) and forms
// the statistics.
#include <hip/hip_runtime.h>

#include "common.h"
#include "internal.h"

namespace nvfp4 {

// S1..S4 of w - c, sum w^2, sum (w - w_hat)^2, sum of block ratios, blocks, max |w|
constexpr int kStatFields = 9;

__device__ __forceinline__ double shfl_xor_f64(double v, int m) {
    const uint64_t u = __builtin_bit_cast(uint64_t, v);
    const uint32_t lo = (uint32_t)__shfl_xor((int)(uint32_t)u, m, 64);
    const uint32_t hi = (uint32_t)__shfl_xor((int)(uint32_t)(u >> 32), m, 64);
    return __builtin_bit_cast(double, ((uint64_t)hi << 32) | lo);
}

template <int SRC>
__device__ __forceinline__ void load_unit(const uint8_t *x, int64_t cols, int64_t ld_bytes, int64_t u, float (&v)[16]) {
    const int64_t e = u * 16;
    const int64_t r = e / cols, c = e - r * cols;
    if constexpr (SRC == NVFP4_F32) {
        const u32x4 *p = reinterpret_cast<const u32x4 *>(x + r * ld_bytes + c * 4);
#pragma unroll
        for (int q = 0; q < 4; q++) {
            const u32x4 w = p[q];
#pragma unroll
            for (int i = 0; i < 4; i++) v[q * 4 + i] = u2f(w[i]);
        }
    } else {
        const u32x4 *p = reinterpret_cast<const u32x4 *>(x + r * ld_bytes + c * 2);
#pragma unroll
        for (int q = 0; q < 2; q++) {
            const u32x4 w = p[q];
#pragma unroll
            for (int i = 0; i < 4; i++) {
                if constexpr (SRC == NVFP4_BF16) {
                    v[q * 8 + 2 * i] = u2f(w[i] << 16);
                    v[q * 8 + 2 * i + 1] = u2f(w[i] & 0xFFFF0000u);
                } else {
                    v[q * 8 + 2 * i] = (float)__builtin_bit_cast(_Float16, (uint16_t)(w[i] & 0xFFFFu));
                    v[q * 8 + 2 * i + 1] = (float)__builtin_bit_cast(_Float16, (uint16_t)(w[i] >> 16));
                }
            }
        }
    }
}

template <int SRC, bool HAS_Q>
__global__ __launch_bounds__(256) void k_stats(const uint8_t *__restrict__ x, int64_t cols, int64_t ld_bytes,
                                               int64_t units, const uint8_t *__restrict__ codes,
                                               const uint8_t *__restrict__ scales, const float *__restrict__ g,
                                               double *__restrict__ partials) {
    __shared__ double red[4][kStatFields];
    const int lane = threadIdx.x & 63, wid = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const double gd = HAS_Q ? (double)*g : 0.0;
    float c0[16];
    load_unit<SRC>(x, cols, ld_bytes, 0, c0);
    const double shift = (double)c0[0];
    double s1 = 0, s2 = 0, s3 = 0, s4 = 0, w2 = 0, d2 = 0, rsum = 0, nblk = 0;
    float amax = 0.0f;
    const int64_t nwaves = (int64_t)gridDim.x * 4;
    const int64_t n = units * 16;
    for (int64_t base = ((int64_t)blockIdx.x * 4 + wid) * 64; base < units; base += nwaves * 64) {
        const int64_t u = base + lane;
        const bool valid = u < units;
        float v[16];
        if (valid) {
            load_unit<SRC>(x, cols, ld_bytes, u, v);
        } else {
#pragma unroll
            for (int i = 0; i < 16; i++) v[i] = 0.0f;
        }
        // lanes past the end hold zeros and shift by 0, so they add nothing
        const double sh = valid ? shift : 0.0;
        double b1 = 0.0;  // sum of w over the unit: the block mean comes from the raw values, so a
        float bmax = 0.0f;  // constant block gets its own value as mean and a spread of exactly 0
#pragma unroll
        for (int i = 0; i < 16; i++) {
            const double w = (double)v[i];
            const double d = w - sh;
            const double dd = d * d;
            b1 += w;
            s2 += dd;
            s3 += dd * d;
            s4 += dd * dd;
            w2 += w * w;
            bmax = fmaxf(bmax, fabsf(v[i]));
        }
        s1 += b1 - 16.0 * sh;
        if constexpr (HAS_Q) {
            if (valid) {
                const u32x2 cw = *reinterpret_cast<const u32x2 *>(codes + u * 8);
                const float s = e4m3_to_f32(scales[u]);
                float e[16];
                fp4_unpack8_f32(cw[0], e);
                fp4_unpack8_f32(cw[1], e + 8);
#pragma unroll
                for (int i = 0; i < 16; i++) {
                    const double d = (double)v[i] - (double)(e[i] * s) * gd;  // e2m1 x s is exact in fp32
                    d2 += d * d;
                }
            }
        }
        amax = fmaxf(amax, bmax);
        // block of 64: lanes 4k .. 4k + 3; elements past the end of the matrix are not counted
        double bsum = b1 + shfl_xor_f64(b1, 1);
        bsum += shfl_xor_f64(bsum, 2);
        float bm = fmaxf(bmax, __shfl_xor(bmax, 1, 64));
        bm = fmaxf(bm, __shfl_xor(bm, 2, 64));
        const int64_t first = (u & ~(int64_t)3) * 16;
        const double cnt = (double)((n - first) < 64 ? (n - first) : 64);
        const double mu = first < n ? bsum / cnt : 0.0;  // the block's mean
        double sq = 0.0;
        if (valid) {
#pragma unroll
            for (int i = 0; i < 16; i++) {
                const double d = (double)v[i] - mu;
                sq += d * d;
            }
        }
        sq += shfl_xor_f64(sq, 1);
        sq += shfl_xor_f64(sq, 2);
        const double sd = sqrt(sq / cnt);
        if ((lane & 3) == 0 && first < n && sd > 0.0) {
            rsum += (double)bm / sd;
            nblk += 1.0;
        }
    }
    // wave sums, then the workgroup's
    double acc[kStatFields] = {s1, s2, s3, s4, w2, d2, rsum, nblk, (double)amax};
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) {
#pragma unroll
        for (int f = 0; f < kStatFields - 1; f++) acc[f] += shfl_xor_f64(acc[f], o);
        acc[kStatFields - 1] = fmax(acc[kStatFields - 1], shfl_xor_f64(acc[kStatFields - 1], o));
    }
    if (lane == 0)
#pragma unroll
        for (int f = 0; f < kStatFields; f++) red[wid][f] = acc[f];
    __syncthreads();
    if (threadIdx.x < kStatFields) {
        const int f = threadIdx.x;
        double r = red[0][f];
        for (int w = 1; w < 4; w++) r = f == kStatFields - 1 ? fmax(r, red[w][f]) : r + red[w][f];
        partials[(int64_t)blockIdx.x * kStatFields + f] = r;
    }
}

// One workgroup: the partial sums in a fixed order, then the statistics.
__global__ __launch_bounds__(256) void k_stats_final(const double *__restrict__ partials, int nparts, int64_t n,
                                                     const uint8_t *__restrict__ x, int src, int has_q,
                                                     double *__restrict__ out) {
    __shared__ double red[256];
    __shared__ double tot[kStatFields];
    for (int f = 0; f < kStatFields; f++) {
        double r = 0.0;  // sums start at 0; so does the maximum of |w|
        for (int i = threadIdx.x; i < nparts; i += 256) {
            const double v = partials[(int64_t)i * kStatFields + f];
            r = f == kStatFields - 1 ? fmax(r, v) : r + v;
        }
        red[threadIdx.x] = r;
        __syncthreads();
        for (int o = 128; o >= 1; o >>= 1) {
            if (threadIdx.x < o)
                red[threadIdx.x] = f == kStatFields - 1 ? fmax(red[threadIdx.x], red[threadIdx.x + o])
                                                        : red[threadIdx.x] + red[threadIdx.x + o];
            __syncthreads();
        }
        if (threadIdx.x == 0) tot[f] = red[0];
        __syncthreads();
    }
    if (threadIdx.x == 0) {
        const double shift = src == NVFP4_F32   ? (double)u2f(*reinterpret_cast<const uint32_t *>(x))
                             : src == NVFP4_BF16 ? (double)u2f((uint32_t)*reinterpret_cast<const uint16_t *>(x) << 16)
                                                 : (double)__builtin_bit_cast(_Float16, *reinterpret_cast<const uint16_t *>(x));
        // central moments of w from the moments e1..e4 of w - c about 0
        const double nn = (double)n;
        const double e1 = tot[0] / nn, e2 = tot[1] / nn, e3 = tot[2] / nn, e4 = tot[3] / nn;
        const double m2 = e2 - e1 * e1;
        const double m4 = e4 - 4.0 * e1 * e3 + 6.0 * e1 * e1 * e2 - 3.0 * e1 * e1 * e1 * e1;
        out[0] = has_q ? sqrt(tot[5]) / sqrt(tot[4]) : __builtin_nan("");
        out[1] = m4 / (m2 * m2) - 3.0;
        out[2] = tot[7] > 0.0 ? tot[6] / tot[7] : __builtin_nan("");
        out[3] = shift + e1;
        out[4] = sqrt(m2 > 0.0 ? m2 : 0.0);
        out[5] = tot[8];
        out[6] = tot[7];
    }
}

size_t stats_ws_bytes() { return (size_t)kStatsMaxGroups * kStatFields * sizeof(double); }

template <int SRC>
static void launch_stats_t(const void *x, int64_t rows, int64_t cols, int64_t ld_x, const nvfp4_tensor *q,
                           double *out, double *partials, int num_cus, hipStream_t stream) {
    constexpr int EB = SRC == NVFP4_F32 ? 4 : 2;
    const int64_t units = rows * cols / 16;
    int64_t grid = (units + 255) / 256;
    const int64_t cap = (int64_t)num_cus * 4 < kStatsMaxGroups ? (int64_t)num_cus * 4 : kStatsMaxGroups;
    if (grid > cap) grid = cap;
    if (grid < 1) grid = 1;
    if (q)
        hipLaunchKernelGGL((k_stats<SRC, true>), dim3((unsigned)grid), dim3(256), 0, stream, (const uint8_t *)x, cols,
                           ld_x * EB, units, q->codes, q->scales, q->global_scale, partials);
    else
        hipLaunchKernelGGL((k_stats<SRC, false>), dim3((unsigned)grid), dim3(256), 0, stream, (const uint8_t *)x,
                           cols, ld_x * EB, units, nullptr, nullptr, nullptr, partials);
    hipLaunchKernelGGL(k_stats_final, dim3(1), dim3(256), 0, stream, partials, (int)grid, rows * cols,
                       (const uint8_t *)x, SRC, q ? 1 : 0, out);
}

hipError_t launch_stats(const void *x, nvfp4_dtype dt, int64_t rows, int64_t cols, int64_t ld_x,
                        const nvfp4_tensor *q, double *out, void *workspace, int num_cus, hipStream_t stream) {
    double *partials = reinterpret_cast<double *>(workspace);
    switch (dt) {
    case NVFP4_F32: launch_stats_t<NVFP4_F32>(x, rows, cols, ld_x, q, out, partials, num_cus, stream); break;
    case NVFP4_BF16: launch_stats_t<NVFP4_BF16>(x, rows, cols, ld_x, q, out, partials, num_cus, stream); break;
    default: launch_stats_t<NVFP4_F16>(x, rows, cols, ld_x, q, out, partials, num_cus, stream); break;
    }
    return hipGetLastError();
}

}  // namespace nvfp4
