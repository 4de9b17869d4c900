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
// of 64 and finish its mean and spread with two quad shuffles each.  Each workgroup writes its
// partial sums to the workspace; one workgroup then adds them in a fixed order (deterministic) and
// forms the statistics.
//
// Bound: with double-precision sums the kernel does about ten double operations per element (its
// unit's four power sums, the conversion, the error term), which at MI355X's vector fp64 rate
// costs about as long as reading a bf16 matrix from HBM; an f32 matrix is bound by HBM.
#include <hip/hip_runtime.h>

#include "common.h"
#include "internal.h"

namespace nvfp4 {

// S1..S4 of w - c, sum w^2, sum (w - w_hat)^2, sum of block ratios, blocks, max |w|
constexpr int kStatFields = 9;
constexpr int kFinalThreads = 256;

// Exchange with the lane whose index differs in bit 0 (XOR1) or bit 1 (XOR2) of the quad (DPP).
constexpr int kQuadXor1 = 0xB1, kQuadXor2 = 0x4E;
template <int CTRL>
__device__ __forceinline__ double quad_xor_f64(double v) {
    const uint64_t u = __builtin_bit_cast(uint64_t, v);
    const uint32_t lo = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)(uint32_t)u, CTRL, 0xF, 0xF, false);
    const uint32_t hi = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)(uint32_t)(u >> 32), CTRL, 0xF, 0xF, false);
    return __builtin_bit_cast(double, ((uint64_t)hi << 32) | lo);
}
template <int CTRL>
__device__ __forceinline__ float quad_xor_f32(float v) {
    return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL, 0xF, 0xF, false));
}

__device__ __forceinline__ double shfl_xor_f64(double v, int m) {
    const uint64_t u = __builtin_bit_cast(uint64_t, v);
    const uint32_t lo = (uint32_t)__shfl_xor((int)(uint32_t)u, m, 64);
    const uint32_t hi = (uint32_t)__shfl_xor((int)(uint32_t)(u >> 32), m, 64);
    return __builtin_bit_cast(double, ((uint64_t)hi << 32) | lo);
}

// Wave-iterations each wave has in flight: enough bytes per wave to cover the memory latency,
// within the registers that keep four waves per SIMD.
template <int SRC>
constexpr int kStatsItersInFlight = SRC == NVFP4_F32 ? 1 : 2;

// Raw words of one unit: 16 source elements, and its 8 code bytes and scale byte.
template <int SRC>
struct Unit {
    static constexpr int EB = SRC == NVFP4_F32 ? 4 : 2;
    static constexpr int W = 4 * EB;
    uint32_t x[W];
    u32x2 codes;
    uint32_t scale;
};

// Position of a wave-iteration's first unit: its unit index and the (row, column) of its first
// element, all wave-uniform; advanced by a fixed step with no division.
struct WavePos {
    int64_t u, r, c;
    __device__ __forceinline__ void advance(int64_t step_units, int64_t step_r, int64_t step_c, int64_t cols) {
        u += step_units;
        r += step_r;
        c += step_c;
        if (c >= cols) {
            c -= cols;
            r += 1;
        }
    }
};

// Loads the unit of this lane in the wave-iteration at p (zeros past the end).  A unit never
// straddles rows (cols % 16 == 0).  A dense matrix (row stride == cols) is addressed linearly;
// otherwise the unit's offset from the wave-iteration's first element is split into whole rows
// and a column with a 32-bit division.
template <int SRC, bool HAS_Q, bool DENSE>
__device__ __forceinline__ void load_unit(Unit<SRC> &d, const WavePos &p, int lane, int64_t units,
                                          const uint8_t *__restrict__ x, uint32_t cols, int64_t ld_bytes,
                                          const uint8_t *__restrict__ codes, const uint8_t *__restrict__ scales) {
    using U = Unit<SRC>;
    const int64_t u = p.u + lane;
    if (u >= units) {
#pragma unroll
        for (int i = 0; i < U::W; i++) d.x[i] = 0;
        d.codes = u32x2{0, 0};
        d.scale = 0;
        return;
    }
    const uint8_t *a;
    if constexpr (DENSE) {
        a = x + u * 16 * U::EB;
    } else {
        const uint32_t e = (uint32_t)p.c + 16u * (uint32_t)lane;
        const uint32_t qr = e / cols, c = e - qr * cols;
        a = x + (p.r + qr) * ld_bytes + (int64_t)c * U::EB;
    }
    const u32x4 *src = reinterpret_cast<const u32x4 *>(a);
#pragma unroll
    for (int q = 0; q < U::W / 4; q++) {
        const u32x4 w = src[q];
#pragma unroll
        for (int i = 0; i < 4; i++) d.x[q * 4 + i] = w[i];
    }
    if constexpr (HAS_Q) {
        d.codes = *reinterpret_cast<const u32x2 *>(codes + u * 8);
        d.scale = scales[u];
    }
}

// w[0][0], the shift of the power sums
template <int SRC>
__device__ __forceinline__ double first_value(const uint8_t *x) {
    if constexpr (SRC == NVFP4_F32) return (double)u2f(*reinterpret_cast<const uint32_t *>(x));
    else if constexpr (SRC == NVFP4_BF16) return (double)u2f((uint32_t)*reinterpret_cast<const uint16_t *>(x) << 16);
    else return (double)(float)__builtin_bit_cast(_Float16, *reinterpret_cast<const uint16_t *>(x));
}

// Running sums of one lane.
struct StatAcc {
    double s1 = 0, s2 = 0, s3 = 0, s4 = 0, w2 = 0, d2 = 0, rsum = 0, nblk = 0;
    float amax = 0.0f;
};

// Elements 2j, 2j + 1 of a unit.
template <int SRC>
__device__ __forceinline__ f32x2 unit_pair(const Unit<SRC> &d, int j) {
    if constexpr (SRC == NVFP4_F32) {
        return f32x2{u2f(d.x[2 * j]), u2f(d.x[2 * j + 1])};
    } else if constexpr (SRC == NVFP4_BF16) {
        return f32x2{u2f(d.x[j] << 16), u2f(d.x[j] & 0xFFFF0000u)};
    } else {
        return f32x2{(float)__builtin_bit_cast(_Float16, (uint16_t)(d.x[j] & 0xFFFFu)),
                     (float)__builtin_bit_cast(_Float16, (uint16_t)(d.x[j] >> 16))};
    }
}

// Power sums of one unit about its own first value u0 (t = w - u0), and its squared error.
struct UnitSums {
    double t1 = 0.0, t2 = 0.0, t3 = 0.0, t4 = 0.0, d2 = 0.0;
    float bmax = 0.0f;
};

// Elements 4G .. 4G + 3 of a unit, with their two code bytes (E2M1 pairs) decoded in place.
template <int SRC, bool HAS_Q, int G>
__device__ __forceinline__ void add_group(UnitSums &us, const Unit<SRC> &d, double u0, double sg) {
    f32x2 e01 = {0.0f, 0.0f}, e23 = {0.0f, 0.0f};
    if constexpr (HAS_Q) {
        e01 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(d.codes[G >> 1], 1.0f, (G & 1) * 2);
        e23 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(d.codes[G >> 1], 1.0f, (G & 1) * 2 + 1);
    }
    const f32x2 p0 = unit_pair<SRC>(d, 2 * G), p1 = unit_pair<SRC>(d, 2 * G + 1);
    const float v[4] = {p0[0], p0[1], p1[0], p1[1]};
    const float e[4] = {e01[0], e01[1], e23[0], e23[1]};
#pragma unroll
    for (int i = 0; i < 4; i++) {
        const double w = (double)v[i];
        const double t = w - u0;
        const double tt = t * t;
        us.t1 += t;
        us.t2 += tt;
        us.t3 = fma(tt, t, us.t3);
        us.t4 = fma(tt, tt, us.t4);
        if constexpr (HAS_Q) {
            const double r = fma(-(double)e[i], sg, w);  // w - w_hat, one rounding
            us.d2 = fma(r, r, us.d2);
        }
        us.bmax = fmaxf(us.bmax, fabsf(v[i]));
    }
    // Pin the sums here: without it the compiler sinks the products towards their later uses and
    // keeps all sixteen values of the unit live (register pressure, spills).
    asm volatile("" : "+v"(us.t1), "+v"(us.t2), "+v"(us.t3), "+v"(us.t4), "+v"(us.d2));
}

// Adds unit u (words in d; lanes with u >= units hold zeros and take part in the shuffles only) to
// the sums, in one pass over its 16 values.
//
// Each unit's power sums are taken about its own first value u0, so the per-element work is four
// sums; they are moved to the common shift c per unit with the binomial expansion
// sum (t + delta)^k, delta = u0 - c, and sum w^2 = T2 + 2 u0 T1 + 16 u0^2.  As every value of a set
// lies within sqrt(count - 1) standard deviations of its mean, the shift by u0 costs at most a
// small multiple of the rounding unit in each sum.
//
// The spread of each block of 64 is combined from its four units: a unit's mean is u0 + T1/16 and
// its M2 is T2 - T1^2/16; the block's M2 is the sum of the units' M2 plus 16 (mean_unit -
// mean_block)^2 per unit.  A constant block gets exactly 0.
template <int SRC, bool HAS_Q>
__device__ __forceinline__ void add_unit(StatAcc &a, const Unit<SRC> &d, int64_t u, int64_t units, int lane,
                                         double shift, double gd) {
    const int64_t n = units * 16;
    const bool valid = u < units;
    const double u0 = (double)unit_pair<SRC>(d, 0)[0];
    // w_hat = e2m1 x (s x g): s x g and its products with e2m1 values are exact in double
    const double sg = HAS_Q ? (double)e4m3_to_f32((uint8_t)d.scale) * gd : 0.0;
    UnitSums us;
    add_group<SRC, HAS_Q, 0>(us, d, u0, sg);
    add_group<SRC, HAS_Q, 1>(us, d, u0, sg);
    add_group<SRC, HAS_Q, 2>(us, d, u0, sg);
    add_group<SRC, HAS_Q, 3>(us, d, u0, sg);
    const double t1 = us.t1, t2 = us.t2, t3 = us.t3, t4 = us.t4;
    // to the common shift (lanes past the end hold zeros and shift by 0: they add nothing)
    const double dl = u0 - (valid ? shift : 0.0), dl2 = dl * dl;
    a.s1 += t1 + 16.0 * dl;
    a.s2 += t2 + dl * (2.0 * t1 + 16.0 * dl);
    a.s3 += t3 + 3.0 * dl * t2 + dl2 * (3.0 * t1 + 16.0 * dl);
    a.s4 += t4 + 4.0 * dl * t3 + dl2 * (6.0 * t2 + 4.0 * dl * t1 + 16.0 * dl2);
    a.w2 += t2 + u0 * (2.0 * t1 + 16.0 * u0);
    if constexpr (HAS_Q) a.d2 += us.d2;
    a.amax = fmaxf(a.amax, us.bmax);
    // block of 64: lanes 4k .. 4k + 3 (lanes past the end count 0 elements)
    double bs = 16.0 * u0 + t1;
    bs += quad_xor_f64<kQuadXor1>(bs);
    bs += quad_xor_f64<kQuadXor2>(bs);
    float bm = fmaxf(us.bmax, quad_xor_f32<kQuadXor1>(us.bmax));
    bm = fmaxf(bm, quad_xor_f32<kQuadXor2>(bm));
    const int64_t left = n - (u & ~(int64_t)3) * 16;
    double mb = bs * 0.015625;
    if (__builtin_expect(left < 64, 0)) mb = left > 0 ? bs / (double)left : 0.0;
    const double dev = (u0 + t1 * 0.0625) - mb;
    double m2 = valid ? (t2 - t1 * (t1 * 0.0625)) + 16.0 * dev * dev : 0.0;
    m2 += quad_xor_f64<kQuadXor1>(m2);
    m2 += quad_xor_f64<kQuadXor2>(m2);
    double var = m2 * 0.015625;
    if (__builtin_expect(left < 64, 0)) var = left > 0 ? m2 / (double)left : 0.0;
    if ((lane & 3) == 0 && left > 0 && var > 0.0) {
        a.rsum += (double)bm / sqrt(var);
        a.nblk += 1.0;
    }
}

// One workgroup of 4 waves; wave-iteration k of wave w covers units (w + k * waves) * 64 + lane.
template <int SRC, bool HAS_Q, bool DENSE>
__global__ __launch_bounds__(256, 4) void k_stats(const uint8_t *__restrict__ x, int64_t cols, int64_t ld_bytes,
                                                  int64_t units, const uint8_t *__restrict__ codes,
                                                  const uint8_t *__restrict__ scales, const float *__restrict__ g,
                                                  double *__restrict__ partials) {
    __shared__ double red[4][kStatFields];
    const int lane = threadIdx.x & 63, wid = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const double gd = HAS_Q ? (double)*g : 0.0;
    const double shift = first_value<SRC>(x);
    const int64_t step_units = (int64_t)gridDim.x * 4 * 64;
    const int64_t step_e = step_units * 16;
    const int64_t step_r = step_e / cols, step_c = step_e - step_r * cols;
    WavePos p;
    p.u = ((int64_t)blockIdx.x * 4 + wid) * 64;
    p.r = (p.u * 16) / cols;
    p.c = p.u * 16 - p.r * cols;
    StatAcc a;
    // K wave-iterations per trip, their loads all issued before any is reduced
    constexpr int K = kStatsItersInFlight<SRC>;
    while (p.u < units) {
        Unit<SRC> d[K];
        int64_t uk[K];
#pragma unroll
        for (int k = 0; k < K; k++) {
            uk[k] = p.u + lane;
            load_unit<SRC, HAS_Q, DENSE>(d[k], p, lane, units, x, (uint32_t)cols, ld_bytes, codes, scales);
            p.advance(step_units, step_r, step_c, cols);
        }
#pragma unroll
        for (int k = 0; k < K; k++) add_unit<SRC, HAS_Q>(a, d[k], uk[k], units, lane, shift, gd);
    }
    // wave sums, then the workgroup's
    double acc[kStatFields] = {a.s1, a.s2, a.s3, a.s4, a.w2, a.d2, a.rsum, a.nblk, (double)a.amax};
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
        double r2 = red[0][f];
        for (int w = 1; w < 4; w++) r2 = f == kStatFields - 1 ? fmax(r2, red[w][f]) : r2 + red[w][f];
        partials[(int64_t)f * gridDim.x + blockIdx.x] = r2;  // field-major: the final pass reads rows
    }
}

// One workgroup: the partial sums in a fixed order, then the statistics.
__global__ __launch_bounds__(kFinalThreads) void k_stats_final(const double *__restrict__ partials, int nparts,
                                                               int64_t n, const uint8_t *__restrict__ x, int src,
                                                               int has_q, double *__restrict__ out) {
    __shared__ double red[kFinalThreads / 64][kStatFields];
    const int t = threadIdx.x, lane = t & 63, wid = t >> 6;
    // all loads first (at most kStatsMaxGroups / kFinalThreads per field), then the sums in order
    constexpr int kPer = kStatsMaxGroups / kFinalThreads;
    static_assert(kPer * kFinalThreads == kStatsMaxGroups, "partials per final thread");
    double v[kStatFields][kPer];
#pragma unroll
    for (int f = 0; f < kStatFields; f++)
#pragma unroll
        for (int k = 0; k < kPer; k++) {
            const int i = t + k * kFinalThreads;
            v[f][k] = i < nparts ? partials[(int64_t)f * nparts + i] : 0.0;  // 0 is neutral for max |w| too
        }
    double acc[kStatFields];
#pragma unroll
    for (int f = 0; f < kStatFields; f++) {
        double r = v[f][0];
#pragma unroll
        for (int k = 1; k < kPer; k++) r = f == kStatFields - 1 ? fmax(r, v[f][k]) : r + v[f][k];
        acc[f] = r;
    }
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
    if (t == 0) {
        double tot[kStatFields];
#pragma unroll
        for (int f = 0; f < kStatFields; f++) {
            double r = red[0][f];
            for (int w = 1; w < kFinalThreads / 64; w++) r = f == kStatFields - 1 ? fmax(r, red[w][f]) : r + red[w][f];
            tot[f] = r;
        }
        const double shift = src == NVFP4_F32 ? first_value<NVFP4_F32>(x)
                             : src == NVFP4_BF16 ? first_value<NVFP4_BF16>(x) : first_value<NVFP4_F16>(x);
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
    // wave-iterations of 64 units, spread evenly over at most 4 workgroups (16 waves, the
    // residency the kernel's registers allow) per CU
    const int64_t iters = (units + 63) / 64;
    const int64_t max_waves = 4 * (int64_t)(num_cus * 4 < kStatsMaxGroups ? num_cus * 4 : kStatsMaxGroups);
    const int64_t per_wave = (iters + max_waves - 1) / max_waves;
    const int64_t waves = (iters + per_wave - 1) / per_wave;
    const int64_t grid = (waves + 3) / 4;
    const uint8_t *xb = (const uint8_t *)x;
    const bool dense = ld_x == cols || rows == 1;
#define NVFP4_STATS_LAUNCH(HQ, DN)                                                                               \
    hipLaunchKernelGGL((k_stats<SRC, HQ, DN>), dim3((unsigned)grid), dim3(256), 0, stream, xb, cols, ld_x * EB, \
                       units, HQ ? q->codes : nullptr, HQ ? q->scales : nullptr, HQ ? q->global_scale : nullptr,   \
                       partials)
    if (q) {
        if (dense) NVFP4_STATS_LAUNCH(true, true);
        else NVFP4_STATS_LAUNCH(true, false);
    } else {
        if (dense) NVFP4_STATS_LAUNCH(false, true);
        else NVFP4_STATS_LAUNCH(false, false);
    }
#undef NVFP4_STATS_LAUNCH
    hipLaunchKernelGGL(k_stats_final, dim3(1), dim3(kFinalThreads), 0, stream, partials, (int)grid, rows * cols,
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
