// NVFP4 quantization / requantization kernels for gfx950.
//
// What is computed ("Qwen-Image NVFP4 on a 16 GB Ada GPU", section "What NVFP4 is and how it differs
// from NF4"; "Qwen-Rapid-AIO-NVFP4", section "Why This Exists" for the FP8 source):
//   v      = source value widened to fp32 (E4M3 source: fl(e4m3(b) * src_scale))
//   g      = fl(amax / 2688)                        per tensor (amax run-time or static)
//   s_byte = E4M3_RNE_SAT(fl(bamax / fl(6 g)))      per 16 consecutive elements of a row
//   code   = sign(v) | E2M1_RNE_SAT(fl(|v| * fl(1 / fl(s g))))   per element, packed low nibble first
//
// Launch structure (all on the caller's stream):
//   k_ws_clear          zero the amax word of the workspace (a kernel, not a memset, so that the
//                       sequence can be captured into a graph)
//   k_amax<SRC>         max |v| over the tensor as an integer max of the magnitude bit patterns
//                       (non-negative floats order like their bit patterns; NaN patterns sort
//                       above infinity, so a non-finite input shows up in the result)
//   k_encode<SRC>       one wave encodes 64 blocks (1024 elements) per tile:
//                         - every lane loads 16 bytes per 16-byte vector, so each load instruction
//                           covers 1 KiB of contiguous input;
//                         - block maxima are reduced over the lanes that share a block, then
//                           re-distributed so that lane L owns block L of the tile and does the
//                           per-block divisions once;
//                         - the per-block reciprocal goes back to the lanes holding the elements,
//                           which convert two values per instruction to E2M1.
#include <hip/hip_runtime.h>

#include "common.h"
#include "internal.h"

namespace nvfp4 {

template <int SRC>
struct SrcTraits;
template <>
struct SrcTraits<NVFP4_F32> {
    static constexpr int kElemBytes = 4;
};
template <>
struct SrcTraits<NVFP4_BF16> {
    static constexpr int kElemBytes = 2;
};
template <>
struct SrcTraits<NVFP4_F16> {
    static constexpr int kElemBytes = 2;
};
template <>
struct SrcTraits<NVFP4_E4M3> {
    static constexpr int kElemBytes = 1;
};

// Elements per 16-byte vector and vectors per 16-element block.
template <int SRC>
constexpr int kEpv = 16 / SrcTraits<SRC>::kElemBytes;
template <int SRC>
constexpr int kVpb = 16 / kEpv<SRC>;

// Widen one 16-byte vector to fp32 values.
template <int SRC>
__device__ __forceinline__ void widen(const u32x4 &raw, float sc, float (&v)[kEpv<SRC>]) {
    if constexpr (SRC == NVFP4_F32) {
#pragma unroll
        for (int i = 0; i < 4; i++) v[i] = u2f(raw[i]);
    } else if constexpr (SRC == NVFP4_BF16) {
#pragma unroll
        for (int i = 0; i < 4; i++) {
            v[2 * i] = u2f(raw[i] << 16);
            v[2 * i + 1] = u2f(raw[i] & 0xFFFF0000u);
        }
    } else if constexpr (SRC == NVFP4_F16) {
#pragma unroll
        for (int i = 0; i < 4; i++) {
            v[2 * i] = (float)__builtin_bit_cast(_Float16, (uint16_t)(raw[i] & 0xFFFFu));
            v[2 * i + 1] = (float)__builtin_bit_cast(_Float16, (uint16_t)(raw[i] >> 16));
        }
    } else {
#pragma unroll
        for (int i = 0; i < 4; i++) {
            f32x2 lo = __builtin_amdgcn_cvt_pk_f32_fp8(raw[i], false);
            f32x2 hi = __builtin_amdgcn_cvt_pk_f32_fp8(raw[i], true);
            v[4 * i + 0] = lo[0] * sc;
            v[4 * i + 1] = lo[1] * sc;
            v[4 * i + 2] = hi[0] * sc;
            v[4 * i + 3] = hi[1] * sc;
        }
    }
}

// Largest magnitude bit pattern of one vector.  For an E4M3 source the magnitude byte (sign
// cleared) is used: the E4M3 grid is monotone in its bit pattern and multiplying by a positive
// scale keeps the order, so max |v| = fl(e4m3(max byte) * scale).
template <int SRC>
__device__ __forceinline__ uint32_t vec_absmax_bits(const u32x4 &raw) {
    uint32_t m = 0;
    if constexpr (SRC == NVFP4_F32) {
#pragma unroll
        for (int i = 0; i < 4; i++) m = max(m, raw[i] & 0x7FFFFFFFu);
    } else if constexpr (SRC == NVFP4_BF16) {
#pragma unroll
        for (int i = 0; i < 4; i++) {
            m = max(m, (raw[i] << 16) & 0x7FFF0000u);
            m = max(m, raw[i] & 0x7FFF0000u);
        }
    } else if constexpr (SRC == NVFP4_F16) {
        // fp16 magnitudes also order like their bit patterns; widen the maximum once.
        uint32_t h = 0;
#pragma unroll
        for (int i = 0; i < 4; i++) {
            h = max(h, raw[i] & 0x7FFFu);
            h = max(h, (raw[i] >> 16) & 0x7FFFu);
        }
        float f = (float)__builtin_bit_cast(_Float16, (uint16_t)h);
        m = f2u(f);
        if (h > 0x7C00u) m = 0x7FC00000u;  // NaN stays above infinity
    } else {
#pragma unroll
        for (int i = 0; i < 4; i++) {
            uint32_t w = raw[i] & 0x7F7F7F7Fu;
            m = max(m, max(max(w & 0xFFu, (w >> 8) & 0xFFu), max((w >> 16) & 0xFFu, w >> 24)));
        }
    }
    return m;
}

__global__ void k_ws_clear(uint32_t *ws) { ws[threadIdx.x] = 0u; }

// Address of 16-byte vector `vi` of the tensor (vectors numbered row-major over the logical
// [rows x cols] shape).  Contiguous tensors are linear; otherwise split into row and column.
__device__ __forceinline__ const u32x4 *vec_addr(const uint8_t *x, uint64_t vi, uint32_t vpr, int64_t ld_bytes,
                                                 bool contiguous) {
    if (contiguous) return reinterpret_cast<const u32x4 *>(x) + vi;
    uint64_t r = vi / vpr;
    uint64_t c = vi - r * vpr;
    return reinterpret_cast<const u32x4 *>(x + r * (uint64_t)ld_bytes) + c;
}

template <int SRC>
__global__ __launch_bounds__(256) void k_amax(const uint8_t *__restrict__ x, uint64_t nvec, uint32_t vpr,
                                              int64_t ld_bytes, int contiguous, uint32_t *__restrict__ ws) {
    __shared__ uint32_t red[4];
    uint32_t m = 0;
    const uint64_t stride = (uint64_t)gridDim.x * blockDim.x;
    uint64_t i = (uint64_t)blockIdx.x * blockDim.x + threadIdx.x;
    // four independent loads in flight per lane
    for (; i + 3 * stride < nvec; i += 4 * stride) {
        u32x4 a = *vec_addr(x, i, vpr, ld_bytes, contiguous);
        u32x4 b = *vec_addr(x, i + stride, vpr, ld_bytes, contiguous);
        u32x4 c = *vec_addr(x, i + 2 * stride, vpr, ld_bytes, contiguous);
        u32x4 d = *vec_addr(x, i + 3 * stride, vpr, ld_bytes, contiguous);
        m = max(m, max(max(vec_absmax_bits<SRC>(a), vec_absmax_bits<SRC>(b)),
                       max(vec_absmax_bits<SRC>(c), vec_absmax_bits<SRC>(d))));
    }
    for (; i < nvec; i += stride) m = max(m, vec_absmax_bits<SRC>(*vec_addr(x, i, vpr, ld_bytes, contiguous)));
    m = wave_max_u32(m);
    const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
    if (lane == 0) red[wid] = m;
    __syncthreads();
    if (threadIdx.x == 0) {
        uint32_t t = max(max(red[0], red[1]), max(red[2], red[3]));
        atomicMax(ws, t);
    }
}

// Global scale from the amax word (or the static amax) -- every thread computes the same value.
template <int SRC>
__device__ __forceinline__ float global_scale(const uint32_t *ws, const float *amax_in, float sc, bool *nonfinite) {
    float amax;
    if (amax_in) {
        amax = *amax_in;
    } else if constexpr (SRC == NVFP4_E4M3) {
        uint32_t b = *ws;
        *nonfinite = (b == 0x7Fu);
        amax = e4m3_to_f32(b) * sc;
        if (!(amax <= 3.402823466e38f)) *nonfinite = true;
    } else {
        uint32_t bits = *ws;
        *nonfinite = bits >= 0x7F800000u;
        amax = u2f(bits);
    }
    return amax / 2688.0f;
}

template <int SRC>
__global__ __launch_bounds__(256) void k_encode(const uint8_t *__restrict__ x, uint64_t nblocks, uint32_t bpr,
                                                int64_t ld_bytes, int contiguous, const float *__restrict__ src_scale,
                                                const float *__restrict__ amax_in, const uint32_t *__restrict__ ws,
                                                uint8_t *__restrict__ codes, uint8_t *__restrict__ scales,
                                                float *__restrict__ g_out, int32_t *__restrict__ flags) {
    constexpr int EPV = kEpv<SRC>;
    constexpr int VPB = kVpb<SRC>;
    constexpr int BPL = 64 / VPB;  // blocks covered by one 64-lane load
    const int lane = threadIdx.x & 63;
    const float sc = (SRC == NVFP4_E4M3 && src_scale) ? *src_scale : 1.0f;
    bool nonfinite = false;
    const float g = global_scale<SRC>(ws, amax_in, sc, &nonfinite);
    if (blockIdx.x == 0 && threadIdx.x == 0) {
        *g_out = g;
        if (nonfinite && flags) atomicOr(flags, 1);
    }
    const float six_g = 6.0f * g;
    const uint32_t vpr = bpr * VPB;  // vectors per row
    const uint64_t ntiles = (nblocks + 63) / 64;
    const uint64_t wave0 = ((uint64_t)blockIdx.x * blockDim.x + threadIdx.x) >> 6;
    const uint64_t nwaves = ((uint64_t)gridDim.x * blockDim.x) >> 6;

    for (uint64_t tile = wave0; tile < ntiles; tile += nwaves) {
        const uint64_t blk0 = tile * 64;
        // ---- load VPB vectors per lane: vector j*64+lane of the tile ----
        u32x4 raw[VPB];
#pragma unroll
        for (int j = 0; j < VPB; j++) {
            const uint32_t vt = j * 64 + lane;
            const uint64_t blk = blk0 + vt / VPB;
            if (blk < nblocks) {
                raw[j] = *vec_addr(x, blk * VPB + vt % VPB, vpr, ld_bytes, contiguous);
            } else {
                raw[j] = u32x4{0u, 0u, 0u, 0u};
            }
        }
        // ---- block maxima: reduce over the VPB lanes holding one block ----
        uint32_t pm[VPB];
#pragma unroll
        for (int j = 0; j < VPB; j++) {
            pm[j] = vec_absmax_bits<SRC>(raw[j]);
#pragma unroll
            for (int o = 1; o < VPB; o <<= 1) pm[j] = max(pm[j], (uint32_t)__shfl_xor((int)pm[j], o, 64));
        }
        // ---- lane L takes block L of the tile ----
        uint32_t bm;
        if constexpr (VPB == 1) {
            bm = pm[0];
        } else {
            const int src = (lane % BPL) * VPB;
            const int jj = lane / BPL;
            bm = 0;
#pragma unroll
            for (int j = 0; j < VPB; j++) {
                uint32_t t = (uint32_t)__shfl((int)pm[j], src, 64);
                if (j == jj) bm = t;
            }
        }
        float bamax;
        bool bad;
        if constexpr (SRC == NVFP4_E4M3) {
            bad = (bm == 0x7Fu);
            bamax = e4m3_to_f32(bm) * sc;
            bad = bad || !(bamax <= 3.402823466e38f);
        } else {
            bad = bm >= 0x7F800000u;
            bamax = u2f(bm);
        }
        const uint64_t myblk = blk0 + lane;
        bad = bad && (myblk < nblocks);
        if (__any(bad) && lane == 0 && flags) atomicOr(flags, 1);
        // ---- per-block scale byte and reciprocal ----
        uint32_t sbyte = 0;
        if (g != 0.0f) sbyte = e4m3_from_f32(bamax / six_g);
        const float s = e4m3_to_f32(sbyte);
        const float r = (s == 0.0f) ? 0.0f : 1.0f / (s * g);
        if (myblk < nblocks) scales[myblk] = (uint8_t)sbyte;
        // ---- encode: each lane converts its own vectors with its block's reciprocal ----
#pragma unroll
        for (int j = 0; j < VPB; j++) {
            const uint32_t vt = j * 64 + lane;
            const uint64_t blk = blk0 + vt / VPB;
            float rj;
            if constexpr (VPB == 1) {
                rj = r;
            } else {
                rj = __shfl(r, j * BPL + lane / VPB, 64);
            }
            float v[EPV];
            widen<SRC>(raw[j], sc, v);
            float y[EPV];
            if (__builtin_expect(__builtin_isinf(rj), 0)) {
                // tiny s * g: fl(1 / d) overflowed; |v| * inf saturates, 0 stays 0 (no 0 * inf)
#pragma unroll
                for (int e = 0; e < EPV; e++) y[e] = (v[e] == 0.0f) ? v[e] : v[e] * rj;
            } else {
#pragma unroll
                for (int e = 0; e < EPV; e++) y[e] = v[e] * rj;
            }
            if (blk < nblocks) {
                uint8_t *dst = codes + (blk * VPB + vt % VPB) * (EPV / 2);
                if constexpr (EPV == 4) {
                    *reinterpret_cast<uint16_t *>(dst) = (uint16_t)fp4_pack4(y);
                } else if constexpr (EPV == 8) {
                    *reinterpret_cast<uint32_t *>(dst) = fp4_pack8(y);
                } else {
                    *reinterpret_cast<u32x2 *>(dst) = u32x2{fp4_pack8(y), fp4_pack8(y + 8)};
                }
            }
        }
    }
}

static int grid_for(uint64_t work_items, int per_block, int max_blocks) {
    uint64_t b = (work_items + per_block - 1) / per_block;
    if (b < 1) b = 1;
    if (b > (uint64_t)max_blocks) b = max_blocks;
    return (int)b;
}

template <int SRC>
static hipError_t launch_quantize_t(const void *x, int64_t ld_x, int64_t rows, int64_t cols, const float *src_scale,
                                    const float *amax_in, const nvfp4_tensor *out, int32_t *flags, uint32_t *ws,
                                    int num_cus, hipStream_t stream) {
    constexpr int EB = SrcTraits<SRC>::kElemBytes;
    const int64_t ld_bytes = ld_x * EB;
    const int contiguous = (ld_x == cols) ? 1 : 0;
    const uint64_t nblocks = (uint64_t)rows * (uint64_t)(cols / 16);
    const uint32_t bpr = (uint32_t)(cols / 16);
    if (!amax_in) {
        hipLaunchKernelGGL(k_ws_clear, dim3(1), dim3(1), 0, stream, ws);
        const uint64_t nvec = nblocks * kVpb<SRC>;
        const int grid = grid_for(nvec, 256 * 4, num_cus * 8);
        hipLaunchKernelGGL(k_amax<SRC>, dim3(grid), dim3(256), 0, stream, (const uint8_t *)x, nvec,
                           bpr * (uint32_t)kVpb<SRC>, ld_bytes, contiguous, ws);
    }
    // one wave per 64-block tile, 4 waves per workgroup; cap at 16 workgroups per CU
    const uint64_t ntiles = (nblocks + 63) / 64;
    const int grid = grid_for(ntiles, 4, num_cus * 16);
    hipLaunchKernelGGL(k_encode<SRC>, dim3(grid), dim3(256), 0, stream, (const uint8_t *)x, nblocks, bpr, ld_bytes,
                       contiguous, src_scale, amax_in, ws, out->codes, out->scales, out->global_scale, flags);
    return hipGetLastError();
}

hipError_t launch_quantize(const void *x, nvfp4_dtype dt, int64_t ld_x, const float *src_scale, const float *amax_in,
                           const nvfp4_tensor *out, int32_t *flags, void *workspace, int num_cus,
                           hipStream_t stream) {
    uint32_t *ws = reinterpret_cast<uint32_t *>(workspace);
    const int64_t rows = out->rows, cols = out->cols;
    switch (dt) {
    case NVFP4_F32:
        return launch_quantize_t<NVFP4_F32>(x, ld_x, rows, cols, src_scale, amax_in, out, flags, ws, num_cus, stream);
    case NVFP4_BF16:
        return launch_quantize_t<NVFP4_BF16>(x, ld_x, rows, cols, src_scale, amax_in, out, flags, ws, num_cus, stream);
    case NVFP4_F16:
        return launch_quantize_t<NVFP4_F16>(x, ld_x, rows, cols, src_scale, amax_in, out, flags, ws, num_cus, stream);
    default:
        return launch_quantize_t<NVFP4_E4M3>(x, ld_x, rows, cols, src_scale, amax_in, out, flags, ws, num_cus, stream);
    }
}

}  // namespace nvfp4
