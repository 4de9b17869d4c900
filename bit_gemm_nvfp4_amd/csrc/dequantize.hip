// NVFP4 expansion ("expander") for gfx950.
//
// "Qwen-Image NVFP4 on a 16 GB Ada GPU", section "Running the NVFP4 weights on Ada", describes the
// expander as a byte table giving each byte's two E2M1 values, with each block's scale applied to its
// 16 values; section "What NVFP4 is and how it differs from NF4" gives the value as
// E2M1 x block scale x global scale.  Here the byte -> two values step is the hardware FP4 -> fp32
// conversion (two codes per instruction), then w = fl(fl(e2m1 * s) * g); e2m1 * s is exact, so this
// is one rounding of the exact product.  bf16 output is the round-to-nearest-even of that fp32.
//
// Each lane expands 8 elements per chunk (one dword of codes, one scale byte shared by 2 lanes) and
// writes 16 bytes (bf16) or 32 bytes (fp32); consecutive lanes touch consecutive addresses.  A lane
// takes 4 chunks a grid apart with all their loads issued first (8 % faster than one chunk per
// lane at a grid stride on a 3072 x 3072 matrix, the same at 12288 x 3072).
#include <hip/hip_runtime.h>

#include "common.h"
#include "internal.h"

namespace nvfp4 {

constexpr int kDeqPerLane = 4;  // chunks of 8 elements per lane per pass, all loaded first

template <bool BF16_OUT>
__global__ __launch_bounds__(256) void k_dequant(const uint32_t *__restrict__ codes, const uint8_t *__restrict__ scales,
                                                 const float *__restrict__ gptr, uint64_t nchunks, uint32_t cpr,
                                                 int64_t ld_out, int contiguous, void *__restrict__ out) {
    const float g = *gptr;
    const uint64_t stride = (uint64_t)gridDim.x * blockDim.x;
    for (uint64_t i0 = (uint64_t)blockIdx.x * blockDim.x + threadIdx.x; i0 < nchunks; i0 += kDeqPerLane * stride) {
        // chunk i0 + j * stride for j < kDeqPerLane: consecutive lanes take consecutive chunks
        uint32_t w[kDeqPerLane], sb[kDeqPerLane];
#pragma unroll
        for (int j = 0; j < kDeqPerLane; j++) {
            const uint64_t i = i0 + j * stride;
            w[j] = i < nchunks ? codes[i] : 0u;
            sb[j] = i < nchunks ? scales[i >> 1] : 0u;
        }
#pragma unroll
        for (int j = 0; j < kDeqPerLane; j++) {
            const uint64_t i = i0 + j * stride;
            if (i >= nchunks) break;
            const float s = e4m3_to_f32(sb[j]);
            float v[8];
            fp4_unpack8_f32(w[j], v);
#pragma unroll
            for (int q = 0; q < 8; q++) v[q] = (v[q] * s) * g;
            uint64_t e;  // element offset of the first of the 8 values in the output
            if (contiguous) {
                e = i * 8;
            } else {
                const uint64_t r = i / cpr;
                e = r * (uint64_t)ld_out + (i - r * cpr) * 8;
            }
            if constexpr (BF16_OUT) {
                bf16x8 o;
#pragma unroll
                for (int k = 0; k < 8; k++) o[k] = (__bf16)v[k];
                *reinterpret_cast<bf16x8 *>(reinterpret_cast<__bf16 *>(out) + e) = o;
            } else {
                f32x4 *dst = reinterpret_cast<f32x4 *>(reinterpret_cast<float *>(out) + e);
                dst[0] = f32x4{v[0], v[1], v[2], v[3]};
                dst[1] = f32x4{v[4], v[5], v[6], v[7]};
            }
        }
    }
}

hipError_t launch_dequantize(const nvfp4_tensor *in, void *out, nvfp4_dtype out_dtype, int64_t ld_out, int num_cus,
                             hipStream_t stream) {
    const uint64_t nchunks = (uint64_t)in->rows * (uint64_t)(in->cols / 8);
    const uint32_t cpr = (uint32_t)(in->cols / 8);
    const int contiguous = (ld_out == in->cols) ? 1 : 0;
    // one pass of kDeqPerLane chunks per lane where the grid allows (passes repeat beyond 2^20
    // workgroups)
    uint64_t grid = (nchunks + 256 * kDeqPerLane - 1) / (256 * kDeqPerLane);
    if (grid > ((uint64_t)1 << 20)) grid = (uint64_t)1 << 20;
    if (grid < 1) grid = 1;
    if (out_dtype == NVFP4_BF16) {
        hipLaunchKernelGGL(k_dequant<true>, dim3((unsigned)grid), dim3(256), 0, stream,
                           reinterpret_cast<const uint32_t *>(in->codes), in->scales, in->global_scale, nchunks, cpr,
                           ld_out, contiguous, out);
    } else {
        hipLaunchKernelGGL(k_dequant<false>, dim3((unsigned)grid), dim3(256), 0, stream,
                           reinterpret_cast<const uint32_t *>(in->codes), in->scales, in->global_scale, nchunks, cpr,
                           ld_out, contiguous, out);
    }
    return hipGetLastError();
}

}  // namespace nvfp4
