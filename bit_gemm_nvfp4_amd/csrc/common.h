// Device-side building blocks shared by the NVFP4 kernels (gfx950 / CDNA4, wave64).
//
// Format facts used here ("Qwen-Image NVFP4 on a 16 GB Ada GPU", section "What NVFP4 is and how it
// differs from NF4"): E2M1 codes with magnitudes {0, .5, 1, 1.5, 2, 3, 4, 6} and a sign bit, one FP8
// E4M3 scale per 16 elements of a row, one fp32 global scale, two codes per byte (low nibble first).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "nvfp4.h"

namespace nvfp4 {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int kWave = 64;

// Bit casts take their operand by value: applying __builtin_bit_cast directly to an element of an
// ext_vector_type reads the vector's first element with this compiler, so elements are copied first.
__device__ __forceinline__ uint32_t f2u(float f) { return __builtin_bit_cast(uint32_t, f); }
__device__ __forceinline__ float u2f(uint32_t u) { return __builtin_bit_cast(float, u); }
__device__ __forceinline__ bf16x2 as_bf16x2(uint32_t u) { return __builtin_bit_cast(bf16x2, u); }

// ---------------------------------------------------------------------------------------------
// E4M3 (OCP e4m3fn) block-scale bytes.
// ---------------------------------------------------------------------------------------------
// Round-to-nearest-even of a non-negative fp32 value onto the E4M3 grid, saturating at 448 (0x7E;
// NaN also gives 0x7E).  Normal range: round the fp32 mantissa at bit 20 (3 kept bits) by integer
// add and rebias the exponent; subnormal range (t < 2^-6, step 2^-9): rint(t * 2^9), where the
// scaling by a power of two is exact and rint rounds half to even.  Both are computed and the
// right one selected, so the conversion has no branches.
__device__ __forceinline__ uint32_t e4m3_from_f32(float t) {
    const uint32_t sub = (uint32_t)__builtin_rintf(__builtin_fminf(t, 0.015625f) * 512.0f);
    const uint32_t u = f2u(t);
    const uint32_t r = u + 0x7FFFFu + ((u >> 20) & 1u);
    uint32_t code = (((r >> 23) - 120u) << 3) | ((r >> 20) & 7u);
    code = code < 0x7Eu ? code : 0x7Eu;
    const uint32_t v = t < 0.015625f ? sub : code;
    return t < 448.0f ? v : 0x7Eu;
}

// Value of a non-negative E4M3 byte (0x00..0x7E) as fp32 (exact): the hardware OCP e4m3
// conversion.
__device__ __forceinline__ float e4m3_to_f32(uint32_t b) { return __builtin_amdgcn_cvt_f32_fp8((int)b, 0); }

// ---------------------------------------------------------------------------------------------
// E2M1 codes: hardware conversions with a unit scale.
// ---------------------------------------------------------------------------------------------
// Two fp32 -> two E2M1 codes written into byte SEL of `word` (first value in the low nibble).
// With scale 1.0 the instruction is a plain round-to-nearest-even conversion that saturates at
// +-6 and keeps the sign of zero.  The GPU tests pin this against the oracle on every fp32 value in
// [0, 6], every E2M1 midpoint and its neighbours, and values above 6.
template <int SEL>
__device__ __forceinline__ uint32_t fp4_pk(uint32_t word, float a, float b) {
    return __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(word, a, b, 1.0f, SEL);
}

// Eight fp32 -> one dword of eight E2M1 codes (element i in nibble i).  Every byte of the result is
// written, so the starting value of the dword does not matter (an input register avoids a move).
__device__ __forceinline__ uint32_t fp4_pack8(const float *y) {
    uint32_t w = f2u(y[0]);
    w = fp4_pk<0>(w, y[0], y[1]);
    w = fp4_pk<1>(w, y[2], y[3]);
    w = fp4_pk<2>(w, y[4], y[5]);
    w = fp4_pk<3>(w, y[6], y[7]);
    return w;
}

// Four fp32 -> the low 16 bits of a dword (element i in nibble i); the high 16 bits are unspecified.
__device__ __forceinline__ uint32_t fp4_pack4(const float *y) {
    uint32_t w = f2u(y[0]);
    w = fp4_pk<0>(w, y[0], y[1]);
    w = fp4_pk<1>(w, y[2], y[3]);
    return w;
}

// One dword of eight E2M1 codes -> eight fp32 values (exact).
__device__ __forceinline__ void fp4_unpack8_f32(uint32_t w, float *v) {
    f32x2 p0 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 0);
    f32x2 p1 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 1);
    f32x2 p2 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 2);
    f32x2 p3 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 3);
    v[0] = p0[0]; v[1] = p0[1]; v[2] = p1[0]; v[3] = p1[1];
    v[4] = p2[0]; v[5] = p2[1]; v[6] = p3[0]; v[7] = p3[1];
}

// One dword of eight E2M1 codes -> four pairs of bf16 values (exact).
__device__ __forceinline__ void fp4_unpack8_bf16x2(uint32_t w, bf16x2 *v) {
    v[0] = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, 1.0f, 0);
    v[1] = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, 1.0f, 1);
    v[2] = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, 1.0f, 2);
    v[3] = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, 1.0f, 3);
}

// ---------------------------------------------------------------------------------------------
// Wave reductions (64 lanes): DPP moves within each row of 16 lanes (lanes i ^ 1, i ^ 2, then the
// half-row and row mirrors), then one lane of each of the four rows read into a scalar.  The result
// is the same in every lane, and the order of the operations is fixed.
// ---------------------------------------------------------------------------------------------
// Every pattern used reads a lane of the same row, so no lane takes the bound-control zero; written
// this way, the move folds into the add or max that consumes it (one DPP instruction per step).
template <int CTRL>
__device__ __forceinline__ uint32_t dpp_u32(uint32_t v) {
    return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, CTRL, 0xF, 0xF, true);
}
constexpr int kDppXor1 = 0xB1;        // quad_perm [1, 0, 3, 2]
constexpr int kDppXor2 = 0x4E;        // quad_perm [2, 3, 0, 1]
constexpr int kDppHalfMirror = 0x141; // lane i <-> 7 - i within each 8
constexpr int kDppMirror = 0x140;     // lane i <-> 15 - i within each 16
constexpr int kDppRowRor4 = 0x124;    // lane i takes lane (i - 4) mod 16 of its row of 16
constexpr int kDppRowRor8 = 0x128;    // lane i takes lane (i - 8) mod 16 of its row of 16

__device__ __forceinline__ uint32_t readlane_u32(uint32_t v, int l) {
    return (uint32_t)__builtin_amdgcn_readlane((int)v, l);
}

__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
    v = max(v, dpp_u32<kDppXor1>(v));
    v = max(v, dpp_u32<kDppXor2>(v));
    v = max(v, dpp_u32<kDppHalfMirror>(v));
    v = max(v, dpp_u32<kDppMirror>(v));
    return max(max(readlane_u32(v, 0), readlane_u32(v, 16)), max(readlane_u32(v, 32), readlane_u32(v, 48)));
}

__device__ __forceinline__ uint32_t wave_sum_u32(uint32_t v) {
    v += dpp_u32<kDppXor1>(v);
    v += dpp_u32<kDppXor2>(v);
    v += dpp_u32<kDppHalfMirror>(v);
    v += dpp_u32<kDppMirror>(v);
    return (readlane_u32(v, 0) + readlane_u32(v, 16)) + (readlane_u32(v, 32) + readlane_u32(v, 48));
}

__device__ __forceinline__ float wave_sum_f32(float v) {
    v += u2f(dpp_u32<kDppXor1>(f2u(v)));
    v += u2f(dpp_u32<kDppXor2>(f2u(v)));
    v += u2f(dpp_u32<kDppHalfMirror>(f2u(v)));
    v += u2f(dpp_u32<kDppMirror>(f2u(v)));
    return (u2f(readlane_u32(f2u(v), 0)) + u2f(readlane_u32(f2u(v), 16))) +
           (u2f(readlane_u32(f2u(v), 32)) + u2f(readlane_u32(f2u(v), 48)));
}

// s_waitcnt immediate: wait until at most `vm` vector-memory and `lgkm` LDS operations are pending.
constexpr int waitcnt_imm(int vm, int lgkm) { return (vm & 15) | (7 << 4) | ((lgkm & 15) << 8) | ((vm >> 4) << 14); }

// Buffer resource over `bytes` bytes at `base` (raw addressing: offsets in bytes, at most 2^31 - 1 of
// them in range; a load at an offset past the range returns zeros).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t buffer_rsrc(const void *base, uint64_t bytes) {
    const int n = bytes < 0x7FFFFFFFull ? (int)bytes : 0x7FFFFFFF;
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0, n, 0x00020000);
}
// An offset past every buffer_rsrc range.
constexpr uint32_t kOffsetPastRange = 0x80000000u;

// 16 bytes per lane from buffer `r` at (voff + soff) straight into LDS: lane l writes lds + 16 l.
// The compiler does not see these LDS writes: wait for the load (vmcnt) before reading them.
__device__ __forceinline__ void load_to_lds16(__amdgpu_buffer_rsrc_t r, void *lds, uint32_t voff, uint32_t soff) {
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void *)lds, 16, voff, soff, 0, 0);
}

// Pack two fp32 values that are exactly representable in bf16 (the decoded e2m1 x s products)
// into one dword of two bf16 (first value in the low half): the high halves are the bf16 values.
__device__ __forceinline__ uint32_t pack_bf16_exact(float lo, float hi) {
    return __builtin_amdgcn_perm(f2u(hi), f2u(lo), 0x07060302u);
}

}  // namespace nvfp4
