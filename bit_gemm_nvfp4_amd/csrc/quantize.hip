// NVFP4 quantization / requantization kernels for gfx950.
//
// What is computed ("Qwen-Image NVFP4 on a 16 GB Ada GPU", section "What NVFP4 is and how it differs
// from NF4"; "Qwen-Rapid-AIO-NVFP4", section "Why This Exists" for the FP8 source):
//   v      = source value widened to fp32 (E4M3 source: fl(e4m3(b) * src_scale))
//   g      = fl(amax / 2688)                        per tensor (amax run-time or static)
//   s_byte = E4M3_RNE_SAT(fl(bamax / fl(6 g)))      per 16 consecutive elements of a row
//   code   = sign(v) | E2M1_RNE_SAT(fl(|v| * fl(1 / fl(s g))))   per element, packed low nibble first
//
// Work decomposition: one wave encodes a tile of 64 blocks (1024 elements).  Every lane loads 16
// bytes per 16-byte vector, so each load instruction covers 1 KiB of contiguous input; block maxima
// are reduced over the lanes that share a block and re-distributed so that lane L owns block L of
// the tile and does the per-block divisions once; the per-block reciprocal goes back to the lanes
// holding the elements, which convert two values per instruction to E2M1.  The maximum is an
// integer max of magnitude bit patterns (non-negative floats order like their bit patterns; NaN
// patterns sort above infinity, so a non-finite input shows up in it).
//
// FP8 tensorwise output ("Qwen3-VL-8B-Instruct-heretic-NVFP4", "Quantization Details": float8_e4m3fn,
// tensorwise, round to nearest, for embed_tokens and lm_head; "Runtime / hardware": FP4 weights
// against dynamically quantized FP8 activations), the same kernels with OUTF = kOutFp8:
//   scale = fl(amax / 448) (1 when amax = 0); byte = sign | E4M3 nearest-even of fl(|v| / scale),
//   saturating at 448.  The hardware packed conversion (v_cvt_pk_fp8_f32) rounds to nearest even;
//   the quotient is clamped to +-448 first, so it never overflows.
//
// Launches (on the caller's stream): run-time amax -> k_quant_fused, one launch that reads the input
// once (below); static amax -> k_encode, one pass.
#include <hip/hip_runtime.h>

#include <atomic>

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

// Address of 16-byte vector `vi` of the tensor (vectors numbered row-major over the logical
// [rows x cols] shape).  Contiguous tensors are linear; otherwise split into row and column.
__device__ __forceinline__ const u32x4 *vec_addr(const uint8_t *x, uint64_t vi, uint32_t vpr, int64_t ld_bytes,
                                                 bool contiguous) {
    if (contiguous) return reinterpret_cast<const u32x4 *>(x) + vi;
    uint64_t r = vi / vpr;
    uint64_t c = vi - r * vpr;
    return reinterpret_cast<const u32x4 *>(x + r * (uint64_t)ld_bytes) + c;
}

// ---------------------------------------------------------------------------------------------
// One wave, one tile = 64 consecutive blocks (1024 elements).  Lane l holds vectors j * 64 + l of
// the tile (j < VPB), so each load instruction of the wave covers 1 KiB of contiguous input.
// ---------------------------------------------------------------------------------------------
struct TileGeom {
    const uint8_t *x;
    uint64_t nblocks;
    uint32_t vpr;  // vectors per row
    int64_t ld_bytes;
    int contiguous;
};

template <int SRC>
struct TileRegs {
    u32x4 raw[kVpb<SRC>];
};

template <int SRC>
__device__ __forceinline__ void tile_load(TileRegs<SRC> &t, const TileGeom &gm, uint64_t tile, int lane) {
    constexpr int VPB = kVpb<SRC>;
#pragma unroll
    for (int j = 0; j < VPB; j++) {
        const uint32_t vt = j * 64 + lane;
        const uint64_t blk = tile * 64 + vt / VPB;
        if (blk < gm.nblocks)
            t.raw[j] = *vec_addr(gm.x, blk * VPB + vt % VPB, gm.vpr, gm.ld_bytes, gm.contiguous);
        else
            t.raw[j] = u32x4{0u, 0u, 0u, 0u};
    }
}

// Block maxima: reduce over the VPB lanes holding one block, then hand block L of the tile to lane
// L.  Returns the largest magnitude bit pattern of lane L's block (0 past the end of the tensor).
template <int SRC>
__device__ __forceinline__ uint32_t tile_block_max(const TileRegs<SRC> &t, int lane) {
    constexpr int VPB = kVpb<SRC>;
    constexpr int BPL = 64 / VPB;  // blocks covered by one 64-lane load
    uint32_t pm[VPB];
#pragma unroll
    for (int j = 0; j < VPB; j++) {
        pm[j] = vec_absmax_bits<SRC>(t.raw[j]);
        // the VPB lanes of a block are neighbours (lanes i ^ 1, and i ^ 2 for four)
        if constexpr (VPB >= 2) pm[j] = max(pm[j], dpp_u32<kDppXor1>(pm[j]));
        if constexpr (VPB >= 4) pm[j] = max(pm[j], dpp_u32<kDppXor2>(pm[j]));
    }
    if constexpr (VPB == 1) {
        return pm[0];
    } else {
        const int src = (lane % BPL) * VPB;
        const int jj = lane / BPL;
        uint32_t bm = 0;
#pragma unroll
        for (int j = 0; j < VPB; j++) {
            const uint32_t v = (uint32_t)__shfl((int)pm[j], src, 64);
            if (j == jj) bm = v;
        }
        return bm;
    }
}

// Per-block scale byte and reciprocal for the block whose largest magnitude pattern is `bm` (lane
// L of a tile owns block L), given the global scale g (and 6 g).  No branches; a zero scale (g = 0,
// or a block of zeros) gives reciprocal 0.
struct BlockScale {
    uint32_t sbyte;
    float r;
};

template <int SRC>
__device__ __forceinline__ float block_amax(uint32_t bm, float sc) {
    if constexpr (SRC == NVFP4_E4M3) return e4m3_to_f32(bm) * sc;
    else return u2f(bm);
}

template <int SRC>
__device__ __forceinline__ bool block_nonfinite(uint32_t bm, float sc) {
    if constexpr (SRC == NVFP4_E4M3) return bm == 0x7Fu || !(block_amax<SRC>(bm, sc) <= 3.402823466e38f);
    else return bm >= 0x7F800000u;
}

template <int SRC>
__device__ __forceinline__ BlockScale block_scale(uint32_t bm, float g, float six_g, float sc) {
    const float q = block_amax<SRC>(bm, sc) / six_g;
    BlockScale b;
    b.sbyte = g != 0.0f ? e4m3_from_f32(q) : 0u;
    const float s = e4m3_to_f32(b.sbyte);
    const float rd = 1.0f / (s * g);
    b.r = s == 0.0f ? 0.0f : rd;
    return b;
}

// Write one tile: the scale bytes (lane L: block L) and the codes, each lane converting its own
// vectors with its block's reciprocal.  The conversions take one of two wave-uniform paths: the
// plain one, or, when some block's reciprocal overflowed, one that keeps zeros at zero.  Tiles
// wholly inside the tensor store without per-lane bounds checks.  The stores are non-temporal:
// little of the output is read back soon, and the kernel ends about 0.5 us sooner when the L2
// holds no dirty output lines to write back at its end.
template <int SRC>
__device__ __forceinline__ void tile_store(const TileRegs<SRC> &t, BlockScale b, float sc, uint64_t tile,
                                           uint64_t nblocks, uint8_t *__restrict__ codes,
                                           uint8_t *__restrict__ scales, int lane) {
    constexpr int EPV = kEpv<SRC>;
    constexpr int VPB = kVpb<SRC>;
    constexpr int BPL = 64 / VPB;
    const uint64_t blk0 = tile * 64;
    const bool full = blk0 + 64 <= nblocks;  // wave-uniform
    if (full || blk0 + lane < nblocks) __builtin_nontemporal_store((uint8_t)b.sbyte, scales + blk0 + lane);
    float rj[VPB];
#pragma unroll
    for (int j = 0; j < VPB; j++) rj[j] = VPB == 1 ? b.r : __shfl(b.r, j * BPL + lane / VPB, 64);
    uint32_t out[VPB][EPV / 8 > 0 ? EPV / 8 : 1];
    auto convert = [&](int j, bool keep_zero) {
        float v[EPV];
        widen<SRC>(t.raw[j], sc, v);
        float y[EPV];
#pragma unroll
        for (int e = 0; e < EPV; e++) y[e] = (keep_zero && v[e] == 0.0f) ? v[e] : v[e] * rj[j];
        if constexpr (EPV == 4) {
            out[j][0] = fp4_pack4(y);
        } else if constexpr (EPV == 8) {
            out[j][0] = fp4_pack8(y);
        } else {
            out[j][0] = fp4_pack8(y);
            out[j][1] = fp4_pack8(y + 8);
        }
    };
    if (__builtin_expect(__any(__builtin_isinf(b.r)), 0)) {
        // tiny s * g: fl(1 / d) overflowed; |v| * inf saturates, 0 stays 0 (no 0 * inf)
#pragma unroll
        for (int j = 0; j < VPB; j++) convert(j, true);
    } else {
#pragma unroll
        for (int j = 0; j < VPB; j++) convert(j, false);
    }
    // vector vt = j * 64 + lane of the tile holds elements (blk0 * VPB + vt) * EPV ..
    uint8_t *dst = codes + (blk0 * VPB + lane) * (EPV / 2);
    auto store = [&](int j) {
        if constexpr (EPV == 4) {
            __builtin_nontemporal_store((uint16_t)out[j][0], reinterpret_cast<uint16_t *>(dst + j * 64 * (EPV / 2)));
        } else if constexpr (EPV == 8) {
            __builtin_nontemporal_store(out[j][0], reinterpret_cast<uint32_t *>(dst + j * 64 * (EPV / 2)));
        } else {
            __builtin_nontemporal_store(u32x2{out[j][0], out[j][1]}, reinterpret_cast<u32x2 *>(dst + j * 64 * (EPV / 2)));
        }
    };
    if (full) {
#pragma unroll
        for (int j = 0; j < VPB; j++) store(j);
    } else {
#pragma unroll
        for (int j = 0; j < VPB; j++)
            if (blk0 + (j * 64 + lane) / VPB < nblocks) store(j);
    }
}

// Encode one tile whose lane-L block maximum is `bm`.  CHECK_FINITE: set bit 0 of `flags` for a
// non-finite block here (callers that derive the global scale from the run-time tensor maximum
// flag that maximum instead, which covers every block).
template <int SRC, bool CHECK_FINITE = true>
__device__ __forceinline__ void tile_encode(const TileRegs<SRC> &t, uint32_t bm, float g, float six_g, float sc,
                                            uint64_t tile, uint64_t nblocks, uint8_t *__restrict__ codes,
                                            uint8_t *__restrict__ scales, int32_t *__restrict__ flags, int lane) {
    if constexpr (CHECK_FINITE) {
        const bool bad = block_nonfinite<SRC>(bm, sc) && (tile * 64 + lane < nblocks);
        if (__any(bad) && lane == 0 && flags) atomicOr(flags, 1);
    }
    tile_store<SRC>(t, block_scale<SRC>(bm, g, six_g, sc), sc, tile, nblocks, codes, scales, lane);
}

// amax word (integer max of magnitude patterns; for E4M3 the largest magnitude byte) -> fp32 amax.
template <int SRC>
__device__ __forceinline__ float amax_from_bits(uint32_t bits, float sc, bool *nonfinite) {
    if constexpr (SRC == NVFP4_E4M3) {
        *nonfinite = (bits == 0x7Fu);
        const float a = e4m3_to_f32(bits) * sc;
        if (!(a <= 3.402823466e38f)) *nonfinite = true;
        return a;
    } else {
        *nonfinite = bits >= 0x7F800000u;
        return u2f(bits);
    }
}

// Output formats of the quantize kernels.
constexpr int kOutNvfp4 = 0;  // codes + block scales + global scale
constexpr int kOutFp8 = 1;    // E4M3 bytes + one tensor scale

// FP8 tensor scale from amax.
__device__ __forceinline__ float fp8_scale(float amax) { return amax == 0.0f ? 1.0f : amax / 448.0f; }

// Four quotients -> four E4M3 bytes (element i in byte i), each clamped to +-448 first.
__device__ __forceinline__ uint32_t fp8_pack4(float q0, float q1, float q2, float q3) {
    int w = __builtin_amdgcn_cvt_pk_fp8_f32(__builtin_amdgcn_fmed3f(q0, -448.0f, 448.0f),
                                            __builtin_amdgcn_fmed3f(q1, -448.0f, 448.0f), 0, false);
    w = __builtin_amdgcn_cvt_pk_fp8_f32(__builtin_amdgcn_fmed3f(q2, -448.0f, 448.0f),
                                        __builtin_amdgcn_fmed3f(q3, -448.0f, 448.0f), w, true);
    return (uint32_t)w;
}

// Write one tile as FP8: vector vt = j * 64 + lane of the tile holds elements (blk0 * VPB + vt) * EPV
// and becomes EPV bytes at the same element offset.  Each quotient is a correctly rounded fp32
// division by the tensor scale.
template <int SRC>
__device__ __forceinline__ void tile_store_fp8(const TileRegs<SRC> &t, float scale, float sc, uint64_t tile,
                                               uint64_t nblocks, uint8_t *__restrict__ out, int lane) {
    constexpr int EPV = kEpv<SRC>;
    constexpr int VPB = kVpb<SRC>;
    const uint64_t blk0 = tile * 64;
    const bool full = blk0 + 64 <= nblocks;  // wave-uniform
    uint32_t w[VPB][EPV / 4];
#pragma unroll
    for (int j = 0; j < VPB; j++) {
        float v[EPV];
        widen<SRC>(t.raw[j], sc, v);
#pragma unroll
        for (int e = 0; e < EPV; e += 4)
            w[j][e / 4] = fp8_pack4(v[e] / scale, v[e + 1] / scale, v[e + 2] / scale, v[e + 3] / scale);
    }
    uint8_t *dst = out + (blk0 * VPB + lane) * EPV;
    auto store = [&](int j) {
        uint8_t *d = dst + j * 64 * EPV;
        if constexpr (EPV == 4) {
            __builtin_nontemporal_store(w[j][0], reinterpret_cast<uint32_t *>(d));
        } else if constexpr (EPV == 8) {
            __builtin_nontemporal_store(u32x2{w[j][0], w[j][1]}, reinterpret_cast<u32x2 *>(d));
        } else {
            __builtin_nontemporal_store(u32x4{w[j][0], w[j][1], w[j][2], w[j][3]}, reinterpret_cast<u32x4 *>(d));
        }
    };
    if (full) {
#pragma unroll
        for (int j = 0; j < VPB; j++) store(j);
    } else {
#pragma unroll
        for (int j = 0; j < VPB; j++)
            if (blk0 + (j * 64 + lane) / VPB < nblocks) store(j);
    }
}

// Largest magnitude pattern over the lane's vectors of a tile (no per-block reduction).
template <int SRC>
__device__ __forceinline__ uint32_t tile_lane_max(const TileRegs<SRC> &t) {
    uint32_t m = 0;
#pragma unroll
    for (int j = 0; j < kVpb<SRC>; j++) m = max(m, vec_absmax_bits<SRC>(t.raw[j]));
    return m;
}

// ---------------------------------------------------------------------------------------------
// Static (calibrated) amax: the global scale is known up front, so one pass encodes.
// ---------------------------------------------------------------------------------------------
template <int SRC, int OUTF>
__global__ __launch_bounds__(256) void k_encode(TileGeom gm, const float *__restrict__ src_scale,
                                                const float *__restrict__ amax_in, uint8_t *__restrict__ codes,
                                                uint8_t *__restrict__ scales, float *__restrict__ g_out,
                                                int32_t *__restrict__ flags) {
    const int lane = threadIdx.x & 63, wid = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const float sc = (SRC == NVFP4_E4M3 && src_scale) ? *src_scale : 1.0f;
    const float g = OUTF == kOutFp8 ? fp8_scale(*amax_in) : *amax_in / 2688.0f;
    if (blockIdx.x == 0 && threadIdx.x == 0) *g_out = g;
    const float six_g = 6.0f * g;
    const uint64_t ntiles = (gm.nblocks + 63) / 64;
    const uint64_t nwaves = (uint64_t)gridDim.x * 4;
    uint64_t tile = (uint64_t)blockIdx.x * 4 + wid;
    if (tile >= ntiles) return;
    TileRegs<SRC> cur;
    tile_load<SRC>(cur, gm, tile, lane);
    for (;;) {
        const uint64_t next = tile + nwaves;
        TileRegs<SRC> nxt;
        if (next < ntiles) tile_load<SRC>(nxt, gm, next, lane);  // prefetch while encoding
        if constexpr (OUTF == kOutFp8) {
            // vectors past the end of the tensor were loaded as zeros
            if (__any(block_nonfinite<SRC>(tile_lane_max<SRC>(cur), sc)) && lane == 0 && flags) atomicOr(flags, 1);
            tile_store_fp8<SRC>(cur, g, sc, tile, gm.nblocks, codes, lane);
        } else {
            const uint32_t bm = tile_block_max<SRC>(cur, lane);
            tile_encode<SRC>(cur, bm, g, six_g, sc, tile, gm.nblocks, codes, scales, flags, lane);
        }
        if (next >= ntiles) break;
        tile = next;
        cur = nxt;
    }
}

// ---------------------------------------------------------------------------------------------
// Single-pass path: one launch of one workgroup of NWV waves per CU (16 waves: four per SIMD, with
// at most 128 VGPRs; 8 waves: two per SIMD), so that every workgroup is resident at once on an
// otherwise idle GPU.  Each wave loads its TPW tiles and keeps them in registers while the grid
// agrees on amax, then encodes them from registers, so the input crosses HBM once.  Tiles beyond
// the register capacity are streamed for the maximum and read again for the encode.
//
// Agreement on amax: every workgroup publishes one 64-bit word (call tag << 32 | its partial
// maximum) in its workspace slot, then polls all slots until each carries this call's tag and
// takes the maximum of their payloads.  Every workgroup reads every slot (one per CU, so a poll
// moves a few KB), so the maximum reaches all of them one memory round trip after the last slot
// is written, with no relay through a leader.  The payload travels inside the atomic word, so
// relaxed device-scope atomics suffice (no cache maintenance in the loop).
//
// Call tags: each workgroup slot has a tag record next to it, which the workgroup sets to the
// call's tag once its poll has found every slot carrying that tag.  A call's tag is one more than
// the largest tag record.  Every workgroup reads the records before it publishes (the tag is part
// of the published word) and a record is only written after every slot of the call is published,
// so all workgroups of a call read the same records and agree on the tag; the next call on the
// workspace, which the stream (or the caller's events) starts only after every workgroup of this
// one has finished, gets a larger one.  Nothing is cleared between calls, and a launch captured in
// a HIP graph (same kernel arguments on every replay) still works.  The records are written at
// distinct addresses, and the publish is a plain store, so nothing on the path to the agreement
// waits on a contended address.
//
// The polls are bounded: if other work kept some workgroups from being scheduled for that long,
// bit 1 of `flags` is set and the outputs are invalid, instead of a hang.  Workgroups that time out
// write no record; the late workgroups read the same records, find every slot of the call
// published, and write theirs, so the next call still gets a new tag.  A workgroup whose own slot
// already carries the call's tag before it publishes (a workspace that was not zeroed before first
// use, or calls that overlapped on it) sets bit 2 of `flags`: the polls may then have passed early.
// ---------------------------------------------------------------------------------------------
constexpr int kHeadWords = 16;  // reserved workspace words
// Workgroup slots of the workspace: kHeadWords words, one 32-bit tag record per slot, then one
// 64-bit slot per workgroup (16 KiB hold 1360: several workgroups per CU on any current part).
constexpr int kMaxSlots = (int)((kQuantizeWsBytes - kHeadWords * 4) / 12);
constexpr size_t kSlotByteOffset = (kHeadWords * 4 + kMaxSlots * 4 + 7) / 8 * 8;
static_assert(kSlotByteOffset + kMaxSlots * 8 <= kQuantizeWsBytes, "quantize workspace layout");
// The largest grid of the single-pass kernel on a device: one workgroup per CU, within the slots.
constexpr int max_grid_for(int num_cus) { return num_cus < kMaxSlots ? num_cus : kMaxSlots; }

constexpr uint32_t kPollLimit = 1u << 22;

// The body of the single-pass kernel for one tensor, worked on by the launch's workgroups lo .. hi - 1
// (all of them for one tensor; a share of them in a batch).  Every workgroup of the launch takes
// part in one agreement: it publishes its tensor's partial maximum in its own slot and waits for
// every slot, and the amax of its tensor is the maximum over the slots lo .. hi - 1.
template <int SRC, int TPW, int PB, int OUTF, int NWV, int LPW>
__device__ __forceinline__ void quant_fused_part(const TileGeom &gm, const float *__restrict__ src_scale,
                                                 uint32_t *__restrict__ ws, int nrec, uint8_t *__restrict__ codes,
                                                 uint8_t *__restrict__ scales, float *__restrict__ g_out,
                                                 int32_t *__restrict__ flags, uint32_t lo, uint32_t hi) {
    constexpr int VPB = kVpb<SRC>;
    __shared__ uint32_t red[NWV];
    __shared__ uint32_t amax_bits;
    // LDS-resident tiles: LPW per wave, each lane's vectors at [wave][tile][vector][lane]
    __shared__ u32x4 lds_tiles[LPW > 0 ? NWV * LPW * VPB * 64 : 1];
    const int lane = threadIdx.x & 63, wid = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const uint64_t ntiles = (gm.nblocks + 63) / 64;
    const uint64_t wave = (uint64_t)(blockIdx.x - lo) * NWV + wid, nwaves = (uint64_t)(hi - lo) * NWV;
    const float sc = (SRC == NVFP4_E4M3 && src_scale) ? *src_scale : 1.0f;
    uint32_t *records = ws + kHeadWords;
    uint64_t *slots = reinterpret_cast<uint64_t *>(reinterpret_cast<uint8_t *>(ws) + kSlotByteOffset);
    // tag records (wave 0): issued first, used after the tiles are in, so their latency is hidden.
    // nrec (the largest grid this device runs, the same for every call on it) bounds the records
    // any call on this workspace can have written.
    uint32_t rec[4] = {0u, 0u, 0u, 0u};
    uint64_t own_prev = 0;
    if (wid == 0) {
#pragma unroll
        for (int k = 0; k < 4; k++)
            if (lane + 64 * k < nrec)
                rec[k] = __hip_atomic_load(&records[lane + 64 * k], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        if (lane == 0) own_prev = __hip_atomic_load(&slots[blockIdx.x], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }

    // ---- phase 1: load the resident tiles, block maxima (NVFP4), tensor maximum ----
    // Tile s of the wave is tile wave + s * nwaves of the tensor: s < TPW stay in registers,
    // TPW <= s < TPW + LPW are kept in LDS, the rest is streamed.
    TileRegs<SRC> t[TPW];
    uint32_t bm[TPW];
    uint32_t bm_lds[LPW > 0 ? LPW : 1];
    uint32_t m = 0;
    u32x4 *my_lds = lds_tiles + (size_t)wid * (LPW > 0 ? LPW : 0) * VPB * 64;
    const auto resident_max = [&](int s) {
        if constexpr (OUTF == kOutFp8) {
            m = max(m, tile_lane_max<SRC>(t[s]));
        } else {
            bm[s] = tile_block_max<SRC>(t[s], lane);
            m = max(m, bm[s]);
        }
    };
    const auto lds_tile_max = [&](int l, const TileRegs<SRC> &x) {
        if constexpr (OUTF == kOutFp8) {
            m = max(m, tile_lane_max<SRC>(x));
        } else {
            bm_lds[l] = tile_block_max<SRC>(x, lane);
            m = max(m, bm_lds[l]);
        }
    };
    // (Where the LDS tiles fit in one round through the registers, that round measured faster.)
    if (gm.contiguous && (LPW == 0 || LPW > TPW)) {
        // Every load of the phase in flight at once: the LDS tiles go straight into LDS
        // (direct-to-LDS loads, no pass through registers), then the register tiles.  Vectors past
        // the end of the tensor read as zeros through the resource's range, so there is no branch.
        // (The offsets stay below 2^31: the resident tiles are the first (TPW + LPW) x waves tiles.)
        const __amdgpu_buffer_rsrc_t rx = buffer_rsrc(gm.x, gm.nblocks * VPB * 16);
        const auto vec_off = [&](uint64_t tile, int j) {
            const uint32_t vt = j * 64 + lane;
            const uint64_t blk = tile * 64 + vt / VPB;
            return blk < gm.nblocks ? (uint32_t)((blk * VPB + vt % VPB) * 16) : kOffsetPastRange;
        };
#pragma unroll
        for (int l = 0; l < LPW; l++)
#pragma unroll
            for (int j = 0; j < VPB; j++)
                load_to_lds16(rx, my_lds + (l * VPB + j) * 64, vec_off(wave + (TPW + l) * nwaves, j), 0);
#pragma unroll
        for (int s = 0; s < TPW; s++)
#pragma unroll
            for (int j = 0; j < VPB; j++)
                t[s].raw[j] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rx, vec_off(wave + s * nwaves, j), 0, 0));
        __builtin_amdgcn_sched_barrier(0);  // every load issued before the first maximum waits
#pragma unroll
        for (int s = 0; s < TPW; s++) resident_max(s);
        if constexpr (LPW > 0) {
            // the wave's own LDS tiles: landed once all its loads have (the compiler does not
            // see the direct-to-LDS writes, so wait explicitly)
            __builtin_amdgcn_s_waitcnt(waitcnt_imm(0, 15));
#pragma unroll
            for (int l = 0; l < LPW; l++) {
                TileRegs<SRC> x;
#pragma unroll
                for (int j = 0; j < VPB; j++) x.raw[j] = my_lds[(l * VPB + j) * 64 + lane];
                lds_tile_max(l, x);
            }
        }
    } else {
        // the LDS tiles pass through the register tiles first, in rounds of TPW
#pragma unroll
        for (int r0 = 0; r0 < LPW; r0 += TPW) {
#pragma unroll
            for (int i = 0; i < TPW; i++)
                if (r0 + i < LPW) tile_load<SRC>(t[i], gm, wave + (TPW + r0 + i) * nwaves, lane);
#pragma unroll
            for (int i = 0; i < TPW; i++) {
                if (r0 + i < LPW) {
                    lds_tile_max(r0 + i, t[i]);
#pragma unroll
                    for (int j = 0; j < VPB; j++) my_lds[((r0 + i) * VPB + j) * 64 + lane] = t[i].raw[j];
                }
            }
        }
#pragma unroll
        for (int s = 0; s < TPW; s++) tile_load<SRC>(t[s], gm, wave + s * nwaves, lane);
#pragma unroll
        for (int s = 0; s < TPW; s++) resident_max(s);
    }
    // tiles beyond the resident ones are streamed, PB loads in flight per wave
    for (uint64_t tile = wave + (TPW + LPW) * nwaves; tile < ntiles; tile += PB * nwaves) {
        TileRegs<SRC> o[PB];
#pragma unroll
        for (int b = 0; b < PB; b++) tile_load<SRC>(o[b], gm, tile + b * nwaves, lane);
#pragma unroll
        for (int b = 0; b < PB; b++)
#pragma unroll
            for (int j = 0; j < kVpb<SRC>; j++) m = max(m, vec_absmax_bits<SRC>(o[b].raw[j]));
    }
    m = wave_max_u32(m);
    if (lane == 0) red[wid] = m;
    // the call's tag: one more than the largest tag record (all workgroups read the same records,
    // since none is written before every slot of the call is published)
    uint32_t epoch = 0;
    if (wid == 0) {
        uint32_t t = max(max(rec[0], rec[1]), max(rec[2], rec[3]));
        for (int i = 256 + lane; i < nrec; i += 64)  // parts with more than 256 workgroups
            t = max(t, __hip_atomic_load(&records[i], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT));
        epoch = wave_max_u32(t) + 1u;
    }
    __syncthreads();
    if (wid == 0) {
        if (lane == 0) {
            uint32_t wgmax = 0;
#pragma unroll
            for (int i = 0; i < NWV; i++) wgmax = max(wgmax, red[i]);
            __hip_atomic_store(&slots[blockIdx.x], ((uint64_t)epoch << 32) | wgmax, __ATOMIC_RELAXED,
                               __HIP_MEMORY_SCOPE_AGENT);
            // its own slot already tagged for this call: the workspace was not zeroed before first
            // use, or was shared by overlapping calls
            if ((uint32_t)(own_prev >> 32) == epoch && flags) atomicOr(flags, 4);
        }
        // ---- wait for every slot of this call; all loads of a chunk of 8 slots per lane in
        // flight at once ----
        const uint32_t G = gridDim.x;
        uint32_t a = 0;
        bool agreed = false;
        for (uint32_t it = 0;; it++) {
            bool ready = true;
            a = 0;
            for (uint32_t base = 0; base < G; base += 512) {
                uint64_t v[8];
#pragma unroll
                for (int k = 0; k < 8; k++) {
                    const uint32_t i = base + (uint32_t)lane + 64u * k;
                    v[k] = i < G ? __hip_atomic_load(&slots[i], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT)
                                 : (uint64_t)epoch << 32;
                }
#pragma unroll
                for (int k = 0; k < 8; k++) {
                    const uint32_t i = base + (uint32_t)lane + 64u * k;
                    if ((uint32_t)(v[k] >> 32) != epoch) ready = false;
                    if (i >= lo && i < hi) a = max(a, (uint32_t)v[k]);
                }
            }
            if (__all(ready)) {
                agreed = true;
                break;
            }
            if (it >= kPollLimit) {
                if (lane == 0 && flags) atomicOr(flags, 2);
                break;
            }
            __builtin_amdgcn_s_sleep(1);
        }
        a = wave_max_u32(a);
        if (lane == 0) amax_bits = a;
        // every slot carried this call's tag, so every workgroup has read the records: write this one
        if (lane == 0 && agreed)
            __hip_atomic_store(&records[blockIdx.x], epoch, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    __syncthreads();
    m = amax_bits;
    bool nonfinite = false;
    const float amax = amax_from_bits<SRC>(m, sc, &nonfinite);
    const float g = OUTF == kOutFp8 ? fp8_scale(amax) : amax / 2688.0f;
    if (blockIdx.x == lo && threadIdx.x == 0) {
        *g_out = g;
        if (nonfinite && flags) atomicOr(flags, 1);
    }
    const float six_g = 6.0f * g;
    if constexpr (OUTF == kOutFp8) {
        // ---- phase 2 (FP8): convert the resident tiles, then the streamed ones ----
#pragma unroll
        for (int s = 0; s < TPW; s++) {
            const uint64_t tile = wave + s * nwaves;
            if (tile < ntiles) tile_store_fp8<SRC>(t[s], g, sc, tile, gm.nblocks, codes, lane);
        }
#pragma unroll
        for (int l = 0; l < LPW; l++) {
            const uint64_t tile = wave + (TPW + l) * nwaves;
            if (tile < ntiles) {
#pragma unroll
                for (int j = 0; j < VPB; j++) t[0].raw[j] = my_lds[(l * VPB + j) * 64 + lane];
                tile_store_fp8<SRC>(t[0], g, sc, tile, gm.nblocks, codes, lane);
            }
        }
        for (uint64_t tile = wave + (TPW + LPW) * nwaves; tile < ntiles; tile += PB * nwaves) {
            TileRegs<SRC> o[PB];
#pragma unroll
            for (int b = 0; b < PB; b++) tile_load<SRC>(o[b], gm, tile + b * nwaves, lane);
#pragma unroll
            for (int b = 0; b < PB; b++)
                if (tile + b * nwaves < ntiles) tile_store_fp8<SRC>(o[b], g, sc, tile + b * nwaves, gm.nblocks, codes, lane);
        }
        return;
    }

    // ---- phase 2: encode the resident tiles, then the streamed ones ----
    // the per-block divisions of all resident tiles first (independent, so they overlap), then
    // the conversions and stores tile by tile
    BlockScale bs[TPW];
#pragma unroll
    for (int s = 0; s < TPW; s++) bs[s] = block_scale<SRC>(bm[s], g, six_g, sc);
#pragma unroll
    for (int s = 0; s < TPW; s++) {
        const uint64_t tile = wave + s * nwaves;
        if (tile < ntiles) tile_store<SRC>(t[s], bs[s], sc, tile, gm.nblocks, codes, scales, lane);
    }
    // then the LDS tiles, each through a register tile
#pragma unroll
    for (int l = 0; l < LPW; l++) {
        const uint64_t tile = wave + (TPW + l) * nwaves;
        if (tile < ntiles) {
#pragma unroll
            for (int j = 0; j < VPB; j++) t[0].raw[j] = my_lds[(l * VPB + j) * 64 + lane];
            tile_store<SRC>(t[0], block_scale<SRC>(bm_lds[l], g, six_g, sc), sc, tile, gm.nblocks, codes, scales,
                            lane);
        }
    }
    for (uint64_t tile = wave + (TPW + LPW) * nwaves; tile < ntiles; tile += PB * nwaves) {
        TileRegs<SRC> o[PB];
#pragma unroll
        for (int b = 0; b < PB; b++) tile_load<SRC>(o[b], gm, tile + b * nwaves, lane);
#pragma unroll
        for (int b = 0; b < PB; b++) {
            const uint64_t tb = tile + b * nwaves;
            if (tb < ntiles)
                tile_encode<SRC, false>(o[b], tile_block_max<SRC>(o[b], lane), g, six_g, sc, tb, gm.nblocks, codes,
                                        scales, flags, lane);
        }
    }
}

template <int SRC, int TPW, int PB, int OUTF, int NWV, int LPW>
__global__ __launch_bounds__(NWV * 64) void k_quant_fused(TileGeom gm, const float *__restrict__ src_scale,
                                                          uint32_t *__restrict__ ws, int nrec,
                                                          uint8_t *__restrict__ codes,
                                                          uint8_t *__restrict__ scales, float *__restrict__ g_out,
                                                          int32_t *__restrict__ flags) {
    quant_fused_part<SRC, TPW, PB, OUTF, NWV, LPW>(gm, src_scale, ws, nrec, codes, scales, g_out, flags, 0u,
                                                   gridDim.x);
}

// A batch of tensors in one launch: tensor i is worked on by the workgroups part[i].wg_lo ..
// part[i].wg_hi - 1 (consecutive ranges covering the grid), each with its own amax.
struct QPart {
    TileGeom gm;
    const float *src_scale;
    uint8_t *codes;
    uint8_t *scales;
    float *g_out;
    uint32_t wg_lo, wg_hi;
};
struct QBatch {
    QPart part[kQuantizeMaxBatch];
    int n;
};

template <int SRC, int TPW, int NWV>
__global__ __launch_bounds__(NWV * 64) void k_quant_fused_batch(QBatch b, uint32_t *__restrict__ ws, int nrec,
                                                                int32_t *__restrict__ flags) {
    int i = 0;
    while (i + 1 < b.n && blockIdx.x >= b.part[i].wg_hi) i++;
    const QPart &p = b.part[i];
    quant_fused_part<SRC, TPW, 1, kOutNvfp4, NWV, 0>(p.gm, p.src_scale, ws, nrec, p.codes, p.scales, p.g_out, flags,
                                                     p.wg_lo, p.wg_hi);
}

// ---------------------------------------------------------------------------------------------
// Run-time amax as a pass of its own (the two-launch form): per-workgroup maxima of the magnitude
// bit patterns into the workspace, then one workgroup reduces them and writes amax as fp32.  No
// workgroup waits for another, so it makes no assumption about which kernels share the GPU.
// ---------------------------------------------------------------------------------------------
template <int SRC>
__global__ __launch_bounds__(256) void k_amax_partial(TileGeom gm, uint32_t *__restrict__ partial) {
    __shared__ uint32_t red[4];
    const int lane = threadIdx.x & 63, wid = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const uint64_t ntiles = (gm.nblocks + 63) / 64;
    const uint64_t nwaves = (uint64_t)gridDim.x * 4;
    uint32_t m = 0;
    uint64_t tile = (uint64_t)blockIdx.x * 4 + wid;
    // two tiles in flight per wave
    for (; tile + nwaves < ntiles; tile += 2 * nwaves) {
        TileRegs<SRC> a, b;
        tile_load<SRC>(a, gm, tile, lane);
        tile_load<SRC>(b, gm, tile + nwaves, lane);
        m = max(m, max(tile_lane_max<SRC>(a), tile_lane_max<SRC>(b)));
    }
    if (tile < ntiles) {
        TileRegs<SRC> a;
        tile_load<SRC>(a, gm, tile, lane);
        m = max(m, tile_lane_max<SRC>(a));
    }
    m = wave_max_u32(m);
    if (lane == 0) red[wid] = m;
    __syncthreads();
    if (threadIdx.x == 0) partial[blockIdx.x] = max(max(red[0], red[1]), max(red[2], red[3]));
}

template <int SRC>
__global__ __launch_bounds__(256) void k_amax_final(const uint32_t *__restrict__ partial, int nparts,
                                                    const float *__restrict__ src_scale, float *__restrict__ amax_out,
                                                    int32_t *__restrict__ flags) {
    __shared__ uint32_t red[4];
    const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
    uint32_t m = 0;
    for (int i = threadIdx.x; i < nparts; i += 256) m = max(m, partial[i]);
    m = wave_max_u32(m);
    if (lane == 0) red[wid] = m;
    __syncthreads();
    if (threadIdx.x == 0) {
        const float sc = (SRC == NVFP4_E4M3 && src_scale) ? *src_scale : 1.0f;
        bool nonfinite = false;
        *amax_out = amax_from_bits<SRC>(max(max(red[0], red[1]), max(red[2], red[3])), sc, &nonfinite);
        if (nonfinite && flags) atomicOr(flags, 1);
    }
}

static int grid_for(uint64_t work_items, int per_block, int max_blocks) {
    uint64_t b = (work_items + per_block - 1) / per_block;
    if (b < 1) b = 1;
    if (b > (uint64_t)max_blocks) b = max_blocks;
    return (int)b;
}

// Largest residency (tiles per wave) whose registers still leave room for four waves per SIMD (at
// most 128 VGPRs).
template <int SRC>
constexpr int kMaxTpw4 = SRC == NVFP4_F32 ? 4 : SRC == NVFP4_BF16 ? 5 : SRC == NVFP4_F16 ? 8 : 12;
// With part of the tiles in LDS (16 waves sharing the 160 KiB, less 1 KiB for the reductions):
// register tiles and LDS tiles per wave, the register tiles fewer where the LDS tiles' block maxima
// would push the wave past 128 VGPRs.  Tensors beyond that keep the same residency and stream the
// rest (read once for the maximum, again for the encode), one tile in flight per wave.
template <int SRC>
constexpr int kTpw16L = SRC == NVFP4_F32 ? 4 : SRC == NVFP4_BF16 ? 4 : SRC == NVFP4_F16 ? 8 : 8;
template <int SRC>
constexpr int kLds16 = (159 * 1024 / 16) / (1024 * SrcTraits<SRC>::kElemBytes);

// Workgroups of k_quant_fused<SRC, TPW, PB, OUTF, NWV, LPW> that can be resident on one CU (at
// least one is assumed), from the runtime's occupancy calculation; computed once per instantiation.
template <int SRC, int TPW, int PB, int OUTF, int NWV, int LPW>
static int fused_per_cu() {
    static std::atomic<int> cached{0};
    int n = cached.load(std::memory_order_relaxed);
    if (n == 0) {
        int b = 0;
        if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&b, k_quant_fused<SRC, TPW, PB, OUTF, NWV, LPW>, NWV * 64, 0) !=
                hipSuccess ||
            b < 1)
            b = 1;
        n = b;
        cached.store(n, std::memory_order_relaxed);
    }
    return n;
}

// The grid barrier needs every workgroup resident at once, so the grid never exceeds what the
// CUs hold; waves then take more tiles than TPW and stream the rest.
// Output pointers of one quantize call: NVFP4 codes / block scales / global scale, or FP8 bytes (in
// `codes`) and the tensor scale (in `scale`).
struct QOut {
    uint8_t *codes;
    uint8_t *scales;
    float *scale;
};

template <int SRC, int TPW, int OUTF, int NWV, int PB = 1, int LPW = 0>
static void launch_fused(const TileGeom &gm, int grid, const float *src_scale, uint32_t *ws, const QOut &out,
                         int32_t *flags, int num_cus, hipStream_t stream) {
    const int cap = fused_per_cu<SRC, TPW, PB, OUTF, NWV, LPW>() * num_cus;
    if (grid > cap) grid = cap;
    // every launch on this device stays within max_grid_for(num_cus) workgroups, so that many tag
    // records cover every record a call on this workspace can have written
    hipLaunchKernelGGL((k_quant_fused<SRC, TPW, PB, OUTF, NWV, LPW>), dim3(grid), dim3(NWV * 64), 0, stream, gm,
                       src_scale, ws, max_grid_for(num_cus), out.codes, out.scales, out.scale, flags);
}

// Resident launch: tiles per wave rounded up to a supported residency, at most T.
template <int SRC, int OUTF, int NWV, int T>
static void launch_resident(const TileGeom &gm, int grid, uint64_t tpw, const float *src_scale, uint32_t *ws,
                            const QOut &out, int32_t *flags, int num_cus, hipStream_t stream) {
#define NVFP4_LAUNCH(T_) launch_fused<SRC, (T_), OUTF, NWV>(gm, grid, src_scale, ws, out, flags, num_cus, stream)
    if (tpw <= 1) NVFP4_LAUNCH(1);
    else if (tpw <= 2) NVFP4_LAUNCH(2);
    else if (tpw <= 3) NVFP4_LAUNCH(3);
    else if (tpw <= 4 || T < 5) NVFP4_LAUNCH(T < 4 ? T : 4);
    else if (tpw <= 5 || T < 6) NVFP4_LAUNCH(T < 5 ? T : 5);
    else if (tpw <= 6 || T < 8) NVFP4_LAUNCH(T < 6 ? T : 6);
    else if (tpw <= 8 || T < 12) NVFP4_LAUNCH(T < 8 ? T : 8);
    else if (tpw <= 12 || T < 16) NVFP4_LAUNCH(T < 12 ? T : 12);
    else NVFP4_LAUNCH(T);
#undef NVFP4_LAUNCH
}

// Tiles spread over all CUs, one workgroup of 16 waves each (four waves per SIMD hide each other's
// latencies): all tiles in registers when they fit the 128-VGPR budget (fewer workgroups for small
// tensors), else part of them in LDS; beyond that residency the rest is streamed (read twice).
template <int SRC, int OUTF>
static void launch_fused_any(const TileGeom &gm, const float *src_scale, uint32_t *ws, const QOut &out,
                             int32_t *flags, int num_cus, hipStream_t stream) {
    const uint64_t ntiles = (gm.nblocks + 63) / 64;
    const int max_grid = max_grid_for(num_cus);
    const int grid16 = grid_for(ntiles, 16, max_grid);
    const uint64_t tpw16 = (ntiles + 16 * (uint64_t)grid16 - 1) / (16 * (uint64_t)grid16);
    if constexpr (SRC == NVFP4_F32 && OUTF == kOutNvfp4) {
        // fp32 carries four elements per 16-byte vector, half the encode work per byte of the 16-bit
        // sources: where each of 16 waves would hold three tiles or more and 8 waves per CU can still
        // keep every tile in registers, one 8-wave workgroup per CU starts sooner and finishes
        // sooner (3072 x 3072: 14.3 -> 13.6 us; a 4096 x 3072 bf16 tensor, by contrast, took 11.6 ->
        // 12.2 us with 8 waves, and 512 x 12288 fp32, two tiles per wave at 16, 10.5 -> 10.6 us).
        const int grid8 = grid_for(ntiles, 8, max_grid);
        const uint64_t tpw8 = (ntiles + 8 * (uint64_t)grid8 - 1) / (8 * (uint64_t)grid8);
        if (tpw16 >= 3 && tpw8 <= (uint64_t)(2 * kMaxTpw4<SRC>)) {
            launch_resident<SRC, OUTF, 8, 2 * kMaxTpw4<SRC>>(gm, grid8, tpw8, src_scale, ws, out, flags, max_grid,
                                                               stream);
            return;
        }
    }
    if (tpw16 <= (uint64_t)kMaxTpw4<SRC>) {
        launch_resident<SRC, OUTF, 16, kMaxTpw4<SRC>>(gm, grid16, tpw16, src_scale, ws, out, flags, max_grid, stream);
        return;
    }
    launch_fused<SRC, kTpw16L<SRC>, OUTF, 16, 1, kLds16<SRC>>(gm, grid16, src_scale, ws, out, flags, max_grid, stream);
}

template <int SRC, int OUTF>
static hipError_t launch_quantize_t(const void *x, int64_t ld_x, int64_t rows, int64_t cols, const float *src_scale,
                                    const float *amax_in, const QOut &out, int32_t *flags, uint32_t *ws,
                                    int num_cus, hipStream_t stream) {
    constexpr int EB = SrcTraits<SRC>::kElemBytes;
    TileGeom gm;
    gm.x = (const uint8_t *)x;
    gm.nblocks = (uint64_t)rows * (uint64_t)(cols / 16);
    gm.vpr = (uint32_t)(cols / 16) * (uint32_t)kVpb<SRC>;
    gm.ld_bytes = ld_x * EB;
    gm.contiguous = (ld_x == cols) ? 1 : 0;
    const uint64_t ntiles = (gm.nblocks + 63) / 64;
    if (!amax_in) {
        launch_fused_any<SRC, OUTF>(gm, src_scale, ws, out, flags, num_cus, stream);
        return hipGetLastError();
    }
    hipLaunchKernelGGL((k_encode<SRC, OUTF>), dim3(grid_for(ntiles, 4, num_cus * 8)), dim3(256), 0, stream, gm,
                       src_scale, amax_in, out.codes, out.scales, out.scale, flags);
    return hipGetLastError();
}

// Workgroups of k_quant_fused_batch<SRC, TPW, NWV> one CU holds at once (at least one is assumed).
template <int SRC, int TPW, int NWV>
static int batch_per_cu() {
    static std::atomic<int> cached{0};
    int n = cached.load(std::memory_order_relaxed);
    if (n == 0) {
        int b = 0;
        if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&b, k_quant_fused_batch<SRC, TPW, NWV>, NWV * 64, 0) !=
                hipSuccess ||
            b < 1)
            b = 1;
        n = b;
        cached.store(n, std::memory_order_relaxed);
    }
    return n;
}

// The batch's workgroups are shared out in proportion to the tensors' tiles (at least one each,
// about 16 tiles per workgroup at least, at most one workgroup per CU), and the tiles per wave
// that the largest share needs pick the residency; beyond the register residency nothing is
// launched (the caller then quantizes the tensors one by one).
template <int SRC>
static hipError_t launch_quantize_batch_t(int count, const void *const *x, const int64_t *ld_x,
                                          const float *const *src_scale, const nvfp4_tensor *out,
                                          int32_t *flags, uint32_t *ws, int num_cus, hipStream_t stream,
                                          bool *batched) {
    constexpr int NWV = 16;
    constexpr int EB = SrcTraits<SRC>::kElemBytes;
    QBatch b{};
    b.n = count;
    uint64_t tiles[kQuantizeMaxBatch], total = 0;
    for (int i = 0; i < count; i++) {
        TileGeom &gm = b.part[i].gm;
        gm.x = (const uint8_t *)x[i];
        gm.nblocks = (uint64_t)out[i].rows * (uint64_t)(out[i].cols / 16);
        gm.vpr = (uint32_t)(out[i].cols / 16) * (uint32_t)kVpb<SRC>;
        gm.ld_bytes = ld_x[i] * EB;
        gm.contiguous = (ld_x[i] == out[i].cols) ? 1 : 0;
        b.part[i].src_scale = src_scale ? src_scale[i] : nullptr;
        b.part[i].codes = out[i].codes;
        b.part[i].scales = out[i].scales;
        b.part[i].g_out = out[i].global_scale;
        tiles[i] = (gm.nblocks + 63) / 64;
        total += tiles[i];
    }
    const uint64_t max_grid = (uint64_t)max_grid_for(num_cus);
    uint64_t grid = (total + 15) / 16;
    if (grid > max_grid) grid = max_grid;
    if (grid < (uint64_t)count) grid = (uint64_t)count;
    if (grid > max_grid) return hipSuccess;  // more tensors than workgroups: not batched
    uint64_t share[kQuantizeMaxBatch], used = 0;
    for (int i = 0; i < count; i++) {
        share[i] = total ? tiles[i] * grid / total : 1;
        if (share[i] < 1) share[i] = 1;
        used += share[i];
    }
    while (used > grid) {  // rounding up to one workgroup each can overshoot: trim the largest shares
        int k = 0;
        for (int i = 1; i < count; i++)
            if (share[i] > share[k]) k = i;
        share[k]--;
        used--;
    }
    while (used < grid) {  // hand the rest to the shares with the most tiles per workgroup
        int k = 0;
        for (int i = 1; i < count; i++)
            if (tiles[i] * share[k] > tiles[k] * share[i]) k = i;
        share[k]++;
        used++;
    }
    uint64_t tpw = 1;
    uint32_t lo = 0;
    for (int i = 0; i < count; i++) {
        const uint64_t t = (tiles[i] + NWV * share[i] - 1) / (NWV * share[i]);
        tpw = t > tpw ? t : tpw;
        b.part[i].wg_lo = lo;
        lo += (uint32_t)share[i];
        b.part[i].wg_hi = lo;
    }
    constexpr int T = kMaxTpw4<SRC>;
    if (tpw > (uint64_t)T) return hipSuccess;  // beyond the register residency: not batched
#define NVFP4_LAUNCH_BATCH(T_)                                                                                   \
    do {                                                                                                         \
        if ((uint64_t)batch_per_cu<SRC, (T_), NWV>() * (uint64_t)num_cus < grid) return hipSuccess;             \
        hipLaunchKernelGGL((k_quant_fused_batch<SRC, (T_), NWV>), dim3((unsigned)grid), dim3(NWV * 64), 0,      \
                           stream, b, ws, max_grid_for(num_cus), flags);                                       \
    } while (0)
    if (tpw <= 1) NVFP4_LAUNCH_BATCH(1);
    else if (tpw <= 2) NVFP4_LAUNCH_BATCH(2);
    else if (tpw <= 3) NVFP4_LAUNCH_BATCH(3);
    else if (tpw <= 4 || T < 5) NVFP4_LAUNCH_BATCH(T < 4 ? T : 4);
    else if (tpw <= 5 || T < 6) NVFP4_LAUNCH_BATCH(T < 5 ? T : 5);
    else if (tpw <= 6 || T < 8) NVFP4_LAUNCH_BATCH(T < 6 ? T : 6);
    else if (tpw <= 8 || T < 12) NVFP4_LAUNCH_BATCH(T < 8 ? T : 8);
    else NVFP4_LAUNCH_BATCH(T < 12 ? T : 12);
#undef NVFP4_LAUNCH_BATCH
    *batched = true;
    return hipGetLastError();
}

hipError_t launch_quantize_batch(int count, const void *const *x, nvfp4_dtype dt, const int64_t *ld_x,
                                 const float *const *src_scale, const nvfp4_tensor *out, int32_t *flags,
                                 void *workspace, int num_cus, hipStream_t stream, bool *batched) {
    *batched = false;
    if (count < 1 || count > kQuantizeMaxBatch) return hipSuccess;
    uint32_t *ws = reinterpret_cast<uint32_t *>(workspace);
    switch (dt) {
    case NVFP4_F32:
        return launch_quantize_batch_t<NVFP4_F32>(count, x, ld_x, src_scale, out, flags, ws, num_cus, stream, batched);
    case NVFP4_BF16:
        return launch_quantize_batch_t<NVFP4_BF16>(count, x, ld_x, src_scale, out, flags, ws, num_cus, stream, batched);
    case NVFP4_F16:
        return launch_quantize_batch_t<NVFP4_F16>(count, x, ld_x, src_scale, out, flags, ws, num_cus, stream, batched);
    default:
        return launch_quantize_batch_t<NVFP4_E4M3>(count, x, ld_x, src_scale, out, flags, ws, num_cus, stream, batched);
    }
}

template <int SRC>
static hipError_t launch_amax_t(const void *x, int64_t ld_x, int64_t rows, int64_t cols, const float *src_scale,
                                float *amax_out, int32_t *flags, uint32_t *ws, int num_cus, hipStream_t stream) {
    TileGeom gm;
    gm.x = (const uint8_t *)x;
    gm.nblocks = (uint64_t)rows * (uint64_t)(cols / 16);
    gm.vpr = (uint32_t)(cols / 16) * (uint32_t)kVpb<SRC>;
    gm.ld_bytes = ld_x * SrcTraits<SRC>::kElemBytes;
    gm.contiguous = (ld_x == cols) ? 1 : 0;
    const uint64_t ntiles = (gm.nblocks + 63) / 64;
    const int cap = num_cus * 4 < kAmaxMaxParts ? num_cus * 4 : kAmaxMaxParts;
    const int grid = grid_for(ntiles, 8, cap);  // about 8 tiles per workgroup (2 per wave) at least
    hipLaunchKernelGGL((k_amax_partial<SRC>), dim3(grid), dim3(256), 0, stream, gm, ws);
    hipLaunchKernelGGL((k_amax_final<SRC>), dim3(1), dim3(256), 0, stream, (const uint32_t *)ws, grid, src_scale,
                       amax_out, flags);
    return hipGetLastError();
}

hipError_t launch_amax(const void *x, nvfp4_dtype dt, int64_t ld_x, int64_t rows, int64_t cols, const float *src_scale,
                       float *amax_out, int32_t *flags, void *workspace, int num_cus, hipStream_t stream) {
    uint32_t *ws = reinterpret_cast<uint32_t *>(workspace);
    switch (dt) {
    case NVFP4_F32: return launch_amax_t<NVFP4_F32>(x, ld_x, rows, cols, src_scale, amax_out, flags, ws, num_cus, stream);
    case NVFP4_BF16: return launch_amax_t<NVFP4_BF16>(x, ld_x, rows, cols, src_scale, amax_out, flags, ws, num_cus, stream);
    case NVFP4_F16: return launch_amax_t<NVFP4_F16>(x, ld_x, rows, cols, src_scale, amax_out, flags, ws, num_cus, stream);
    default: return launch_amax_t<NVFP4_E4M3>(x, ld_x, rows, cols, src_scale, amax_out, flags, ws, num_cus, stream);
    }
}

template <int OUTF>
static hipError_t launch_quantize_any(const void *x, nvfp4_dtype dt, int64_t ld_x, int64_t rows, int64_t cols,
                                      const float *src_scale, const float *amax_in, const QOut &out, int32_t *flags,
                                      uint32_t *ws, int num_cus, hipStream_t stream) {
    switch (dt) {
    case NVFP4_F32:
        return launch_quantize_t<NVFP4_F32, OUTF>(x, ld_x, rows, cols, src_scale, amax_in, out, flags, ws, num_cus,
                                                  stream);
    case NVFP4_BF16:
        return launch_quantize_t<NVFP4_BF16, OUTF>(x, ld_x, rows, cols, src_scale, amax_in, out, flags, ws, num_cus,
                                                   stream);
    case NVFP4_F16:
        return launch_quantize_t<NVFP4_F16, OUTF>(x, ld_x, rows, cols, src_scale, amax_in, out, flags, ws, num_cus,
                                                  stream);
    default:
        return launch_quantize_t<NVFP4_E4M3, OUTF>(x, ld_x, rows, cols, src_scale, amax_in, out, flags, ws, num_cus,
                                                   stream);
    }
}

hipError_t launch_quantize(const void *x, nvfp4_dtype dt, int64_t ld_x, const float *src_scale, const float *amax_in,
                           const nvfp4_tensor *out, int32_t *flags, void *workspace, int num_cus,
                           hipStream_t stream) {
    const QOut o{out->codes, out->scales, out->global_scale};
    return launch_quantize_any<kOutNvfp4>(x, dt, ld_x, out->rows, out->cols, src_scale, amax_in, o, flags,
                                          reinterpret_cast<uint32_t *>(workspace), num_cus, stream);
}

hipError_t launch_quantize_fp8(const void *x, nvfp4_dtype dt, int64_t ld_x, int64_t rows, int64_t cols,
                               const float *src_scale, const float *amax_in, uint8_t *out, float *out_scale,
                               int32_t *flags, void *workspace, int num_cus, hipStream_t stream) {
    const QOut o{out, nullptr, out_scale};
    return launch_quantize_any<kOutFp8>(x, dt, ld_x, rows, cols, src_scale, amax_in, o, flags,
                                        reinterpret_cast<uint32_t *>(workspace), num_cus, stream);
}

}  // namespace nvfp4
