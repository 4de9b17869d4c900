// NVFP4-weight GEMM for gfx950: C[M x N] fp32 = A . W_hat^T, W an NVFP4 tensor [N x K].
//
// What is computed: "Qwen-Image NVFP4 on a 16 GB Ada GPU", section "Running the NVFP4 weights on
// Ada": without FP4 matrix hardware the packed weights are expanded to bf16 before the multiply and
// the activations stay bf16 (W4A16); section "What NVFP4 is and how it differs from NF4": Blackwell
// multiplies weights and activations both in 4 bits (W4A4, here with run-time quantized activations
// as in "Qwen3-VL-8B-Instruct-heretic-NVFP4", "Runtime / hardware").
//
// Design for CDNA4 (prior art kept only where it holds): the E4M3 block scale is per 16 elements
// with a 3-bit mantissa, while gfx950's scaled FP4 matrix instructions take power-of-two scales per
// 32 elements, so they cannot reproduce NVFP4 values.  e2m1 x s has at most 6 significant bits and
// lies in [2^-10, 2688], so it is exact in bf16: tiles are expanded exactly to bf16 in LDS and fed
// to the bf16 matrix cores (v_mfma_f32_32x32x16_bf16, fp32 accumulation); the global scale(s)
// multiply the fp32 sums in the epilogue.
//
// k_gemm_mfma (K % 64 == 0): BM x BN output tile per workgroup, K in steps of 64.
//   - bf16 A rows go straight from global memory into LDS (buffer loads with the LDS bit), three
//     stages deep, so a tile arrives two steps before it is used without passing through registers;
//     each 128-byte LDS row stores its 16-byte chunks XOR-swizzled by the row index, which keeps the
//     matrix-fragment reads free of bank conflicts without padding.
//   - NVFP4 operands (W, and A in the W4A4 form) are loaded two steps ahead into registers, one
//     code dword (8 elements) and its scale byte per unit, spread evenly over all threads; the
//     units of step s + 1 are expanded exactly and written to the other LDS stage between the
//     matrix instructions of step s.  One barrier per step.
//   - Wave tiles up to 64 x 96 keep all four 16-deep fragment slices of a step in registers and
//     place the barrier after the second slice: the expansion goes between the matrix
//     instructions of slices 0 and 1, and the first two slices of the next step are read under
//     those of slices 2 and 3, so no fragment read waits at the start of a step.
//   - The block scale byte is decoded by the hardware FP8 conversion (OCP e4m3).
//   - W4A4 expands both operands to f16 instead of bf16: e2m1 x s lies in [2^-10, 2688] with at
//     most 6 significant bits, so it is exact in f16 as well, and the f16 form needs half the
//     instructions (packed conversion, then one packed multiply per pair).
// k_gemm_tile: the same tiling for K % 64 != 0, with plain loads and bounds checks on K.
// Workgroup ids are remapped so that the workgroups the hardware places on one XCD (ids congruent
// mod 8) take neighbouring tiles that share W columns in that XCD's L2.
//
// k_gemv: for M <= 5 the product is bound by streaming W once from HBM.  A (bf16, or NVFP4 / E4M3
// activations expanded exactly to bf16) sits in LDS; each lane takes whole 16-element blocks of a W
// row, forms the 16-term dot products with bf16 dot2 instructions and applies the block scale once
// per block; a wave reduction finishes each row.  A wave works on two rows at once with all their loads issued ahead of the arithmetic.
#include <hip/hip_runtime.h>

#include <atomic>
#include <cstdlib>

#include <type_traits>

#include "common.h"
#include "internal.h"
#include "lowrank.h"

namespace nvfp4 {

constexpr int kBK = 64;   // K per main-loop step (4 NVFP4 blocks)
constexpr int kPad = 8;   // bf16 elements of row padding in LDS (16 bytes): spreads rows over banks
constexpr int kLdsRow = kBK + kPad;

// Expand 8 codes (one dword) with block scale s into 8 exact bf16 values (4 dwords).
__device__ __forceinline__ u32x4 expand8(uint32_t w, float s) {
    float v[8];
    fp4_unpack8_f32(w, v);
    u32x4 o;
#pragma unroll
    for (int q = 0; q < 4; q++) o[q] = pack_bf16_exact(v[2 * q] * s, v[2 * q + 1] * s);
    return o;
}

typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));

// Expand 8 codes (one dword) with block scale s (as an f16 pair (s, s)) into 8 exact f16 values.
__device__ __forceinline__ u32x4 expand8_f16(uint32_t w, f16x2 s2) {
    u32x4 o;
    o[0] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 0) * s2);
    o[1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 1) * s2);
    o[2] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 2) * s2);
    o[3] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 3) * s2);
    return o;
}

// Activation operand of the tiled kernels.
constexpr int kAmBf16 = 0;   // bf16 rows (W4A16)
constexpr int kAmNvfp4 = 1;  // NVFP4 tensor (W4A4)
constexpr int kAmFp8 = 2;    // E4M3 bytes with one tensor scale (FP8 activations)
constexpr int kAmQuant = 3;  // bf16 rows quantized to NVFP4 in the kernel with a static amax (W4A4)

// Quantize one unit of 8 bf16 activations to NVFP4 with the static global scale g (six_g =
// fl(6 g)): returns the unit's 8 codes (element i in nibble i) and its block's scale byte.  The
// unit's 16-element block is completed by the neighbouring lane (lane ^ 1), which holds the other
// 8 elements: the block amax is exchanged with one DPP move.  The steps and roundings are those of
// the quantize kernel (block scale byte = nearest E4M3 of fl(bamax / six_g), r = fl(1 / fl(s g)),
// code = nearest E2M1 of fl(v r), zero kept at zero), so the codes are what nvfp4_quantize with
// this amax stores.
__device__ __forceinline__ uint32_t quant8_codes(u32x4 raw, float g, float six_g, uint32_t &sbyte) {
    float v[8];
    uint32_t bm = 0;
#pragma unroll
    for (int i = 0; i < 4; i++) {
        v[2 * i] = u2f(raw[i] << 16);
        v[2 * i + 1] = u2f(raw[i] & 0xFFFF0000u);
        const uint32_t m0 = (raw[i] << 16) & 0x7FFFFFFFu, m1 = raw[i] & 0x7FFF0000u;
        bm = bm > m0 ? bm : m0;
        bm = bm > m1 ? bm : m1;
    }
    const uint32_t bo = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)bm, 0xB1, 0xF, 0xF, false);  // lane ^ 1
    bm = bm > bo ? bm : bo;
    const float q = u2f(bm) / six_g;
    sbyte = g != 0.0f ? e4m3_from_f32(q) : 0u;
    const float s = e4m3_to_f32(sbyte);
    const float rd = 1.0f / (s * g);
    const float r = s == 0.0f ? 0.0f : rd;
    float y[8];
#pragma unroll
    for (int e = 0; e < 8; e++) y[e] = v[e] == 0.0f ? v[e] : v[e] * r;
    return fp4_pack8(y);
}

// The same unit quantized and returned as its 8 exact values e2m1 x s in f16.
__device__ __forceinline__ u32x4 quant8_f16(u32x4 raw, float g, float six_g) {
    uint32_t sbyte;
    const uint32_t codes = quant8_codes(raw, g, six_g, sbyte);
    const _Float16 sh = (_Float16)e4m3_to_f32(sbyte);
    return expand8_f16(codes, f16x2{sh, sh});
}

// Quantize one 16-element block of bf16 activations (lo: elements 0..7, hi: 8..15) in one lane,
// with the steps and roundings of quant8_codes: returns the 16 codes (element i in nibble i) and
// the block scale byte.
__device__ __forceinline__ uint64_t quant16_codes(u32x4 lo, u32x4 hi, float g, float six_g, uint32_t &sbyte) {
    float v[16];
    uint32_t bm = 0;
#pragma unroll
    for (int i = 0; i < 8; i++) {
        const uint32_t w = i < 4 ? lo[i] : hi[i - 4];
        v[2 * i] = u2f(w << 16);
        v[2 * i + 1] = u2f(w & 0xFFFF0000u);
        const uint32_t m0 = (w << 16) & 0x7FFFFFFFu, m1 = w & 0x7FFF0000u;
        bm = bm > m0 ? bm : m0;
        bm = bm > m1 ? bm : m1;
    }
    const float q = u2f(bm) / six_g;
    sbyte = g != 0.0f ? e4m3_from_f32(q) : 0u;
    const float s = e4m3_to_f32(sbyte);
    const float rd = 1.0f / (s * g);
    const float r = s == 0.0f ? 0.0f : rd;
    float y[16];
#pragma unroll
    for (int e = 0; e < 16; e++) y[e] = v[e] == 0.0f ? v[e] : v[e] * r;
    return (uint64_t)fp4_pack8(y) | ((uint64_t)fp4_pack8(y + 8) << 32);
}


// Activations quantized once inside the W4A4 product (the staged form of nvfp4_gemm_qa): the bf16
// rows, the static amax, the workspace arrays the NVFP4 activations go to (those the product then
// reads as its A operand) and the group counters.
struct QaPre {
    const __bf16 *x;
    int64_t ldx;
    const float *amax;
    uint32_t *sync;  // arrival counters [kQaMaxGroups], then departure counters [kQaMaxGroups]
    uint8_t *codes;  // [M][K / 2]
    uint8_t *scales; // [M][K / 16]
    uint32_t spin_limit;  // polls of the group counter before a member quantizes its whole region itself
};

// Staged quantization of one workgroup's A region.  The members of a group (the workgroups of one
// A row block and K slice, one per N tile) each quantize a share of the group's 16-element blocks
// into the workspace, publish it and wait until every member has: then all of the region is
// there.  Publication: the codes and scale bytes are written with agent-coherent (sc1) stores,
// which do not stay dirty in one XCD's L2, so no writeback of the L2 is needed; every wave waits
// for its stores to complete, then one thread adds 1 to the group's arrival counter; a waiting
// member polls the counter and then acquires at agent scope.  The last member to leave resets the counters to zero,
// so a zeroed counter area stays zeroed from one call to the next.  A member whose wait runs out
// (the group not co-resident for a very long time) quantizes the whole region itself: the values
// are the same, so correctness never depends on the wait.
template <int NT>
__device__ __forceinline__ void qa_stage(const QaPre &pre, int64_t K, int64_t m0, int64_t mrows, int kblk0, int nblk_row, int group,
                         int members, int member, bool publish) {
    __shared__ int timed_out;
    const float g = *pre.amax / 2688.0f;
    const float six_g = 6.0f * g;
    // work unit: four consecutive blocks of a row (64 elements; nblk_row is a multiple of 4)
    const int nq_row = nblk_row / 4;
    const int64_t nq = mrows * nq_row;
    constexpr int kBatch = 4;  // units per thread whose loads are issued before the first is used
    // agent-coherent (sc1) 16-byte stores through buffer resources over the region's rows
    const __amdgpu_buffer_rsrc_t rcode = lr_rsrc(pre.codes + m0 * (K / 2), mrows * (K / 2));
    const __amdgpu_buffer_rsrc_t rscale = lr_rsrc(pre.scales + m0 * (K / 16), mrows * (K / 16));
    constexpr int kSc1 = 16;  // cache policy bit of an agent-coherent store
    auto quantize_units = [&](int64_t q0, int64_t q1) {
        for (int64_t base = q0 + threadIdx.x; base < q1; base += (int64_t)kBatch * NT) {
            u32x4 raw[kBatch][8];
#pragma unroll
            for (int j = 0; j < kBatch; j++) {
                const int64_t q = base + (int64_t)j * NT;
                if (q < q1) {
                    const int64_t r = m0 + q / nq_row, kb = kblk0 + (q % nq_row) * 4;
                    const u32x4 *src = reinterpret_cast<const u32x4 *>(pre.x + r * pre.ldx + kb * 16);
#pragma unroll
                    for (int h = 0; h < 8; h++) raw[j][h] = src[h];
                }
            }
#pragma unroll
            for (int j = 0; j < kBatch; j++) {
                const int64_t q = base + (int64_t)j * NT;
                if (q < q1) {
                    const int64_t rr = q / nq_row, kb = kblk0 + (q % nq_row) * 4;  // row within the region
                    uint64_t cw[4];
                    uint32_t sw = 0;
#pragma unroll
                    for (int t = 0; t < 4; t++) {
                        uint32_t sb;
                        cw[t] = quant16_codes(raw[j][2 * t], raw[j][2 * t + 1], g, six_g, sb);
                        sw |= sb << (8 * t);
                    }
                    const uint32_t co = (uint32_t)(rr * (K / 2) + kb * 8);
                    __builtin_amdgcn_raw_buffer_store_b128(
                        u32x4{(uint32_t)cw[0], (uint32_t)(cw[0] >> 32), (uint32_t)cw[1], (uint32_t)(cw[1] >> 32)}, rcode,
                        co, 0, kSc1);
                    __builtin_amdgcn_raw_buffer_store_b128(
                        u32x4{(uint32_t)cw[2], (uint32_t)(cw[2] >> 32), (uint32_t)cw[3], (uint32_t)(cw[3] >> 32)}, rcode,
                        co + 16, 0, kSc1);
                    __builtin_amdgcn_raw_buffer_store_b32(sw, rscale, (uint32_t)(rr * (K / 16) + kb), 0, kSc1);
                }
            }
        }
        __builtin_amdgcn_s_waitcnt(waitcnt_imm(0, 15));  // this wave's stores are complete
    };
    uint32_t *arrive = pre.sync + group, *depart = pre.sync + kQaMaxGroups + group;
    if (publish) {  // first phase: this member's share, then its arrival
        quantize_units(nq * member / members, nq * (member + 1) / members);
        __syncthreads();
        if (threadIdx.x == 0) __hip_atomic_fetch_add(arrive, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        return;
    }
    // second phase: wait for the group, then leave
    if (threadIdx.x == 0) {
        uint32_t polls = 0;
        while (__hip_atomic_load(arrive, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) < (uint32_t)members &&
               polls < pre.spin_limit) {
            polls++;
            __builtin_amdgcn_s_sleep(1);
        }
        timed_out = __hip_atomic_load(arrive, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) < (uint32_t)members;
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
    }
    __syncthreads();
    if (timed_out) {
        quantize_units(0, nq);
        __syncthreads();
        if (threadIdx.x == 0) __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
        __syncthreads();
    }
    if (threadIdx.x == 0) {
        if (__hip_atomic_fetch_add(depart, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == (uint32_t)members - 1) {
            __hip_atomic_store(arrive, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            __hip_atomic_store(depart, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
    }
}

// Expand 8 E4M3 bytes (two dwords, element i in byte i) into 8 exact f16 values: e4m3 values have
// at most 4 significant bits and lie in [2^-9, 448], inside f16's range.
__device__ __forceinline__ u32x4 expand8_fp8_f16(u32x2 b) {
    u32x4 o;
    o[0] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(b[0], 1.0f, false));
    o[1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(b[0], 1.0f, true));
    o[2] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(b[1], 1.0f, false));
    o[3] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(b[1], 1.0f, true));
    return o;
}

// The same 8 E4M3 values as exact bf16 (the high halves of their exact fp32 values).
__device__ __forceinline__ u32x4 expand8_fp8_bf16(u32x2 b) {
    const f32x2 f0 = __builtin_amdgcn_cvt_pk_f32_fp8(b[0], false), f1 = __builtin_amdgcn_cvt_pk_f32_fp8(b[0], true);
    const f32x2 f2 = __builtin_amdgcn_cvt_pk_f32_fp8(b[1], false), f3 = __builtin_amdgcn_cvt_pk_f32_fp8(b[1], true);
    return u32x4{pack_bf16_exact(f0[0], f0[1]), pack_bf16_exact(f1[0], f1[1]), pack_bf16_exact(f2[0], f2[1]),
                 pack_bf16_exact(f3[0], f3[1])};
}

// Raw global data of one 32-element NVFP4 chunk (two blocks): 16 code bytes and 2 scale bytes.
struct QChunk {
    u32x4 codes;
    uint32_t sc;  // scale byte of block 0 in bits 0..7, block 1 in bits 8..15
};

// Load chunk (row, k0..k0+31) of an NVFP4 operand with `rows` rows and K columns (K % 16 == 0).
// Missing rows and columns read as zero.
__device__ __forceinline__ QChunk load_qchunk(const uint8_t *__restrict__ codes, const uint8_t *__restrict__ scales,
                                              int64_t row, int64_t rows, int64_t K, int64_t k0) {
    QChunk c;
    c.codes = u32x4{0u, 0u, 0u, 0u};
    c.sc = 0u;
    if (row >= rows) return c;
    const uint8_t *crow = codes + row * (K / 2);
    const uint8_t *srow = scales + row * (K / 16);
    if (k0 + 16 <= K) {
        u32x2 lo = *reinterpret_cast<const u32x2 *>(crow + k0 / 2);
        c.codes[0] = lo[0];
        c.codes[1] = lo[1];
        c.sc = srow[k0 / 16];
    }
    if (k0 + 32 <= K) {
        u32x2 hi = *reinterpret_cast<const u32x2 *>(crow + k0 / 2 + 8);
        c.codes[2] = hi[0];
        c.codes[3] = hi[1];
        c.sc |= (uint32_t)srow[k0 / 16 + 1] << 8;
    }
    return c;
}

// A buffer resource over [base, base + bytes): loads at offsets at or past `bytes` return zero
// instead of touching memory, which keeps the main-loop loads free of branches at tile edges.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void *base, int64_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0, (int)bytes, 0x00020000);
}

// Tile id -> (m-tile, n-tile).  The hardware hands workgroup i to XCD i % 8; ids are first remapped
// so that each XCD receives a contiguous run of tile ids, and that run is walked in groups of GM
// m-tiles, so the tiles one XCD works on at a time share a few A row blocks and W column blocks in
// its L2.
__device__ __forceinline__ void tile_coords(int id, int tiles_m, int tiles_n, int &tm, int &tn) {
    const int ntiles = tiles_m * tiles_n;
    const int per_xcd = ntiles / 8;
    if (per_xcd > 0 && id < per_xcd * 8) id = (id % 8) * per_xcd + id / 8;
    const int GM = tiles_m < 4 ? tiles_m : 4;
    const int group = id / (GM * tiles_n);
    const int first_m = group * GM;
    const int gm = (tiles_m - first_m) < GM ? (tiles_m - first_m) : GM;
    const int r = id - group * GM * tiles_n;
    tm = first_m + r % gm;
    tn = r / gm;
}

// The tiles of tile_coords, each XCD's set of tiles started row block by row block: where the
// tiles an XCD takes form a rectangle of GM row blocks x C N tiles, its i-th workgroup takes row
// block i / C, N tile i % C of it, so that the workgroups of one row block start one after another
// (the staged quantization waits for all of them); otherwise the order of tile_coords.
__device__ __forceinline__ void tile_coords_grouped(int lin, int tiles_m, int tiles_n, int &tm, int &tn) {
    const int ntiles = tiles_m * tiles_n;
    const int per_xcd = ntiles / 8;
    constexpr int GM = 4;
    if (per_xcd > 0 && lin < per_xcd * 8 && tiles_m % GM == 0 && per_xcd % GM == 0 && (GM * tiles_n) % per_xcd == 0) {
        const int x = lin % 8, pos = lin / 8;
        const int id0 = x * per_xcd;  // first id of this XCD's range
        const int group = id0 / (GM * tiles_n), r0 = id0 % (GM * tiles_n);
        const int cols = per_xcd / GM;
        tm = group * GM + pos / cols;
        tn = r0 / GM + pos % cols;
        return;
    }
    tile_coords(lin, tiles_m, tiles_n, tm, tn);
}

template <int BM, int BN, int WM, int WN, int AM>
__global__ __launch_bounds__(64 * WM *WN) void k_gemm_tile(const __bf16 *__restrict__ A, int64_t lda,
                                                          const uint8_t *__restrict__ a_codes,
                                                          const uint8_t *__restrict__ a_scales,
                                                          const float *__restrict__ a_g,
                                                          const uint8_t *__restrict__ w_codes,
                                                          const uint8_t *__restrict__ w_scales,
                                                          const float *__restrict__ w_g, float *__restrict__ C,
                                                          int64_t ldc, int64_t M, int64_t N, int64_t K) {
    constexpr bool A_Q = AM == kAmNvfp4, A_F8 = AM == kAmFp8;
    constexpr int NT = 64 * WM * WN;
    constexpr int WTM = BM / WM, WTN = BN / WN;   // wave tile
    constexpr int TM = WTM / 32, TN = WTN / 32;   // 32x32 MFMA tiles per wave
    constexpr int A_BF_PASSES = BM * (kBK / 8) / NT;   // 16-byte bf16 chunks of A per thread
    constexpr int A_Q_PASSES = (BM * 2 + NT - 1) / NT;  // 32-element NVFP4 chunks of A per thread
    constexpr int W_PASSES = (BN * 2 + NT - 1) / NT;
    constexpr int STAGE = (BM + BN) * kLdsRow;          // bf16 elements per LDS stage
    static_assert(BM * (kBK / 8) % NT == 0, "A tile must split evenly over the threads");
    static_assert(WTM % 32 == 0 && WTN % 32 == 0, "wave tile must be a multiple of 32x32");

    // two stages of [A tile | W tile], rows padded to 72 bf16 (144 bytes)
    __shared__ __attribute__((aligned(16))) __bf16 smem[2 * STAGE];

    const int tiles_m = (int)((M + BM - 1) / BM);
    const int tiles_n = (int)((N + BN - 1) / BN);
    int tm_idx, tn_idx;
    tile_coords(blockIdx.x, tiles_m, tiles_n, tm_idx, tn_idx);
    const int64_t m0 = (int64_t)tm_idx * BM;
    const int64_t n0 = (int64_t)tn_idx * BN;

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wid = tid >> 6;
    const int wm = wid / WN, wn = wid % WN;

    // ---- register staging of one K step (two sets: loads run two steps ahead) ----
    struct Staging {
        u32x4 a[AM == kAmBf16 ? A_BF_PASSES : 1];  // 8 bf16 values per pass
        u32x2 a8[A_F8 ? A_BF_PASSES : 1];          // 8 E4M3 bytes per pass
        QChunk aq[A_Q ? A_Q_PASSES : 1];
        QChunk w[W_PASSES];
    };
    Staging st0, st1;

    auto load_step = [&](int64_t k0, Staging &st) {
        if constexpr (AM == kAmBf16) {
#pragma unroll
            for (int p = 0; p < A_BF_PASSES; p++) {
                const int idx = p * NT + tid;
                const int r = idx / (kBK / 8), c8 = idx % (kBK / 8);
                const int64_t gr = m0 + r, gk = k0 + c8 * 8;
                if (gr < M && gk < K) {
                    st.a[p] = *reinterpret_cast<const u32x4 *>(A + gr * lda + gk);
                } else {
                    st.a[p] = u32x4{0u, 0u, 0u, 0u};
                }
            }
        } else if constexpr (A_F8) {
#pragma unroll
            for (int p = 0; p < A_BF_PASSES; p++) {
                const int idx = p * NT + tid;
                const int r = idx / (kBK / 8), c8 = idx % (kBK / 8);
                const int64_t gr = m0 + r, gk = k0 + c8 * 8;
                if (gr < M && gk < K) {
                    st.a8[p] = *reinterpret_cast<const u32x2 *>(a_codes + gr * lda + gk);
                } else {
                    st.a8[p] = u32x2{0u, 0u};
                }
            }
        } else {
#pragma unroll
            for (int p = 0; p < A_Q_PASSES; p++) {
                const int idx = p * NT + tid;
                if (idx < BM * 2) {
                    st.aq[p] = load_qchunk(a_codes, a_scales, m0 + idx / 2, M, K, k0 + (idx % 2) * 32);
                }
            }
        }
#pragma unroll
        for (int p = 0; p < W_PASSES; p++) {
            const int idx = p * NT + tid;
            if (idx < BN * 2) {
                st.w[p] = load_qchunk(w_codes, w_scales, n0 + idx / 2, N, K, k0 + (idx % 2) * 32);
            }
        }
    };

    // Writing one K step into LDS is split into units, each one 16-byte LDS store: a copy of 8 bf16
    // A values, or the exact bf16 expansion of 8 NVFP4 codes (one code dword).  The units are spread
    // over the four 16-deep MFMA slices of the previous step, so that the expansion arithmetic of
    // step ks + 1 issues between the matrix instructions of step ks.
    constexpr int A_UNITS = A_Q ? A_Q_PASSES * 4 : A_BF_PASSES;
    constexpr int W_UNITS = W_PASSES * 4;
    constexpr int UNITS = A_UNITS + W_UNITS;
    float a_s[A_Q ? A_Q_PASSES * 2 : 1], w_s[W_PASSES * 2];
    auto decode_scales = [&](const Staging &st) {
        if constexpr (A_Q) {
#pragma unroll
            for (int p = 0; p < A_Q_PASSES; p++) {
                a_s[2 * p] = e4m3_to_f32(st.aq[p].sc & 0xFFu);
                a_s[2 * p + 1] = e4m3_to_f32((st.aq[p].sc >> 8) & 0xFFu);
            }
        }
#pragma unroll
        for (int p = 0; p < W_PASSES; p++) {
            w_s[2 * p] = e4m3_to_f32(st.w[p].sc & 0xFFu);
            w_s[2 * p + 1] = e4m3_to_f32((st.w[p].sc >> 8) & 0xFFu);
        }
    };
    auto store_unit = [&](int u, __bf16 *As, __bf16 *Bs, const Staging &st) {
        if (u < A_UNITS) {
            if constexpr (AM == kAmBf16) {
                const int idx = u * NT + tid;
                const int r = idx / (kBK / 8), c8 = idx % (kBK / 8);
                *reinterpret_cast<u32x4 *>(&As[r * kLdsRow + c8 * 8]) = st.a[u];
            } else if constexpr (A_F8) {
                const int idx = u * NT + tid;
                const int r = idx / (kBK / 8), c8 = idx % (kBK / 8);
                *reinterpret_cast<u32x4 *>(&As[r * kLdsRow + c8 * 8]) = expand8_fp8_bf16(st.a8[u]);
            } else {
                const int p = u / 4, q = u % 4;
                const int idx = p * NT + tid;
                if (BM * 2 % NT == 0 || idx < BM * 2)
                    *reinterpret_cast<u32x4 *>(&As[(idx / 2) * kLdsRow + (idx % 2) * 32 + q * 8]) =
                        expand8(st.aq[p].codes[q], a_s[2 * p + q / 2]);
            }
        } else {
            const int p = (u - A_UNITS) / 4, q = (u - A_UNITS) % 4;
            const int idx = p * NT + tid;
            if (BN * 2 % NT == 0 || idx < BN * 2)
                *reinterpret_cast<u32x4 *>(&Bs[(idx / 2) * kLdsRow + (idx % 2) * 32 + q * 8]) =
                    expand8(st.w[p].codes[q], w_s[2 * p + q / 2]);
        }
    };
    auto store_step = [&](int stage, const Staging &st) {
        __bf16 *As = smem + stage * STAGE;
        __bf16 *Bs = As + BM * kLdsRow;
        decode_scales(st);
#pragma unroll
        for (int u = 0; u < UNITS; u++) store_unit(u, As, Bs, st);
    };

    f32x16 acc[TM][TN];
#pragma unroll
    for (int i = 0; i < TM; i++)
#pragma unroll
        for (int j = 0; j < TN; j++)
#pragma unroll
            for (int e = 0; e < 16; e++) acc[i][j][e] = 0.0f;

    // Matrix work of one step from LDS stage `stage`, with the LDS writes of the next step (into
    // stage `nstage`, from registers `nxt`) interleaved.
    auto compute = [&](int stage, int nstage, const Staging &nxt) {
        const __bf16 *As = smem + stage * STAGE;
        const __bf16 *Bs = As + BM * kLdsRow;
        __bf16 *nAs = smem + nstage * STAGE;
        __bf16 *nBs = nAs + BM * kLdsRow;
#pragma unroll
        for (int kk = 0; kk < kBK / 16; kk++) {
            const int kc = kk * 16 + 8 * (lane / 32);
            bf16x8 af[TM], bfr[TN];
#pragma unroll
            for (int i = 0; i < TM; i++)
                af[i] = *reinterpret_cast<const bf16x8 *>(&As[(wm * WTM + i * 32 + (lane % 32)) * kLdsRow + kc]);
#pragma unroll
            for (int j = 0; j < TN; j++)
                bfr[j] = *reinterpret_cast<const bf16x8 *>(&Bs[(wn * WTN + j * 32 + (lane % 32)) * kLdsRow + kc]);
#pragma unroll
            for (int i = 0; i < TM; i++)
#pragma unroll
                for (int j = 0; j < TN; j++)
                    acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[i], bfr[j], acc[i][j], 0, 0, 0);
            if (kk == 0) decode_scales(nxt);
#pragma unroll
            for (int u = 0; u < UNITS; u++)
                if (u * (kBK / 16) / UNITS == kk) store_unit(u, nAs, nBs, nxt);
        }
    };

    // Step ks computes from LDS stage ks & 1.  While it runs, the registers hold the global data of
    // step ks + 1 (issued one step earlier) and the loads of step ks + 2 are issued; the expansion
    // of step ks + 1 into the other stage (last read before the previous barrier) is interleaved
    // with the matrix work, and one barrier ends the step.  Loads past the last step repeat the
    // last step (harmless) so that the loop body has no data-dependent branches.
    const int nsteps = (int)((K + kBK - 1) / kBK);
    const int last = nsteps - 1;
    auto kstep = [&](int s) -> int64_t { return (int64_t)(s < last ? s : last) * kBK; };
    load_step(0, st0);
    load_step(kstep(1), st1);
    store_step(0, st0);
    __syncthreads();
    int ks = 0;
    for (; ks + 2 <= nsteps; ks += 2) {
        load_step(kstep(ks + 2), st0);
        compute(0, 1, st1);
        __syncthreads();
        load_step(kstep(ks + 3), st1);
        compute(1, 0, st0);
        __syncthreads();
    }
    if (ks < nsteps) compute(0, 1, st1);

    // ---- epilogue: multiply by the global scale(s), store fp32 ----
    const float gw = *w_g;
    const float ga = AM != kAmBf16 ? *a_g : 1.0f;
#pragma unroll
    for (int i = 0; i < TM; i++) {
#pragma unroll
        for (int j = 0; j < TN; j++) {
            const int64_t col = n0 + wn * WTN + j * 32 + (lane % 32);
#pragma unroll
            for (int e = 0; e < 16; e++) {
                const int64_t row = m0 + wm * WTM + i * 32 + 8 * (e / 4) + 4 * (lane / 32) + (e % 4);
                if (row < M && col < N) {
                    float v = acc[i][j][e];
                    if (AM != kAmBf16) v = v * ga;
                    C[row * ldc + col] = v * gw;
                }
            }
        }
    }
}

// ------------------------------------------------------------------------------------------------
// k_gemm_mfma: K % 64 == 0
// ------------------------------------------------------------------------------------------------
template <int V>
struct StepIdx {
    static constexpr int value = V;
};



template <int BM, int BN, int WM, int WN, int AM, bool LR = false, bool PRE = false>
__global__ __launch_bounds__(64 * WM *WN) void k_gemm_mfma(const __bf16 *__restrict__ A, int64_t lda,
                                                          const uint8_t *__restrict__ a_codes,
                                                          const uint8_t *__restrict__ a_scales,
                                                          const float *__restrict__ a_g,
                                                          const uint8_t *__restrict__ w_codes,
                                                          const uint8_t *__restrict__ w_scales,
                                                          const float *__restrict__ w_g, float *__restrict__ C,
                                                          int64_t ldc, int64_t M, int64_t N, int64_t K,
                                                          int slice_steps, LrArgs lr, QaPre pre) {
    // A_X: activations expanded from registers into LDS as f16 (NVFP4 codes, or E4M3 bytes), with W
    // expanded to f16 too; otherwise bf16 activations are copied straight into LDS.  PRE (NVFP4
    // activations only): the workgroup first takes part in quantizing its A region into the arrays
    // the NVFP4 operand points to (qa_stage), and *a_g is then the static amax.
    constexpr bool A_Q = AM == kAmNvfp4, A_F8 = AM == kAmFp8, A_QS = AM == kAmQuant, A_X = AM != kAmBf16;
    constexpr int NT = 64 * WM * WN;
    constexpr int WTM = BM / WM, WTN = BN / WN;    // wave tile
    constexpr int TM = WTM / 32, TN = WTN / 32;    // 32x32 MFMA tiles per wave
    constexpr int ROWB = kBK * 2;                  // LDS row: 64 16-bit values, no padding
    constexpr int A_STAGE = BM * ROWB, W_STAGE = BN * ROWB;
    constexpr int NA = A_X ? 2 : 3;                // A stages (three for the two-step-ahead DMA)
    constexpr int W_OFF = NA * A_STAGE;
    constexpr int LDS_BYTES = W_OFF + 2 * W_STAGE;
    constexpr int WD = BN * 8 / NT;                // W code dwords per thread per step
    constexpr int AD = A_X ? BM * 8 / NT : 0;      // A units (8 elements each) per thread per step
    constexpr int QD = AD + WD;                    // expansion units per thread per step
    constexpr int A_DMA = A_X ? 0 : BM / 8 / (WM * WN);  // 1 KiB direct-to-LDS loads per wave per step
    // vector-memory instructions issued per step: an NVFP4 unit loads a code dword and a scale byte,
    // an E4M3 unit one 8-byte load
    constexpr int VM_STEP = A_DMA + 2 * WD + (A_F8 || A_QS ? AD : 2 * AD);
    static_assert(LDS_BYTES <= 160 * 1024, "LDS budget");
    static_assert(BN * 8 % NT == 0 && BM * 8 % NT == 0 && (A_X || BM / 8 % (WM * WN) == 0), "even split");
    static_assert(WTM % 32 == 0 && WTN % 32 == 0, "wave tile must be a multiple of 32x32");
    static_assert(VM_STEP < 64, "vmcnt range");
    __shared__ __attribute__((aligned(1024))) uint8_t smem[LDS_BYTES];

    const int tiles_m = (int)((M + BM - 1) / BM);
    const int tiles_n = (int)((N + BN - 1) / BN);
    int tm_idx, tn_idx;
    const int slice = (int)blockIdx.y;
    if constexpr (PRE)
        tile_coords_grouped(blockIdx.x, tiles_m, tiles_n, tm_idx, tn_idx);
    else
        tile_coords(blockIdx.x, tiles_m, tiles_n, tm_idx, tn_idx);
    const int64_t m0 = (int64_t)tm_idx * BM;
    const int64_t n0 = (int64_t)tn_idx * BN;

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wid = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wid / WN, wn = wid % WN;

    // Buffer resources start at the tile's first row; rows past M or N fall outside them and read
    // as zero, so no load needs a bounds check (those rows only feed outputs that are not stored).
    const int64_t mrows = (M - m0) < BM ? (M - m0) : BM;
    const int64_t nrows = (N - n0) < BN ? (N - n0) : BN;
    __amdgpu_buffer_rsrc_t ra = make_rsrc(A, 0);
    __amdgpu_buffer_rsrc_t rc[2], rs[2];  // NVFP4 codes / scales: [0] A (W4A4), [1] W
    rc[0] = rs[0] = make_rsrc(a_codes, 0);
    if constexpr (AM == kAmBf16) {
        ra = make_rsrc(A + m0 * lda, ((mrows - 1) * lda + K) * 2);
    } else if constexpr (A_Q) {
        rc[0] = make_rsrc(a_codes + m0 * (K / 2), mrows * (K / 2));
        rs[0] = make_rsrc(a_scales + m0 * (K / 16), mrows * (K / 16));
    } else if constexpr (A_QS) {
        rc[0] = make_rsrc(A + m0 * lda, ((mrows - 1) * lda + K) * 2);  // bf16 rows, quantized here
    } else {
        rc[0] = make_rsrc(a_codes + m0 * lda, (mrows - 1) * lda + K);  // E4M3 bytes, row stride lda
    }
    rc[1] = make_rsrc(w_codes + n0 * (K / 2), nrows * (K / 2));
    rs[1] = make_rsrc(w_scales + n0 * (K / 16), nrows * (K / 16));

    // LDS rows are 128 bytes (64 16-bit values) and hold their eight 16-byte chunks at chunk index
    // chunk ^ ((row / 2) % 8).  The LDS serves a 16-byte-per-lane access sixteen lanes at a time
    // across its 64 banks (256 bytes); a fragment read has those lanes on 16 consecutive rows at one
    // logical chunk, and this swizzle puts them on 16 distinct 16-byte bank groups (rows of either
    // parity fill one half of the banks; row / 2 spreads the eight of each parity over that half).
    // Expansion unit u of this thread: 8-element chunk d = tid + NT * j of the step's tile (row d / 8,
    // chunk d % 8: one NVFP4 code dword, or 8 E4M3 bytes), j = u for A (u < AD), u - AD for W.
    uint32_t q_coff[QD], q_soff[QD], q_lds[QD];
#pragma unroll
    for (int u = 0; u < QD; u++) {
        const int j = u < AD ? u : u - AD;
        const uint32_t d = (uint32_t)(tid + NT * j), row = d >> 3, c = d & 7;
        q_coff[u] = (A_F8 && u < AD)    ? row * (uint32_t)lda + c * 8
                    : (A_QS && u < AD) ? (row * (uint32_t)lda + c * 8) * 2
                                       : row * (uint32_t)(K / 2) + c * 4;
        q_soff[u] = row * (uint32_t)(K / 16) + (c >> 1);
        q_lds[u] = (u < AD ? 0u : (uint32_t)W_OFF) + row * ROWB + ((c ^ ((row >> 1) & 7)) << 4);
    }
    // Direct-to-LDS load b of this wave fills the 1 KiB LDS block of tile rows (wid * A_DMA + b) * 8
    // .. + 7: lane l writes 16 bytes at l * 16, i.e. row l / 8, swizzled chunk l % 8, so it loads
    // logical chunk (l % 8) ^ ((row / 2) % 8) = (l % 8) ^ (l / 16) ^ (4 if the block is odd).
    static_assert(A_DMA % 2 == 0, "block parity of direct-to-LDS load b is that of b");
    uint32_t a_dma_off[2];
    {
        const uint32_t row = (uint32_t)(wid * A_DMA) * 8 + (uint32_t)(lane >> 3);
        const uint32_t c = (uint32_t)((lane & 7) ^ (lane >> 4));
        a_dma_off[0] = row * (uint32_t)lda * 2 + c * 16;
        a_dma_off[1] = row * (uint32_t)lda * 2 + (c ^ 4u) * 16;
    }
    // Fragment reads: 32x32x16 operands take row (lane % 32), k = 16 kk + 8 (lane / 32) .. + 7; the
    // fragment rows start at multiples of 32, so the swizzle of row lane % 32 is (lane / 2) % 8.
    uint32_t offA[4], offB[4];
#pragma unroll
    for (int kk = 0; kk < 4; kk++) {
        const uint32_t ch = ((uint32_t)(2 * kk + (lane >> 5)) ^ (uint32_t)((lane >> 1) & 7)) << 4;
        offA[kk] = (uint32_t)(wm * WTM + (lane & 31)) * ROWB + ch;
        offB[kk] = (uint32_t)W_OFF + (uint32_t)(wn * WTN + (lane & 31)) * ROWB + ch;
    }

    uint32_t qc[2][QD], qs[2][QD];  // two register sets of code dwords and scale bytes
    u32x2 qa8[2][A_F8 ? AD : 1];     // E4M3 activations: two register sets of 8-byte chunks
    u32x4 qa16[2][A_QS ? AD : 1];    // bf16 activations to quantize: two register sets of 16 bytes
    // static amax -> global scale of the quantized activations (as the quantize kernel forms it)
    static_assert(!PRE || (A_Q && !LR), "staged quantization feeds the NVFP4-activation product");
    const float qs_g = (A_QS || PRE) ? *a_g / 2688.0f : 0.0f;
    const float qs_six_g = 6.0f * qs_g;

    // K slice of this workgroup (split-K: `slice`; otherwise the whole of K)
    const int total_steps = (int)(K / kBK);
    const int kbase = slice * slice_steps;
    const int nsteps = (total_steps - kbase) < slice_steps ? (total_steps - kbase) : slice_steps;
    const int last = nsteps - 1;
    auto stage_a = [&](bool publish) {
        if constexpr (PRE)
            qa_stage<NT>(pre, K, m0, mrows, kbase * (kBK / 16), nsteps * (kBK / 16), slice * tiles_m + tm_idx,
                         tiles_n, tn_idx, publish);
    };
    // Loads past the last step repeat it: harmless, and the loop body stays free of branches.
    auto issue = [&](int s, int a_stage, int r, int u0 = 0, int u1 = 1 << 30) {
        const uint32_t k0 = (uint32_t)((kbase + (s < last ? s : last)) * kBK);
        if constexpr (!A_X) {
#pragma unroll
            for (int b = 0; b < A_DMA; b++)
                load_to_lds16(ra, smem + a_stage * A_STAGE + (wid * A_DMA + b) * 1024,
                              a_dma_off[b & 1] + (uint32_t)(b * 8) * (uint32_t)lda * 2, k0 * 2);
        }
#pragma unroll
        for (int u = 0; u < QD; u++) {
            if (u < u0 || u >= u1) continue;
            if (A_F8 && u < AD) {
                qa8[r][A_F8 ? u : 0] = __builtin_bit_cast(u32x2, __builtin_amdgcn_raw_buffer_load_b64(rc[0], q_coff[u], k0, 0));
                continue;
            }
            if (A_QS && u < AD) {
                qa16[r][A_QS ? u : 0] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rc[0], q_coff[u], k0 * 2, 0));
                continue;
            }
            const int o = u < AD ? 0 : 1;
            qc[r][u] = __builtin_amdgcn_raw_buffer_load_b32(rc[o], q_coff[u], k0 / 2, 0);
            qs[r][u] = __builtin_amdgcn_raw_buffer_load_b8(rs[o], q_soff[u], k0 / 16, 0);
        }
    };
    auto expand_unit = [&](int u, int r, int a_stage, int w_stage) {
        const uint32_t base = u < AD ? (uint32_t)(a_stage * A_STAGE) : (uint32_t)(w_stage * W_STAGE);
        if (A_F8 && u < AD) {
            *reinterpret_cast<u32x4 *>(smem + base + q_lds[u]) = expand8_fp8_f16(qa8[r][A_F8 ? u : 0]);
            return;
        }
        if (A_QS && u < AD) {
            *reinterpret_cast<u32x4 *>(smem + base + q_lds[u]) = quant8_f16(qa16[r][A_QS ? u : 0], qs_g, qs_six_g);
            return;
        }
        const float sc = __builtin_amdgcn_cvt_f32_fp8((int)qs[r][u], 0);
        u32x4 v;
        if constexpr (A_X) {
            const _Float16 sh = (_Float16)sc;
            v = expand8_f16(qc[r][u], f16x2{sh, sh});
        } else {
            v = expand8(qc[r][u], sc);
        }
        *reinterpret_cast<u32x4 *>(smem + base + q_lds[u]) = v;
    };
    // End of a step: this step's loads may still be in flight, everything older (the A tile of the
    // next step) has landed; LDS writes are done; then the workgroup barrier.
    auto end_step = [&]() {
        __builtin_amdgcn_sched_barrier(0);
        __builtin_amdgcn_s_waitcnt(waitcnt_imm(VM_STEP, 0));
        __builtin_amdgcn_s_barrier();
        __builtin_amdgcn_sched_barrier(0);
    };

    f32x16 acc[TM][TN];
#pragma unroll
    for (int i = 0; i < TM; i++)
#pragma unroll
        for (int j = 0; j < TN; j++)
#pragma unroll
            for (int e = 0; e < 16; e++) acc[i][j][e] = 0.0f;

    typedef typename std::conditional<A_X, f16x8, bf16x8>::type frag_t;
    auto mfma = [&](const frag_t &a, const frag_t &b, f32x16 &c) {
        if constexpr (A_X) c = __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
        else c = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
    };
    // Register-resident slices: all four 16-deep fragment slices of a step in registers, when they
    // fit beside the accumulators (wave tiles up to 64 x 96).
    constexpr bool RESIDENT = TM * TN <= 6;
    frag_t af[RESIDENT ? 4 : 2][TM], bfr[RESIDENT ? 4 : 2][TN];
    auto read_frags = [&](int slot, int kk, int sa, int sw) {
#pragma unroll
        for (int i = 0; i < TM; i++)
            af[slot][i] = *reinterpret_cast<const frag_t *>(smem + sa * A_STAGE + offA[kk] + i * 32 * ROWB);
#pragma unroll
        for (int j = 0; j < TN; j++)
            bfr[slot][j] = *reinterpret_cast<const frag_t *>(smem + sw * W_STAGE + offB[kk] + j * 32 * ROWB);
    };
    auto mfmas = [&](int slot) {
#pragma unroll
        for (int i = 0; i < TM; i++)
#pragma unroll
            for (int j = 0; j < TN; j++) mfma(af[slot][i], bfr[slot][j], acc[i][j]);
    };

    // prologue: steps 0 and 1 in flight, step 0 expanded (and, register-resident, slices 0 and 1
    // of step 0 read)
    if constexpr (PRE) {
        // the W tiles of steps 0 and 1 load while this workgroup quantizes its share of A, and
        // step 0's is expanded before the wait for the rest of the group
        issue(0, 0, 0, AD, QD);
        issue(1, 1, 1, AD, QD);
        stage_a(true);
#pragma unroll
        for (int u = AD; u < QD; u++) expand_unit(u, 0, 0, 0);
        stage_a(false);
        issue(0, 0, 0, 0, AD);
        issue(1, 1, 1, 0, AD);
#pragma unroll
        for (int u = 0; u < AD; u++) expand_unit(u, 0, 0, 0);
    } else {
        issue(0, 0, 0);
        issue(1, 1, 1);
#pragma unroll
        for (int u = 0; u < QD; u++) expand_unit(u, 0, 0, 0);
    }
    end_step();
    if constexpr (RESIDENT) {
        read_frags(0, 0, 0, 0);
        read_frags(1, 1, 0, 0);
    }

    // Step s (S = s mod 6, so stage indices are constants).
    // Register-resident: issue the loads of step s + 2 and read slices 2 and 3 of step s; the
    // matrix work of slices 0 and 1 with the expansion of step s + 1 placed between the
    // instructions; the barrier (stage s + 1 complete); the matrix work of slices 2 and 3 with
    // slices 0 and 1 of step s + 1 read between the instructions.  Every fragment read is thus
    // issued at least six matrix instructions before its use, across the barrier too.
    // Otherwise: issue the loads of step s + 2, then the four slices of step s with double-buffered
    // fragments and the expansion of step s + 1 spread between them; the barrier ends the step.
    auto step = [&](auto Sc, int s) {
        constexpr int S = decltype(Sc)::value;
        constexpr int SA = A_X ? S % 2 : S % 3;
        constexpr int SW = S % 2;
        constexpr int SN = (S + 1) % 2;
        issue(s + 2, (S + 2) % 3, S % 2);
        if constexpr (RESIDENT) {
            constexpr int SAN = A_X ? (S + 1) % 2 : (S + 1) % 3;
            read_frags(2, 2, SA, SW);
            read_frags(3, 3, SA, SW);
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int kk = 0; kk < 2; kk++) {
                mfmas(kk);
#pragma unroll
                for (int u = 0; u < QD; u++)
                    if (u * 2 / QD == kk) expand_unit(u, SN, SN, SN);
                // matrix instructions with up to five VALU between them, then the LDS writes
#pragma unroll
                for (int q = 0; q < TM * TN - 1; q++) {
                    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
                    __builtin_amdgcn_sched_group_barrier(0x002, 5, 0);
                }
                __builtin_amdgcn_sched_group_barrier(0x200, (QD + 1) / 2, 0);
                __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
            }
            end_step();
#pragma unroll
            for (int kk = 2; kk < 4; kk++) {
                mfmas(kk);
                read_frags(kk - 2, kk - 2, SAN, SN);
                // one fragment read after each of the first matrix instructions
#pragma unroll
                for (int q = 0; q < TM + TN; q++) {
                    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
                    __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
                }
                __builtin_amdgcn_sched_group_barrier(0x008, TM * TN - TM - TN, 0);
            }
            __builtin_amdgcn_sched_barrier(0);
        } else {
            read_frags(0, 0, SA, SW);
#pragma unroll
            for (int kk = 0; kk < 4; kk++) {
                if (kk < 3) read_frags((kk + 1) & 1, kk + 1, SA, SW);
                mfmas(kk & 1);
#pragma unroll
                for (int u = 0; u < QD; u++)
                    if (u * 4 / QD == kk) expand_unit(u, SN, SN, SN);
                // order within the slice: next fragments' reads, then matrix instructions with the
                // expansion arithmetic placed between them, then the LDS writes
                if (kk < 3) __builtin_amdgcn_sched_group_barrier(0x100, TM + TN, 0);
                __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
                __builtin_amdgcn_sched_group_barrier(0x002, 4, 0);
                __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
                __builtin_amdgcn_sched_group_barrier(0x002, 4, 0);
                __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
                __builtin_amdgcn_sched_group_barrier(0x002, 4, 0);
                __builtin_amdgcn_sched_group_barrier(0x200, 1, 0);
                __builtin_amdgcn_sched_group_barrier(0x008, TM * TN - 3, 0);
            }
            end_step();
        }
    };

    int s = 0;
    for (; s + 6 <= nsteps; s += 6) {
        step(StepIdx<0>{}, s);
        step(StepIdx<1>{}, s + 1);
        step(StepIdx<2>{}, s + 2);
        step(StepIdx<3>{}, s + 3);
        step(StepIdx<4>{}, s + 4);
        step(StepIdx<5>{}, s + 5);
    }
    if (s < nsteps) step(StepIdx<0>{}, s);
    if (s + 1 < nsteps) step(StepIdx<1>{}, s + 1);
    if (s + 2 < nsteps) step(StepIdx<2>{}, s + 2);
    if (s + 3 < nsteps) step(StepIdx<3>{}, s + 3);
    if (s + 4 < nsteps) step(StepIdx<4>{}, s + 4);
    // no direct-to-LDS load may still be writing (and no fragment read still pending) when the
    // workgroup's LDS is released
    __builtin_amdgcn_s_waitcnt(waitcnt_imm(0, 0));

    // ---- epilogue: multiply by the global scale(s), store fp32; a K slice of a split product
    // (w_g == nullptr) stores its raw partial sums into its own [M x ldc] plane of C instead ----
    const bool partial = w_g == nullptr;
    const float gw = partial ? 1.0f : *w_g;
    const float ga = (A_X && !partial) ? ((A_QS || PRE) ? qs_g : *a_g) : 1.0f;
    float *Cs = C + (int64_t)slice * M * ldc;
    if constexpr (LR) {
        // low-rank branch (unsplit products only): scale the sums first, with the same roundings as
        // the store below, then add T . U^T on the matrix cores and store
#pragma unroll
        for (int i = 0; i < TM; i++)
#pragma unroll
            for (int j = 0; j < TN; j++)
#pragma unroll
                for (int e = 0; e < 16; e++) {
                    float v = acc[i][j][e];
                    if (A_X) v = v * ga;
                    acc[i][j][e] = v * gw;
                }
        // T . U^T in chunks of kLrChunk ranks: the tile's rows of T_hi, T_lo and U are staged in LDS
        // (free once the main loop is done) by all threads at once, then read as fragments
        constexpr int LROW = kLrChunk + 8;  // padded bf16 row: fragment reads spread over the banks
        constexpr int LR_UNITS = (2 * BM + BN) * (kLrChunk / 8);  // 16-byte units per chunk
        static_assert((2 * BM + BN) * LROW * 2 <= LDS_BYTES, "LDS for the low-rank chunk");
        static_assert(BM * 8 % NT == 0, "one staging region per pass of the threads");
        __bf16 *lt = reinterpret_cast<__bf16 *>(smem);
        const int r = lr.r;
        // the tile's rows of T_hi, T_lo and U: rows past M or N fall outside and read as zero
        const __amdgpu_buffer_rsrc_t rt[3] = {lr_rsrc(lr.t + m0 * r, mrows * r * 2),
                                              lr_rsrc(lr.t + M * (int64_t)r + m0 * r, mrows * r * 2),
                                              lr_rsrc(lr.u + n0 * r, nrows * r * 2)};
        constexpr int LR_PER = (LR_UNITS + NT - 1) / NT;
        for (int rc0 = 0; rc0 < r; rc0 += kLrChunk) {
            // all of this thread's loads first (no branches around them), then the LDS writes
            bf16x8 v[LR_PER];
#pragma unroll
            for (int q = 0; q < LR_PER; q++) {
                const int d = tid + q * NT;
                const int row = d / (kLrChunk / 8), c8 = (d % (kLrChunk / 8)) * 8;  // LDS row, rank offset
                // the region (T_hi, T_lo, U) is the same for all threads of one q: BM * 8 % NT == 0
                const int which = q * NT < BM * 8 ? 0 : q * NT < 2 * BM * 8 ? 1 : 2;
                const int lrow = row - which * BM;
                const bool in = d < LR_UNITS && rc0 + c8 < r;
                const uint32_t o = in ? (uint32_t)(lrow * r + rc0 + c8) * 2 : kLrOob;
                v[q] = lr_load(which == 0 ? rt[0] : which == 1 ? rt[1] : rt[2], o);
            }
            __syncthreads();  // the previous reads of LDS (main loop or chunk) are done
#pragma unroll
            for (int q = 0; q < LR_PER; q++) {
                const int d = tid + q * NT;
                if (d < LR_UNITS) {
                    const int row = d / (kLrChunk / 8), c8 = (d % (kLrChunk / 8)) * 8;
                    *reinterpret_cast<bf16x8 *>(lt + row * LROW + c8) = v[q];
                }
            }
            __syncthreads();
            const int kend = (r - rc0) < kLrChunk ? (r - rc0) : kLrChunk;
            for (int kk = 0; kk < kend; kk += 16) {
                bf16x8 ah[TM], al[TM], bu[TN];
                const int kc = kk + (lane >> 5) * 8;
#pragma unroll
                for (int i = 0; i < TM; i++) {
                    const int row = wm * WTM + i * 32 + (lane & 31);
                    ah[i] = *reinterpret_cast<const bf16x8 *>(lt + row * LROW + kc);
                    al[i] = *reinterpret_cast<const bf16x8 *>(lt + (BM + row) * LROW + kc);
                }
#pragma unroll
                for (int j = 0; j < TN; j++)
                    bu[j] = *reinterpret_cast<const bf16x8 *>(lt + (2 * BM + wn * WTN + j * 32 + (lane & 31)) * LROW + kc);
#pragma unroll
                for (int i = 0; i < TM; i++)
#pragma unroll
                    for (int j = 0; j < TN; j++) {
                        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ah[i], bu[j], acc[i][j], 0, 0, 0);
                        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(al[i], bu[j], acc[i][j], 0, 0, 0);
                    }
            }
        }
#pragma unroll
        for (int i = 0; i < TM; i++)
#pragma unroll
            for (int j = 0; j < TN; j++) {
                const int64_t col = n0 + wn * WTN + j * 32 + (lane % 32);
#pragma unroll
                for (int e = 0; e < 16; e++) {
                    const int64_t row = m0 + wm * WTM + i * 32 + 8 * (e / 4) + 4 * (lane / 32) + (e % 4);
                    if (row < M && col < N) C[row * ldc + col] = acc[i][j][e];
                }
            }
        return;
    }
#pragma unroll
    for (int i = 0; i < TM; i++) {
#pragma unroll
        for (int j = 0; j < TN; j++) {
            const int64_t col = n0 + wn * WTN + j * 32 + (lane % 32);
#pragma unroll
            for (int e = 0; e < 16; e++) {
                const int64_t row = m0 + wm * WTM + i * 32 + 8 * (e / 4) + 4 * (lane / 32) + (e % 4);
                if (row < M && col < N) {
                    float v = acc[i][j][e];
                    if (!partial) {
                        if (A_X) v = v * ga;
                        v = v * gw;
                    }
                    Cs[row * ldc + col] = v;
                }
            }
        }
    }
}

// Sum of the split-K partial planes P[s] ([M x ldp] each) in slice order, times the global
// scale(s): C = ((sum_s P[s]) * g_a) * g_w.  One thread per output element.  GA: 0 no activation
// scale, 1 *a_g is g_a, 2 *a_g is a static amax (g_a = fl(amax / 2688)).
template <int GA>
__global__ __launch_bounds__(256) void k_splitk_reduce(const float *__restrict__ P, int splits, int64_t M, int64_t N,
                                                       int64_t ldp, const float *__restrict__ a_g,
                                                       const float *__restrict__ w_g, float *__restrict__ C,
                                                       int64_t ldc) {
    const float gw = *w_g;
    const float ga = GA == 1 ? *a_g : GA == 2 ? *a_g / 2688.0f : 1.0f;
    const int64_t total = M * N;
    const int64_t plane = M * ldp;
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < total; i += (int64_t)gridDim.x * blockDim.x) {
        const int64_t r = i / N, c = i - r * N;
        const float *p = P + r * ldp + c;
        float v = p[0];
        for (int s = 1; s < splits; s++) v += p[(int64_t)s * plane];
        if (GA) v = v * ga;
        C[r * ldc + c] = v * gw;
    }
}

// ------------------------------------------------------------------------------------------------
// GEMV, M <= 5
// ------------------------------------------------------------------------------------------------
template <int MM, int AM>
__global__ __launch_bounds__(256) void k_gemv(const __bf16 *__restrict__ A, int64_t lda,
                                              const uint8_t *__restrict__ a_codes,
                                              const uint8_t *__restrict__ a_scales, const float *__restrict__ a_g,
                                              const uint8_t *__restrict__ w_codes,
                                              const uint8_t *__restrict__ w_scales, const float *__restrict__ w_g,
                                              float *__restrict__ C, int64_t ldc, int64_t N, int64_t K) {
    extern __shared__ __attribute__((aligned(16))) uint32_t a_lds[];  // [MM][K/2] bf16 pairs
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int64_t kp = K / 2;
    const int64_t nblk = K / 16;
    const int64_t wave = ((int64_t)blockIdx.x * blockDim.x + tid) >> 6;
    const int64_t nwaves = ((int64_t)gridDim.x * blockDim.x) >> 6;

    // A wave takes two rows at a time (n and n + nwaves) and, per batch, UB blocks per lane of each;
    // all loads of a batch are issued before any is used.  Lanes past the row's last block load
    // that block again and add nothing.
    constexpr int UB = 4;
    u32x2 cw[2][UB];
    uint32_t sb[2][UB];
    auto load_batch = [&](const int64_t (&rows)[2], int64_t b0) {
#pragma unroll
        for (int h = 0; h < 2; h++)
#pragma unroll
            for (int u = 0; u < UB; u++) {
                int64_t b = b0 + lane + 64 * u;
                b = b < nblk ? b : nblk - 1;
                cw[h][u] = *reinterpret_cast<const u32x2 *>(w_codes + rows[h] * (K / 2) + b * 8);
                sb[h][u] = w_scales[rows[h] * nblk + b];
            }
    };
    // the first batch is in flight while A is staged
    int64_t n = wave;
    if (n < N) {
        const int64_t rows[2] = {n, (n + nwaves) < N ? (n + nwaves) : n};
        load_batch(rows, 0);
    }

    // stage A (expanded exactly to bf16 for NVFP4 and E4M3 activations) in LDS
    for (int64_t i = tid; i < MM * (K / 8); i += blockDim.x) {
        const int64_t m = i / (K / 8), c8 = i % (K / 8);
        u32x4 v;
        if constexpr (AM == kAmBf16) {
            v = *reinterpret_cast<const u32x4 *>(A + m * lda + c8 * 8);
        } else if constexpr (AM == kAmNvfp4) {
            const uint32_t w = *reinterpret_cast<const uint32_t *>(a_codes + m * (K / 2) + c8 * 4);
            v = expand8(w, e4m3_to_f32(a_scales[m * (K / 16) + c8 / 2]));
        } else {
            v = expand8_fp8_bf16(*reinterpret_cast<const u32x2 *>(a_codes + m * lda + c8 * 8));
        }
        *reinterpret_cast<u32x4 *>(&a_lds[m * kp + c8 * 4]) = v;
    }
    __syncthreads();

    const float gw = *w_g;
    const float ga = AM != kAmBf16 ? *a_g : 1.0f;
    for (; n < N; n += 2 * nwaves) {
        const int64_t rows[2] = {n, (n + nwaves) < N ? (n + nwaves) : n};
        float acc[2][MM];
#pragma unroll
        for (int h = 0; h < 2; h++)
#pragma unroll
            for (int m = 0; m < MM; m++) acc[h][m] = 0.0f;
        for (int64_t b0 = 0; b0 < nblk; b0 += 64 * UB) {
            if (b0 > 0 || n != wave) load_batch(rows, b0);
#pragma unroll
            for (int u = 0; u < UB; u++) {
                const int64_t b = b0 + lane + 64 * u;
                const int64_t bc = b < nblk ? b : nblk - 1;
#pragma unroll
                for (int h = 0; h < 2; h++) {
                    const float sc = __builtin_amdgcn_cvt_f32_fp8((int)sb[h][u], 0);
                    bf16x2 wv[8];
                    fp4_unpack8_bf16x2(cw[h][u][0], wv);
                    fp4_unpack8_bf16x2(cw[h][u][1], wv + 4);
#pragma unroll
                    for (int m = 0; m < MM; m++) {
                        const u32x4 *ap = reinterpret_cast<const u32x4 *>(&a_lds[m * kp + bc * 8]);
                        const u32x4 a0 = ap[0], a1 = ap[1];
                        float part = 0.0f;
#pragma unroll
                        for (int q = 0; q < 4; q++) {
                            part = __builtin_amdgcn_fdot2_f32_bf16(wv[q], as_bf16x2(a0[q]), part, false);
                            part = __builtin_amdgcn_fdot2_f32_bf16(wv[4 + q], as_bf16x2(a1[q]), part, false);
                        }
                        acc[h][m] += b < nblk ? part * sc : 0.0f;
                    }
                }
            }
        }
#pragma unroll
        for (int h = 0; h < 2; h++) {
            if (h == 1 && rows[1] == rows[0]) break;
#pragma unroll
            for (int m = 0; m < MM; m++) {
                const float t = wave_sum_f32(acc[h][m]);
                if (lane == 0) {
                    float v = t;
                    if (AM != kAmBf16) v = v * ga;
                    C[m * ldc + rows[h]] = v * gw;
                }
            }
        }
    }
}

// Sums over the wave of V per-lane values at once (V a multiple of 4), in about 4.5 instructions per
// value instead of the 11 of a reduction each: lanes exchange halves of their values with the lane
// across bit 0, then bit 1 (each step halves the values a lane holds), so lane class c = lane & 3
// ends up with the quad sums of values c, c + 4, ...; two row rotations finish the rows of 16 lanes
// and four lane reads the wave.  out[] is the same in every lane.
template <int V>
__device__ __forceinline__ void wave_sum_multi(const float (&v)[V], float (&out)[V]) {
    static_assert(V % 4 == 0, "values in groups of four");
    const int lane = threadIdx.x & 63;
    const bool b0 = lane & 1, b1 = lane & 2;
    float h[V / 2];
#pragma unroll
    for (int i = 0; i < V / 2; i++) {
        const float send = b0 ? v[2 * i] : v[2 * i + 1];
        const float keep = b0 ? v[2 * i + 1] : v[2 * i];
        h[i] = keep + u2f(dpp_u32<kDppXor1>(f2u(send)));
    }
    float q[V / 4];
#pragma unroll
    for (int i = 0; i < V / 4; i++) {
        const float send = b1 ? h[2 * i] : h[2 * i + 1];
        const float keep = b1 ? h[2 * i + 1] : h[2 * i];
        q[i] = keep + u2f(dpp_u32<kDppXor2>(f2u(send)));
        q[i] += u2f(dpp_u32<kDppRowRor4>(f2u(q[i])));
        q[i] += u2f(dpp_u32<kDppRowRor8>(f2u(q[i])));
    }
    // lane class c holds value 4 i + c in q[i]
#pragma unroll
    for (int i = 0; i < V / 4; i++)
#pragma unroll
        for (int c = 0; c < 4; c++)
            out[4 * i + c] = (u2f(readlane_u32(f2u(q[i]), c)) + u2f(readlane_u32(f2u(q[i]), 16 + c))) +
                             (u2f(readlane_u32(f2u(q[i]), 32 + c)) + u2f(readlane_u32(f2u(q[i]), 48 + c)));
}

// k_gemv_reg: the same product for K <= 4096 without LDS.  Lane l works on blocks l + 64 u (u < UB) of
// every row it visits, so it loads those blocks of A (expanded to bf16 for NVFP4 and E4M3
// activations) into registers once; lanes past the last block hold zeros there and add nothing.
// A wave takes RW rows (n, n + nwaves, ...) and issues the loads of all of them (A's first, then
// every row's scale bytes, then the rows' codes in order) before any arithmetic, so that with the
// grid sized to the resident waves the whole of W is requested at once; each row's arithmetic then
// waits for that row's codes only (the code is straight-line, so the compiler's wait counts follow
// the order of the loads).  The wave's RW x MM sums are reduced together at the end.  One launch
// covers at most RW x (launched waves) rows; the host offsets further launches for taller W.
template <int MM, int AM, int UB, int RW>
__global__ __launch_bounds__(256) void k_gemv_reg(const __bf16 *__restrict__ A, int64_t lda,
                                                  const uint8_t *__restrict__ a_codes,
                                                  const uint8_t *__restrict__ a_scales, const float *__restrict__ a_g,
                                                  const uint8_t *__restrict__ w_codes,
                                                  const uint8_t *__restrict__ w_scales, const float *__restrict__ w_g,
                                                  float *__restrict__ C, int64_t ldc, int64_t N, int64_t K) {
    constexpr int V = (RW * MM + 3) / 4 * 4;
    const int lane = threadIdx.x & 63;
    const int64_t nblk = K / 16;
    // wave-uniform indices, so that row addresses are scalar and each lane adds a 32-bit offset
    const int64_t wave = (int64_t)blockIdx.x * (blockDim.x >> 6) + __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int64_t nwaves = (int64_t)gridDim.x * (blockDim.x >> 6);
    // lanes past the last block load the last block (in bounds) and multiply it by zeros of A
    uint32_t blk[UB];
#pragma unroll
    for (int u = 0; u < UB; u++) {
        const int64_t b = lane + 64 * u;
        blk[u] = (uint32_t)(b < nblk ? b : nblk - 1);
    }
    u32x2 cw[RW][UB];
    uint32_t sb[RW][UB];
    // rows past the end read row N - 1 and store nothing; the loads are unconditional so that the
    // compiler's wait counts follow this one order of loads
    const auto row_of = [&](int j) {
        const int64_t n = wave + j * nwaves;
        return n < N ? n : N - 1;
    };
    // the scale bytes of all the wave's rows (small) go before any codes: the compiler widens a
    // loaded byte wherever it likes, and waiting for these then never waits for codes
    const __amdgpu_buffer_rsrc_t rs = lr_rsrc(w_scales, N * nblk);
    const auto load_scales = [&]() {
#pragma unroll
        for (int j = 0; j < RW; j++) {
            const uint32_t so = (uint32_t)(row_of(j) * nblk);
#pragma unroll
            for (int u = 0; u < UB; u++) sb[j][u] = __builtin_amdgcn_raw_buffer_load_b8(rs, blk[u], so, 0);
        }
        __builtin_amdgcn_sched_barrier(0);
    };
    const auto load_row = [&](int j) {
        const uint8_t *cr = w_codes + row_of(j) * (K / 2);
#pragma unroll
        for (int u = 0; u < UB; u++) cw[j][u] = *reinterpret_cast<const u32x2 *>(cr + blk[u] * 8u);
        __builtin_amdgcn_sched_barrier(0);
    };
    // A's blocks of this lane, 16 bf16 each.  A's loads go first (a wave's loads complete in issue
    // order); NVFP4 and E4M3 activations are expanded once W's first loads are on their way.
    u32x4 av[MM][UB][2];
    uint32_t as[MM][UB];
#pragma unroll
    for (int m = 0; m < MM; m++)
#pragma unroll
        for (int u = 0; u < UB; u++) {
            if constexpr (AM == kAmBf16) {
                const u32x4 *ap = reinterpret_cast<const u32x4 *>(A + m * lda + blk[u] * 16u);
                av[m][u][0] = ap[0];
                av[m][u][1] = ap[1];
            } else if constexpr (AM == kAmNvfp4) {
                const u32x2 c = *reinterpret_cast<const u32x2 *>(a_codes + m * (K / 2) + blk[u] * 8u);
                av[m][u][0][0] = c[0];
                av[m][u][1][0] = c[1];
                as[m][u] = a_scales[m * nblk + blk[u]];
            } else {
                const u32x4 b = *reinterpret_cast<const u32x4 *>(a_codes + m * lda + blk[u] * 16u);
                av[m][u][0] = b;
            }
        }
    __builtin_amdgcn_sched_barrier(0);
    load_scales();
#pragma unroll
    for (int j = 0; j < RW; j++) load_row(j);
#pragma unroll
    for (int m = 0; m < MM; m++)
#pragma unroll
        for (int u = 0; u < UB; u++) {
            if constexpr (AM == kAmNvfp4) {
                const float s = __builtin_amdgcn_cvt_f32_fp8((int)as[m][u], 0);
                const uint32_t c0 = av[m][u][0][0], c1 = av[m][u][1][0];
                av[m][u][0] = expand8(c0, s);
                av[m][u][1] = expand8(c1, s);
            } else if constexpr (AM == kAmFp8) {
                const u32x4 b = av[m][u][0];
                av[m][u][0] = expand8_fp8_bf16(u32x2{b[0], b[1]});
                av[m][u][1] = expand8_fp8_bf16(u32x2{b[2], b[3]});
            }
        }
    if (nblk < 64 * UB) {  // some lanes hold blocks past the end: their A is zero
#pragma unroll
        for (int u = 0; u < UB; u++)
            if (lane + 64 * u >= nblk)
#pragma unroll
                for (int m = 0; m < MM; m++) av[m][u][0] = av[m][u][1] = u32x4{0u, 0u, 0u, 0u};
    }
    float acc[V];
#pragma unroll
    for (int t = 0; t < V; t++) acc[t] = 0.0f;
#pragma unroll
    for (int j = 0; j < RW; j++) {
#pragma unroll
        for (int u = 0; u < UB; u++) {
            const float sc = __builtin_amdgcn_cvt_f32_fp8((int)sb[j][u], 0);
            bf16x2 wv[8];
            fp4_unpack8_bf16x2(cw[j][u][0], wv);
            fp4_unpack8_bf16x2(cw[j][u][1], wv + 4);
#pragma unroll
            for (int m = 0; m < MM; m++) {
                const u32x4 a0 = av[m][u][0], a1 = av[m][u][1];
                float part = 0.0f;
#pragma unroll
                for (int q = 0; q < 4; q++) {
                    part = __builtin_amdgcn_fdot2_f32_bf16(wv[q], as_bf16x2(a0[q]), part, false);
                    part = __builtin_amdgcn_fdot2_f32_bf16(wv[4 + q], as_bf16x2(a1[q]), part, false);
                }
                acc[j * MM + m] = __builtin_fmaf(part, sc, acc[j * MM + m]);
            }
        }
    }
    float tot[V];
    wave_sum_multi<V>(acc, tot);
    const float gw = *w_g;
    const float ga = AM != kAmBf16 ? *a_g : 1.0f;
    if (lane == 0) {
#pragma unroll
        for (int j = 0; j < RW; j++) {
            const int64_t n = wave + j * nwaves;
            if (n < N)
#pragma unroll
                for (int m = 0; m < MM; m++) {
                    float v = tot[j * MM + m];
                    if (AM != kAmBf16) v = v * ga;
                    C[m * ldc + n] = v * gw;
                }
        }
    }
}

// k_gemv_mfma: the same product for up to 16 rows of A on the matrix cores.  The W rows are the
// 16-row operand of v_mfma_f32_16x16x32_bf16 and the rows of A (expanded exactly to bf16) the
// 16-column operand, so one instruction covers 16 W rows x 32 K whatever M is.  Four waves take 16
// W rows (a row group) at a time; they take the 128-element K chunks c = wave, wave + 4, ...:
// lane l loads 32 codes (16 bytes) of row l % 16 at K offset 32 (l / 16) of each chunk and the two
// scale bytes of those two blocks, and expands them with their block scales into the operands of
// four instructions.  A sits in LDS once per workgroup, with one more row of zeros that the lanes
// past row M read.  The four waves' 16 x 16 tiles are added in a fixed order through LDS.
// Workgroups loop over the row groups with the same trip count (the surplus iterations at the end
// repeat the last row group, from cache, and store nothing), and the loads of the next row group are
// issued before the arithmetic of the current one, so the code has no branch around a load and the
// compiler's waits count exactly.  Loads past K or past W read zeros through the buffer ranges.
constexpr int kGemvFillBatch = 4;  // A units (8 elements) per thread loaded before any is written

template <int AM, int CPW>
__global__ __launch_bounds__(256) void k_gemv_mfma(const __bf16 *__restrict__ A, int64_t lda,
                                                   const uint8_t *__restrict__ a_codes,
                                                   const uint8_t *__restrict__ a_scales, const float *__restrict__ a_g,
                                                   const uint8_t *__restrict__ w_codes,
                                                   const uint8_t *__restrict__ w_scales, const float *__restrict__ w_g,
                                                   float *__restrict__ C, int64_t ldc, int M, int64_t N, int64_t K) {
    extern __shared__ __align__(16) uint8_t gemv_smem[];
    __bf16 *act = reinterpret_cast<__bf16 *>(gemv_smem);
    const int k32 = (int)K;  // K <= 4096: every offset below fits 32 bits
    const uint32_t kh = (uint32_t)k32 / 2, kb = (uint32_t)k32 / 16;  // code and scale bytes per row
    const int nch = (k32 + 127) / 128;
    const int ks = nch * 128 + 8;  // LDS row stride (bf16): 16 bytes past a multiple of 256, so the 16 rows
                                   // of one read fall in different banks
    const int tid = threadIdx.x, lane = tid & 63;
    const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);  // K quarter
    f32x4 *red = reinterpret_cast<f32x4 *>(gemv_smem + (size_t)(M + 1) * ks * 2);
    const int r16 = lane & 15, g4 = lane >> 4;
    const int64_t nrg = (N + 15) / 16;
    const int64_t iters = (nrg + gridDim.x - 1) / gridDim.x;

    // ---- A (rows 0..M-1) as exact bf16 and a row of zeros (row M), 8 elements per unit ----
    const int upr = nch * 16;  // units per row
    const int units = (M + 1) * upr;
    // A through buffer ranges: units past row M - 1, past K or past the last unit read zeros, and
    // their stores land in the zero row (so neither loads nor stores sit under a branch)
    const __amdgpu_buffer_rsrc_t ra =
        AM == kAmBf16  ? buffer_rsrc(A, (uint64_t)((M - 1) * lda + k32) * 2)
        : AM == kAmFp8 ? buffer_rsrc(a_codes, (uint64_t)((M - 1) * lda + k32))
                       : buffer_rsrc(a_codes, (uint64_t)M * kh);
    const __amdgpu_buffer_rsrc_t ras = buffer_rsrc(a_scales, AM == kAmNvfp4 ? (uint64_t)M * kb : 0);
    const auto fill_load = [&](int u) {
        const int m = u / upr;
        const int k8 = (u - m * upr) * 8;
        const uint32_t past = ((u < units) & (m < M) & (k8 < k32)) ? 0u : kOffsetPastRange;
        u32x4 v = u32x4{0u, 0u, 0u, 0u};
        if constexpr (AM == kAmBf16) {
            v = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(
                                              ra, ((uint32_t)(m * lda + k8) * 2) | past, 0, 0));
        } else if constexpr (AM == kAmNvfp4) {
            v[0] = __builtin_amdgcn_raw_buffer_load_b32(ra, (m * kh + k8 / 2) | past, 0, 0);
            v[1] = __builtin_amdgcn_raw_buffer_load_b8(ras, (m * kb + k8 / 16) | past, 0, 0);
        } else {
            const u32x2 b = __builtin_bit_cast(
                u32x2, __builtin_amdgcn_raw_buffer_load_b64(ra, (uint32_t)(m * lda + k8) | past, 0, 0));
            v[0] = b[0];
            v[1] = b[1];
        }
        return v;
    };
    const auto fill_store = [&](int u, u32x4 v) {
        const int m = u / upr;
        const int k8 = (u - m * upr) * 8;
        if constexpr (AM == kAmNvfp4) v = expand8(v[0], __builtin_amdgcn_cvt_f32_fp8((int)v[1], 0));
        else if constexpr (AM == kAmFp8) v = expand8_fp8_bf16(u32x2{v[0], v[1]});
        // zeros past K and in row M; units past the last go to row M too (zeros)
        __bf16 *dst = u < units ? act + m * ks + k8 : act + M * ks + (u % upr) * 8;
        *reinterpret_cast<u32x4 *>(dst) = v;
    };
    u32x4 fv[kGemvFillBatch];
#pragma unroll
    for (int b = 0; b < kGemvFillBatch; b++) fv[b] = fill_load(tid + 256 * b);
    __builtin_amdgcn_sched_barrier(0);

    // ---- the W loads of one row group ----
    const auto rg_of = [&](int64_t it) {
        const int64_t rg = (int64_t)blockIdx.x + it * gridDim.x;
        return rg < nrg ? rg : nrg - 1;
    };
    uint32_t sc[CPW];
    u32x4 q[CPW];
    const auto load_w = [&](int64_t rg) {
        const int64_t r0 = rg * 16, nr = N - r0 < 16 ? N - r0 : 16;
        const __amdgpu_buffer_rsrc_t rc = buffer_rsrc(w_codes + r0 * kh, (uint64_t)nr * kh);
        const __amdgpu_buffer_rsrc_t rs = buffer_rsrc(w_scales + r0 * kb, (uint64_t)nr * kb);
        // rows past the end repeat the last and store nothing
        const uint32_t row = (uint32_t)(r16 < nr ? r16 : (int)nr - 1);
        // offsets of chunks past K get the bit that puts them past the range (an OR, so that the
        // compiler does not branch around the offset arithmetic and the load)
        uint32_t past[CPW];
#pragma unroll
        for (int i = 0; i < CPW; i++) {
            const int c = wv + 4 * i;
            past[i] = ((c < nch) & (c * 128 + 32 * g4 < k32)) ? 0u : kOffsetPastRange;
        }
#pragma unroll
        for (int i = 0; i < CPW; i++)
            sc[i] = __builtin_amdgcn_raw_buffer_load_b16(rs, (row * kb + (wv + 4 * i) * 8 + 2 * g4) | past[i], 0, 0);
#pragma unroll
        for (int i = 0; i < CPW; i++)
            q[i] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(
                                                 rc, (row * kh + (wv + 4 * i) * 64 + 16 * g4) | past[i], 0, 0));
        __builtin_amdgcn_sched_barrier(0);
    };
    load_w(rg_of(0));

    // ---- A into LDS (the first batch was loaded before W; larger A in further batches) ----
#pragma unroll
    for (int b = 0; b < kGemvFillBatch; b++) fill_store(tid + 256 * b, fv[b]);
    for (int base = 256 * kGemvFillBatch; base < units; base += 256 * kGemvFillBatch) {
#pragma unroll
        for (int b = 0; b < kGemvFillBatch; b++) fv[b] = fill_load(base + tid + 256 * b);
#pragma unroll
        for (int b = 0; b < kGemvFillBatch; b++) fill_store(base + tid + 256 * b, fv[b]);
    }
    __syncthreads();

    const float gw = *w_g;
    const float ga = AM != kAmBf16 ? *a_g : 1.0f;
    // the A rows this lane reads: its own, or the zero row past M
    const __bf16 *arow = act + (r16 < M ? r16 : M) * ks + 32 * g4;
    const auto chunk_of = [&](int i) {
        const int c = wv + 4 * i;
        return c < nch ? c : nch - 1;  // chunks past K have zero W
    };
    // one row group: per chunk, the four A reads, then the W expansion (which covers their latency),
    // then the four matrix instructions
    const auto compute = [&]() {
        f32x4 acc = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
        for (int i = 0; i < CPW; i++) {
            bf16x8 av[4];
#pragma unroll
            for (int st = 0; st < 4; st++) av[st] = *reinterpret_cast<const bf16x8 *>(arow + chunk_of(i) * 128 + 8 * st);
            __builtin_amdgcn_sched_barrier(0);
            const float s0 = __builtin_amdgcn_cvt_f32_fp8((int)sc[i], 0);
            const float s1 = __builtin_amdgcn_cvt_f32_fp8((int)sc[i], 1);
            u32x4 w[4];
#pragma unroll
            for (int st = 0; st < 4; st++) w[st] = expand8(q[i][st], st < 2 ? s0 : s1);
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int st = 0; st < 4; st++)
                acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, w[st]), av[st], acc, 0, 0, 0);
        }
        return acc;
    };
    // the waves' tiles, added in a fixed order; lane l holds C[l % 16][r0 + 4 (l / 16) + e]
    const auto finish = [&](int64_t it, f32x4 acc) {
        if (wv > 0) red[(wv - 1) * 64 + lane] = acc;
        __syncthreads();
        const int64_t rg = (int64_t)blockIdx.x + it * gridDim.x;
        if (wv == 0 && r16 < M && rg < nrg) {
            const f32x4 t1 = red[lane], t2 = red[64 + lane], t3 = red[128 + lane];
#pragma unroll
            for (int e = 0; e < 4; e++) {
                const int64_t n = rg * 16 + 4 * g4 + e;
                float v = ((acc[e] + t1[e]) + t2[e]) + t3[e];
                if (AM != kAmBf16) v = v * ga;
                if (n < N) C[r16 * ldc + n] = v * gw;
            }
        }
        __syncthreads();
    };
    // one row group per trip: its loads, then its arithmetic (nothing is pending across the loop)
    for (int64_t it = 0;; it++) {
        finish(it, compute());
        if (it + 1 >= iters) break;
        load_w(rg_of(it + 1));
    }
}

// ------------------------------------------------------------------------------------------------
// host launchers
// ------------------------------------------------------------------------------------------------
// Activation operand of the launchers: bf16 rows, an NVFP4 tensor, or E4M3 bytes.
struct GemmA {
    const void *bf16;       // kAmBf16: [M x K] bf16, row stride lda
    const uint8_t *codes;   // kAmNvfp4: codes; kAmFp8: [M x K] E4M3 bytes, row stride lda
    const uint8_t *scales;  // kAmNvfp4: block scales
    const float *g;         // kAmNvfp4: global scale; kAmFp8: tensor scale
    int64_t lda;
};

size_t gemv_lds_bytes(int64_t M, int64_t K) { return (size_t)M * (size_t)K * 2; }

// Rows per wave of the register GEMV for tall W: at 18 432 x 3072 (M = 2) the resident waves then
// take all of W in one round (6 rows each measured faster than 4 or 8).
constexpr int kGemvRows = 6;

// Waves per CU of the register GEMV: as many as the registers let stay resident (from the
// runtime's occupancy calculation, once per instantiation).
template <int MM, int AM, int UB, int RW>
static int64_t gemv_waves_per_cu() {
    static std::atomic<int> cached{0};
    int n = cached.load(std::memory_order_relaxed);
    if (n == 0) {
        int b = 0;
        if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&b, k_gemv_reg<MM, AM, UB, RW>, 256, 0) != hipSuccess || b < 1)
            b = 1;
        n = b * 4;
        cached.store(n, std::memory_order_relaxed);
    }
    return n;
}

// M <= 4: A in registers (K <= 4096) or LDS; M = 5: A in LDS.  Beyond that the dot products (8 per
// 16-element block and row of A) outweigh the stream of W: at M = 8 the LDS form measured 19.3 us
// against 22.5 us tiled at N = K = 3072, but 48.6 against 37.8 us at N = 18432, so the tiled kernels
// run from M = 6.
// The matrix-core GEMV: up to 16 rows of A, K a multiple of 32 up to 4096 (at most 8 chunks per wave).
static size_t gemv_mfma_lds_bytes(int64_t M, int64_t K) {
    return (size_t)(M + 1) * (size_t)(((K + 127) / 128) * 128 + 8) * 2 + 3 * 64 * 16;
}
static bool gemv_mfma_fits(int64_t M, int64_t K) {
    return M >= 1 && M <= 16 && K > 0 && K % 32 == 0 && K <= 4096 && gemv_mfma_lds_bytes(M, K) <= 160 * 1024;
}
// From this many rows of A the matrix-core GEMV takes over from the register GEMV (at 18432 x 3072,
// M = 3 and 4 took 11.1 and 12.9 us in the register form against 14.5 and 14.8 us; M = 5 24.6 in the
// LDS form against 15.2 us).
constexpr int kGemvMfmaMinM = 5;

bool gemv_applies(int64_t M, int64_t K) {
    return (M >= 1 && M <= 5 && gemv_lds_bytes(M, K) <= 64 * 1024) || (M >= kGemvMfmaMinM && gemv_mfma_fits(M, K));
}

// The grid: enough waves that each takes at most RW rows, capped at the resident waves, with the
// rows spread evenly over the waves.  W taller than RW x (resident waves) rows takes several
// launches, each on its own band of rows (codes, scales and output columns offset by the band).
template <int MM, int AM, int UB, int RW>
static void launch_gemv_reg(const GemmA &a, const nvfp4_tensor *w, float *c, int64_t ldc, int num_cus,
                            hipStream_t stream) {
    const int64_t N = w->rows, K = w->cols;
    const int64_t max_waves = (int64_t)num_cus * gemv_waves_per_cu<MM, AM, UB, RW>();
    const int64_t band = max_waves * RW;
    for (int64_t r0 = 0; r0 < N; r0 += band) {
        const int64_t rows = N - r0 < band ? N - r0 : band;
        const int64_t waves = (rows + RW - 1) / RW;
        const int64_t grid = (waves + 3) / 4;
        hipLaunchKernelGGL((k_gemv_reg<MM, AM, UB, RW>), dim3((unsigned)grid), dim3(256), 0, stream,
                           (const __bf16 *)a.bf16, a.lda, a.codes, a.scales, a.g, w->codes + r0 * (K / 2),
                           w->scales + r0 * (K / 16), w->global_scale, c + r0, ldc, rows, K);
    }
}

// Rows per wave: 2 while the resident waves cover W two rows each, else kGemvRows.
template <int MM, int AM, int UB>
static void launch_gemv_rows(const GemmA &a, const nvfp4_tensor *w, float *c, int64_t ldc, int num_cus,
                             hipStream_t stream) {
    const int64_t N = w->rows;
    if (N <= 2 * (int64_t)num_cus * gemv_waves_per_cu<MM, AM, UB, 2>())
        return launch_gemv_reg<MM, AM, UB, 2>(a, w, c, ldc, num_cus, stream);
    launch_gemv_reg<MM, AM, UB, kGemvRows>(a, w, c, ldc, num_cus, stream);
}

template <int MM, int AM>
static void launch_gemv_t(const GemmA &a, const nvfp4_tensor *w, float *c, int64_t ldc, int num_cus,
                          hipStream_t stream) {
    const int64_t N = w->rows, K = w->cols;
    const int64_t ub = (K / 16 + 63) / 64;  // blocks per lane
    if constexpr (MM <= 4) {  // beyond 4 rows the register form would hold too many blocks of A per lane
        if (ub <= 1) return launch_gemv_rows<MM, AM, 1>(a, w, c, ldc, num_cus, stream);
        if (ub <= 2) return launch_gemv_rows<MM, AM, 2>(a, w, c, ldc, num_cus, stream);
        if (ub <= 3) return launch_gemv_rows<MM, AM, 3>(a, w, c, ldc, num_cus, stream);
        if (ub <= 4) return launch_gemv_rows<MM, AM, 4>(a, w, c, ldc, num_cus, stream);
    }
    // a wave takes two rows per pass, one pass per wave up to 16 workgroups per CU
    int64_t grid = (N + 7) / 8;
    if (grid > (int64_t)num_cus * 16) grid = (int64_t)num_cus * 16;
    if (grid < 1) grid = 1;
    hipLaunchKernelGGL((k_gemv<MM, AM>), dim3((unsigned)grid), dim3(256), gemv_lds_bytes(MM, K), stream,
                       (const __bf16 *)a.bf16, a.lda, a.codes, a.scales, a.g, w->codes, w->scales, w->global_scale, c,
                       ldc, N, K);
}

// Workgroups of k_gemv_mfma<AM, CPW> per CU with `lds` bytes of LDS (runtime occupancy calculation).
template <int AM, int CPW>
static int gemv_mfma_per_cu(size_t lds) {
    int b = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&b, k_gemv_mfma<AM, CPW>, 256, lds) != hipSuccess || b < 1) b = 1;
    return b;
}

// The grid: as many workgroups as fit at once, no more than there are row groups, and then evened
// out so that every workgroup takes the same number of iterations.  (Workgroups of 16 waves taking
// four row groups at once against one copy of A measured slower: 18.0 against 14.5-15.7 us for
// M = 3-8 at 18432 x 3072.)
template <int AM, int CPW>
static void launch_gemv_mfma_t(int64_t M, const GemmA &a, const nvfp4_tensor *w, float *c, int64_t ldc, int num_cus,
                               hipStream_t stream) {
    const int64_t N = w->rows, K = w->cols;
    const size_t lds = gemv_mfma_lds_bytes(M, K);
    const int64_t nrg = (N + 15) / 16;
    int64_t grid = (int64_t)num_cus * gemv_mfma_per_cu<AM, CPW>(lds);
    if (grid > nrg) grid = nrg;
    const int64_t iters = (nrg + grid - 1) / grid;
    grid = (nrg + iters - 1) / iters;
    hipLaunchKernelGGL((k_gemv_mfma<AM, CPW>), dim3((unsigned)grid), dim3(256), lds, stream, (const __bf16 *)a.bf16,
                       a.lda, a.codes, a.scales, a.g, w->codes, w->scales, w->global_scale, c, ldc, (int)M, N, K);
}

template <int AM>
static void launch_gemv_mfma(int64_t M, const GemmA &a, const nvfp4_tensor *w, float *c, int64_t ldc, int num_cus,
                             hipStream_t stream) {
    const int64_t cpw = ((w->cols + 127) / 128 + 3) / 4;  // chunks per wave
    switch (cpw) {
    case 1: return launch_gemv_mfma_t<AM, 1>(M, a, w, c, ldc, num_cus, stream);
    case 2: return launch_gemv_mfma_t<AM, 2>(M, a, w, c, ldc, num_cus, stream);
    case 3: return launch_gemv_mfma_t<AM, 3>(M, a, w, c, ldc, num_cus, stream);
    case 4: return launch_gemv_mfma_t<AM, 4>(M, a, w, c, ldc, num_cus, stream);
    case 5: return launch_gemv_mfma_t<AM, 5>(M, a, w, c, ldc, num_cus, stream);
    case 6: return launch_gemv_mfma_t<AM, 6>(M, a, w, c, ldc, num_cus, stream);
    case 7: return launch_gemv_mfma_t<AM, 7>(M, a, w, c, ldc, num_cus, stream);
    default: return launch_gemv_mfma_t<AM, 8>(M, a, w, c, ldc, num_cus, stream);
    }
}

template <int AM>
static void launch_gemv(int64_t M, const GemmA &a, const nvfp4_tensor *w, float *c, int64_t ldc, int num_cus,
                        hipStream_t stream) {
    if (M >= kGemvMfmaMinM && gemv_mfma_fits(M, w->cols)) return launch_gemv_mfma<AM>(M, a, w, c, ldc, num_cus, stream);
    switch (M) {
    case 1: launch_gemv_t<1, AM>(a, w, c, ldc, num_cus, stream); break;
    case 2: launch_gemv_t<2, AM>(a, w, c, ldc, num_cus, stream); break;
    case 3: launch_gemv_t<3, AM>(a, w, c, ldc, num_cus, stream); break;
    case 4: launch_gemv_t<4, AM>(a, w, c, ldc, num_cus, stream); break;
    default: launch_gemv_t<5, AM>(a, w, c, ldc, num_cus, stream); break;
    }
}

// Tile shapes, chosen per problem by a cost model: rounds of workgroups over the CUs times the work
// one CU does per round (tile area x K steps per workgroup x co-resident tiles), divided by the
// shape's measured throughput per CU relative to the largest tile on MI355X (larger tiles amortize
// the W expansion and the LDS traffic over more output), plus, for split-K, the pass that reads
// the partial planes back.
struct TileCfg {
    int bm, bn, per_cu;
    double eff;
};
static const TileCfg kTiles[] = {
    {256, 256, 1, 1.00},  // 8 waves, 64 x 128 per wave
    {256, 192, 1, 0.97},  // 8 waves, 64 x 96 per wave
    {128, 256, 1, 0.79},  // 8 waves, 64 x 64 per wave
    {128, 128, 2, 0.72},  // 4 waves, 64 x 64 per wave, two workgroups per CU
    {128, 192, 1, 0.75},  // 8 waves, 32 x 96 per wave
};
constexpr double kUsPerTileStep = 2.0;      // one 256 x 256 x 64 step on one CU, microseconds
constexpr double kReduceBytesPerUs = 4.0e6;  // HBM rate of the partial-sum pass
constexpr int kMaxSplits = 8;

GemmPlan plan_gemm(int64_t M, int64_t N, int64_t K, int num_cus, int first_cfg) {
    GemmPlan best{first_cfg, 1, (int)((K + kBK - 1) / kBK)};
    double best_cost = 1e300;
    const int64_t steps = (K + kBK - 1) / kBK;
    const bool splittable = K % kBK == 0;
    for (int i = first_cfg; i < (int)(sizeof(kTiles) / sizeof(kTiles[0])); i++) {
        const TileCfg &t = kTiles[i];
        const double tiles = (double)((M + t.bm - 1) / t.bm) * (double)((N + t.bn - 1) / t.bn);
        const double slots = (double)num_cus * t.per_cu;
        for (int sp = 1; sp <= (splittable ? kMaxSplits : 1); sp *= 2) {
            const int64_t per = (steps + sp - 1) / sp;
            if (sp > 1 && per < 8) break;
            const int used = (int)((steps + per - 1) / per);
            const double rounds = (double)(int64_t)((tiles * used + slots - 1) / slots);
            double cost = rounds * t.per_cu * (t.bm * t.bn / 65536.0) * (double)per * kUsPerTileStep / t.eff;
            if (used > 1) cost += (double)(used + 1) * (double)M * (double)N * 4.0 / kReduceBytesPerUs;
            if (cost < best_cost) {
                best_cost = cost;
                best = GemmPlan{i, used, (int)per};
            }
        }
    }
    return best;
}

size_t gemm_ws_bytes(int64_t M, int64_t N, int64_t K, int num_cus, int first_cfg) {
    if (M <= 0 || N <= 0 || K <= 0 || gemv_applies(M, K)) return 0;
    const GemmPlan p = plan_gemm(M, N, K, num_cus, first_cfg);
    return p.splits > 1 ? (size_t)p.splits * (size_t)M * (size_t)N * 4 : 0;
}

// Returns true when the low-rank branch `lr` (if any) was added in the epilogue.
// k_gemm_mfma addresses one tile's rows with 32-bit buffer offsets
template <int AM>
static bool mfma_fits(int64_t BM, int64_t BN, int64_t K, int64_t lda) {
    const int64_t lim = (int64_t)1 << 31;
    const int64_t a_row_bytes = (AM == kAmBf16 || AM == kAmQuant) ? lda * 2 : AM == kAmNvfp4 ? K / 2 : lda;
    return (BM + 1) * a_row_bytes + K * 2 < lim && BN * (K / 2) < lim;
}

template <int BM, int BN, int WM, int WN, int AM>
static bool launch_tile(const GemmA &a, int64_t M, const nvfp4_tensor *w, float *c, int64_t ldc,
                        const GemmPlan &plan, float *partials, const LrArgs *lr, hipStream_t stream,
                        const QaPre *pre = nullptr) {
    const int64_t N = w->rows, K = w->cols;
    const int64_t tiles = ((M + BM - 1) / BM) * ((N + BN - 1) / BN);
    const int64_t lda = a.lda;
    const bool fits = mfma_fits<AM>(BM, BN, K, lda);
    if constexpr (AM == kAmNvfp4) {
        if (pre) {  // staged quantization (checked to apply: K % 64 == 0, fits)
            if (partials) {
                hipLaunchKernelGGL((k_gemm_mfma<BM, BN, WM, WN, AM, false, true>),
                                   dim3((unsigned)tiles, (unsigned)plan.splits), dim3(64 * WM * WN), 0, stream,
                                   (const __bf16 *)nullptr, lda, a.codes, a.scales, a.g, w->codes, w->scales, nullptr,
                                   partials, N, M, N, K, plan.slice_steps, LrArgs{}, *pre);
                const int64_t total = M * N;
                const int64_t blocks = (total + 255) / 256 < 65536 ? (total + 255) / 256 : 65536;
                hipLaunchKernelGGL((k_splitk_reduce<2>), dim3((unsigned)blocks), dim3(256), 0, stream, partials,
                                   plan.splits, M, N, N, a.g, w->global_scale, c, ldc);
            } else {
                hipLaunchKernelGGL((k_gemm_mfma<BM, BN, WM, WN, AM, false, true>), dim3((unsigned)tiles),
                                   dim3(64 * WM * WN), 0, stream, (const __bf16 *)nullptr, lda, a.codes, a.scales,
                                   a.g, w->codes, w->scales, w->global_scale, c, ldc, M, N, K, (int)(K / kBK),
                                   LrArgs{}, *pre);
            }
            return false;
        }
    }
    if (K % kBK == 0 && fits) {
        if (partials) {
            // K slices into their own planes of the workspace, then the ordered sum and scaling
            hipLaunchKernelGGL((k_gemm_mfma<BM, BN, WM, WN, AM>), dim3((unsigned)tiles, (unsigned)plan.splits),
                               dim3(64 * WM * WN), 0, stream, (const __bf16 *)a.bf16, lda, a.codes, a.scales, a.g,
                               w->codes, w->scales, nullptr, partials, N, M, N, K, plan.slice_steps, LrArgs{}, QaPre{});
            const int64_t total = M * N;
            const int64_t blocks = (total + 255) / 256 < 65536 ? (total + 255) / 256 : 65536;
            hipLaunchKernelGGL((k_splitk_reduce<AM == kAmBf16 ? 0 : AM == kAmQuant ? 2 : 1>), dim3((unsigned)blocks),
                               dim3(256), 0, stream,
                               partials, plan.splits, M, N, N, a.g, w->global_scale, c, ldc);
            return false;
        }
        if (lr) {
            if constexpr (AM == kAmBf16 || AM == kAmNvfp4) {
                hipLaunchKernelGGL((k_gemm_mfma<BM, BN, WM, WN, AM, true>), dim3((unsigned)tiles), dim3(64 * WM * WN),
                                   0, stream, (const __bf16 *)a.bf16, lda, a.codes, a.scales, a.g, w->codes,
                                   w->scales, w->global_scale, c, ldc, M, N, K, (int)(K / kBK), *lr, QaPre{});
                return true;
            }
        }
        hipLaunchKernelGGL((k_gemm_mfma<BM, BN, WM, WN, AM>), dim3((unsigned)tiles), dim3(64 * WM * WN), 0, stream,
                           (const __bf16 *)a.bf16, lda, a.codes, a.scales, a.g, w->codes, w->scales,
                           w->global_scale, c, ldc, M, N, K, (int)(K / kBK), LrArgs{}, QaPre{});
    } else if constexpr (AM != kAmQuant) {  // the fused quantization runs only where K % 64 == 0
        hipLaunchKernelGGL((k_gemm_tile<BM, BN, WM, WN, AM>), dim3((unsigned)tiles), dim3(64 * WM * WN), 0, stream,
                           (const __bf16 *)a.bf16, lda, a.codes, a.scales, a.g, w->codes, w->scales,
                           w->global_scale, c, ldc, M, N, K);
    }
    return false;
}

// Tiles with 256 rows hold the quantizing A path's extra registers only by spilling: that form
// plans over the 128-row shapes.
template <int AM>
constexpr int first_tile_cfg() { return AM == kAmQuant ? kFirstQuantTileCfg : 0; }

template <int AM>
static bool launch_tiled(const GemmA &a, int64_t M, const nvfp4_tensor *w, float *c, int64_t ldc, void *workspace,
                         size_t workspace_bytes, int num_cus, hipStream_t stream, const LrArgs *lr = nullptr,
                         const QaPre *pre = nullptr) {
    GemmPlan plan = plan_gemm(M, w->rows, w->cols, num_cus, first_tile_cfg<AM>());
    float *partials = nullptr;
    if (plan.splits > 1) {
        // split-K needs its partial planes; without room for them the product runs unsplit
        if (workspace && workspace_bytes >= (size_t)plan.splits * (size_t)M * (size_t)w->rows * 4)
            partials = reinterpret_cast<float *>(workspace);
        else
            plan = GemmPlan{plan.cfg, 1, (int)(w->cols / kBK)};
    }
    if constexpr (first_tile_cfg<AM>() == 0) {
        if (plan.cfg == 0) return launch_tile<256, 256, 4, 2, AM>(a, M, w, c, ldc, plan, partials, lr, stream, pre);
        if (plan.cfg == 1) return launch_tile<256, 192, 4, 2, AM>(a, M, w, c, ldc, plan, partials, lr, stream, pre);
    }
    if (plan.cfg == 4) return launch_tile<128, 192, 4, 2, AM>(a, M, w, c, ldc, plan, partials, lr, stream, pre);
    if (plan.cfg == 2) return launch_tile<128, 256, 2, 4, AM>(a, M, w, c, ldc, plan, partials, lr, stream, pre);
    return launch_tile<128, 128, 2, 2, AM>(a, M, w, c, ldc, plan, partials, lr, stream, pre);
}

hipError_t launch_gemm(const void *a_bf16, const nvfp4_tensor *a_q, int64_t M, int64_t lda, const nvfp4_tensor *w,
                       float *c, int64_t ldc, void *workspace, size_t workspace_bytes, int num_cus,
                       hipStream_t stream) {
    const int64_t K = w->cols;
    if (M == 0 || w->rows == 0) return hipGetLastError();
    if (a_q) {
        const GemmA a{nullptr, a_q->codes, a_q->scales, a_q->global_scale, K};
        if (gemv_applies(M, K)) launch_gemv<kAmNvfp4>(M, a, w, c, ldc, num_cus, stream);
        else launch_tiled<kAmNvfp4>(a, M, w, c, ldc, workspace, workspace_bytes, num_cus, stream);
    } else {
        const GemmA a{a_bf16, nullptr, nullptr, nullptr, lda};
        if (gemv_applies(M, K)) launch_gemv<kAmBf16>(M, a, w, c, ldc, num_cus, stream);
        else launch_tiled<kAmBf16>(a, M, w, c, ldc, workspace, workspace_bytes, num_cus, stream);
    }
    return hipGetLastError();
}

hipError_t launch_gemm_lowrank(const void *a_bf16, const nvfp4_tensor *a_q, int64_t M, int64_t lda,
                               const nvfp4_tensor *w, const void *v, const void *u, int r, float *c, int64_t ldc,
                               void *workspace, size_t workspace_bytes, int num_cus, hipStream_t stream) {
    const int64_t N = w->rows, K = w->cols;
    if (M == 0 || N == 0) return hipGetLastError();
    // T_hi, T_lo at the front of the workspace; the rest holds the product's split-K planes
    const size_t tb = lowrank_t_bytes(M);
    uint8_t *ws = reinterpret_cast<uint8_t *>(workspace);
    hipError_t e = launch_lowrank_down(a_bf16, lda, v, M, K, r, ws, stream);
    if (e != hipSuccess) return e;
    const LrArgs lr{reinterpret_cast<const __bf16 *>(ws), reinterpret_cast<const __bf16 *>(u), r};
    bool fused = false;
    if (K == 0) {
        e = launch_fill_zero_f32(c, M, N, ldc, stream);
        if (e != hipSuccess) return e;
    } else if (gemv_applies(M, K)) {
        if (a_q) launch_gemv<kAmNvfp4>(M, GemmA{nullptr, a_q->codes, a_q->scales, a_q->global_scale, K}, w, c, ldc,
                                       num_cus, stream);
        else launch_gemv<kAmBf16>(M, GemmA{a_bf16, nullptr, nullptr, nullptr, lda}, w, c, ldc, num_cus, stream);
    } else if (a_q) {
        const GemmA a{nullptr, a_q->codes, a_q->scales, a_q->global_scale, K};
        fused = launch_tiled<kAmNvfp4>(a, M, w, c, ldc, ws + tb, workspace_bytes - tb, num_cus, stream, &lr);
    } else {
        const GemmA a{a_bf16, nullptr, nullptr, nullptr, lda};
        fused = launch_tiled<kAmBf16>(a, M, w, c, ldc, ws + tb, workspace_bytes - tb, num_cus, stream, &lr);
    }
    if (!fused) return launch_lowrank_up_add(ws, u, r, M, N, c, ldc, stream);
    return hipGetLastError();
}

// Whether the product with activations quantized in the kernel can run fused: the tiled kernel
// with K % 64 == 0 and 32-bit tile offsets.  Elsewhere the caller quantizes into the workspace
// first.
bool gemm_qa_fusable(int64_t M, int64_t K, int64_t lda) {
    if (M <= 0 || K <= 0 || K % kBK != 0 || gemv_applies(M, K)) return false;
    return (int64_t)(256 + 1) * lda * 2 + K * 2 < ((int64_t)1 << 31);
}

hipError_t launch_gemm_qa_fused(const void *a_bf16, const float *amax, int64_t M, int64_t lda, const nvfp4_tensor *w,
                                float *c, int64_t ldc, void *workspace, size_t workspace_bytes, int num_cus,
                                hipStream_t stream) {
    const GemmA a{a_bf16, nullptr, nullptr, amax, lda};
    launch_tiled<kAmQuant>(a, M, w, c, ldc, workspace, workspace_bytes, num_cus, stream);
    return hipGetLastError();
}

static size_t round256(size_t b) { return (b + 255) / 256 * 256; }

// Workgroups of the staged kernel of tile configuration `cfg` that one CU holds at once (queried
// from the runtime for the instantiation itself: registers and LDS decide it).
template <int BM, int BN, int WM, int WN>
static int staged_per_cu() {
    static std::atomic<int> cached{-1};
    int n = cached.load();
    if (n < 0) {
        if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, k_gemm_mfma<BM, BN, WM, WN, kAmNvfp4, false, true>,
                                                         64 * WM * WN, 0) != hipSuccess)
            n = 0;
        cached.store(n);
    }
    return n;
}

static int staged_per_cu(int cfg) {
    switch (cfg) {
    case 0: return staged_per_cu<256, 256, 4, 2>();
    case 1: return staged_per_cu<256, 192, 4, 2>();
    case 2: return staged_per_cu<128, 256, 2, 4>();
    case 3: return staged_per_cu<128, 128, 2, 2>();
    default: return staged_per_cu<128, 192, 4, 2>();
    }
}

bool gemm_qa_staged_applies(int64_t M, int64_t N, int64_t K, int64_t lda, int num_cus) {
    if (M <= 0 || N <= 0 || K <= 0 || K % kBK != 0 || gemv_applies(M, K) || num_cus <= 0) return false;
    const GemmPlan p = plan_gemm(M, N, K, num_cus, 0);
    const TileCfg &t = kTiles[p.cfg];
    const int64_t tiles_m = (M + t.bm - 1) / t.bm, tiles = tiles_m * ((N + t.bn - 1) / t.bn);
    // one round of workgroups on the device (every group co-resident when nothing else runs), and
    // the group counters fit
    return tiles * p.splits <= (int64_t)num_cus * staged_per_cu(p.cfg) && tiles_m * p.splits <= kQaMaxGroups &&
           mfma_fits<kAmNvfp4>(t.bm, t.bn, K, K) && lda >= K;
}

size_t gemm_qa_staged_ws_bytes(int64_t M, int64_t N, int64_t K, int num_cus) {
    if (M <= 0 || K <= 0) return kQaSyncBytes;
    return kQaSyncBytes + round256((size_t)M * (size_t)(K / 2)) + round256((size_t)M * (size_t)(K / 16)) +
           gemm_ws_bytes(M, N, K, num_cus);
}

hipError_t launch_gemm_qa_staged(const void *a_bf16, const float *amax, int64_t M, int64_t lda, const nvfp4_tensor *w,
                                 float *c, int64_t ldc, void *workspace, size_t workspace_bytes, int num_cus,
                                 hipStream_t stream) {
    const int64_t K = w->cols;
    uint8_t *ws = reinterpret_cast<uint8_t *>(workspace);
    const size_t cb = round256((size_t)M * (size_t)(K / 2)), sb = round256((size_t)M * (size_t)(K / 16));
    // the wait's bound: about a second of polling; NVFP4_QA_SPIN_LIMIT overrides it (tests set it
    // tiny to run the fallback on every workgroup that finds its group incomplete)
    const char *env = getenv("NVFP4_QA_SPIN_LIMIT");
    const uint32_t spin_limit = env ? (uint32_t)strtoul(env, nullptr, 10) : (1u << 22);
    const QaPre pre{reinterpret_cast<const __bf16 *>(a_bf16), lda, amax, reinterpret_cast<uint32_t *>(ws),
                    ws + kQaSyncBytes, ws + kQaSyncBytes + cb, spin_limit};
    const GemmA a{nullptr, pre.codes, pre.scales, amax, K};
    const size_t head = kQaSyncBytes + cb + sb;
    launch_tiled<kAmNvfp4>(a, M, w, c, ldc, ws + head, workspace_bytes - head, num_cus, stream, nullptr, &pre);
    return hipGetLastError();
}

hipError_t launch_gemm_fp8(const uint8_t *a_fp8, const float *a_scale, int64_t M, int64_t lda, const nvfp4_tensor *w,
                           float *c, int64_t ldc, void *workspace, size_t workspace_bytes, int num_cus,
                           hipStream_t stream) {
    if (M == 0 || w->rows == 0) return hipGetLastError();
    const GemmA a{nullptr, a_fp8, nullptr, a_scale, lda};
    if (gemv_applies(M, w->cols)) launch_gemv<kAmFp8>(M, a, w, c, ldc, num_cus, stream);
    else launch_tiled<kAmFp8>(a, M, w, c, ldc, workspace, workspace_bytes, num_cus, stream);
    return hipGetLastError();
}

}  // namespace nvfp4
