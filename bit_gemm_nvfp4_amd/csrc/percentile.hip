// Percentile-amax calibration for gfx950: per channel, the nearest-rank p-th percentile and the
// maximum of |x| ("Qwen-Rapid-AIO-NVFP4", section "Recommended Model": p99.9 instead of max
// aggregation; "Qwen-Image NVFP4 on a 16 GB Ada GPU", section "Quality: the error of each matrix":
// nearest rank).
//
// Exact selection by radix on bit patterns: the magnitude bits of a float (sign cleared) order like
// its value, so the k-th smallest |x| is found digit by digit from the top.  Keys are 15 bits for
// bf16 / fp16 (two passes: 8 + 7 bits) and 31 bits for fp32 (four passes: 8 + 8 + 8 + 7 bits).
// Each pass:
//   k_pct_hist    histogram of the next digit over the elements whose higher digits match the
//                 channel's prefix: one workgroup per (64 channels, row chunk), LDS counters
//                 [digit][channel] merged into global counters with integer atomics (so the result
//                 does not depend on the order); the first pass also takes the per-channel
//                 maximum key;
//   k_pct_select  one wave per channel: a prefix sum over its counters picks the digit holding the
//                 remaining rank, narrows the prefix and clears the counters for the next pass;
//                 the last pass writes the results.
// When the rank sits within 16 of either end of a channel (p99.9 over a few thousand rows: the
// 5th largest of 4096), one pass suffices instead:
//   k_pct_topm        every lane keeps, per channel it owns, the M largest keys it has seen (a
//                     compare-exchange chain, branch-free), waves merge theirs through LDS, and each
//                     workgroup stores its list and maximum per channel; for a rank near the bottom
//                     the keys are complemented, so the same code keeps the smallest;
//   k_pct_topm_final  one thread per channel merges the workgroups' lists and picks the rank.
#include <hip/hip_runtime.h>

#include <cstdlib>

#include "common.h"
#include "internal.h"

namespace nvfp4 {

// Workspace layout (uint32 words), nch = cols (per channel) or 1:
//   [0, nch) prefix   [nch, 2 nch) remaining rank   [2 nch, 3 nch) max key   [3 nch, 3 nch + 256 nch) counters
// then, per channel (candidate path, per-channel only): candidate count, overflow mark, max key,
// fallback mark ([259 nch, 263 nch)), and the candidate lists [263 nch, 263 nch + kCandCap nch).
constexpr int kCandCap = 2048;       // candidates kept per channel
constexpr int kSampleStride = 16;    // every 16th row forms the sample that sets the threshold
constexpr int64_t kCandMinRows = 32768;

size_t percentile_ws_min_bytes(int64_t cols, int per_channel) {
    const int64_t nch = per_channel ? cols : 1;
    return (size_t)nch * (3 + 256) * 4;
}

size_t percentile_ws_bytes(int64_t cols, int per_channel) {
    if (!per_channel) return percentile_ws_min_bytes(cols, per_channel);
    return (size_t)cols * (3 + 256 + 4 + kCandCap) * 4;
}

// Zero the first `words` words, except the remaining ranks, which start at k.
__global__ void k_pct_init(uint32_t *ws, int64_t nch, uint32_t k, int64_t words) {
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < words; i += (int64_t)gridDim.x * blockDim.x)
        ws[i] = (i >= nch && i < 2 * nch) ? k : 0u;
}

// One workgroup of 8 waves per (256 channels, row chunk).  Every lane loads 16 bytes of a row (8 bf16 /
// fp16 or 4 fp32 channels), so one wave load covers whole 512-byte (bf16) or 1 KB (fp32) row segments:
// wide enough for the DRAM pages, where 64-channel strips of a 6 KB row read at about 2.8 TB/s.
// U rows are in flight per lane (rows past the chunk are masked).  Counters live in LDS as 16-bit
// halves of [digit][channel] words (128 KB; a chunk has at most 65535 rows, so no half overflows),
// which also halves the lanes that add into one bank.  DT: NVFP4_F32 (31-bit keys), NVFP4_BF16 or
// NVFP4_F16 (15-bit keys).
constexpr int kPctThreads = 512;
constexpr int kPctChannels = 256;   // channels per workgroup of the histogram pass
constexpr int kPctMaxRowsPerWg = 65535;

template <int DT, int U>
__global__ __launch_bounds__(kPctThreads) void k_pct_hist(const uint8_t *__restrict__ x, int64_t rows, int64_t cols,
                                                          int64_t ld_bytes, int per_channel, int rows_per_wg,
                                                          int shift, int dbits, int first_pass,
                                                          uint32_t *__restrict__ ws, const uint32_t *__restrict__ only) {
    constexpr int EPL = (DT == NVFP4_F32) ? 4 : 8;  // channels per lane (one 16-byte load)
    constexpr int WCH = kPctChannels;
    constexpr int LPR = WCH / EPL;                   // lanes per row segment of the workgroup's channels
    constexpr int RPW = 64 / LPR;                    // rows per wave load
    static_assert(LPR <= 64 && 64 % LPR == 0, "a wave covers whole row segments");
    constexpr int NW = kPctThreads / 64;
    constexpr int STEP = NW * RPW;                   // rows per workgroup load step
    __shared__ uint32_t hist[256 * WCH / 2];         // two 16-bit counters per word
    const int64_t nch = per_channel ? cols : 1;
    uint32_t *prefix = ws, *maxkey = ws + 2 * nch, *ghist = ws + 3 * nch;

    const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
    const int64_t c0 = (int64_t)blockIdx.x * WCH;
    if (only) {  // only the marked channels are wanted: a workgroup with none of them has nothing to do
        const bool mine = tid < WCH && c0 + tid < cols && only[c0 + tid] != 0u;
        if (!__syncthreads_or(mine)) return;
    }
    for (int i = tid; i < 256 * WCH / 8; i += kPctThreads) reinterpret_cast<u32x4 *>(hist)[i] = u32x4{0u, 0u, 0u, 0u};

    const int64_t r0 = (int64_t)blockIdx.y * rows_per_wg;
    const int64_t r1 = (r0 + rows_per_wg) < rows ? (r0 + rows_per_wg) : rows;
    const int lc = (lane % LPR) * EPL;  // first local channel of this lane
    const int64_t cl = c0 + lc;
    const bool active = cl < cols;      // cols % 16 == 0: a lane's channels are all in or all out
    uint32_t pre[EPL], mk[EPL];
#pragma unroll
    for (int j = 0; j < EPL; j++) {
        pre[j] = (active && !first_pass) ? prefix[per_channel ? cl + j : 0] : 0u;
        mk[j] = 0u;
    }
    const uint32_t dmask = (1u << dbits) - 1u;
    const int hs = shift + dbits;  // bits above the current digit
    __syncthreads();

    auto account = [&](const u32x4 &v) {
        uint32_t key[EPL];
        if constexpr (DT == NVFP4_F32) {
#pragma unroll
            for (int j = 0; j < 4; j++) key[j] = v[j] & 0x7FFFFFFFu;
        } else {
#pragma unroll
            for (int j = 0; j < 4; j++) {
                key[2 * j] = v[j] & 0x7FFFu;
                key[2 * j + 1] = (v[j] >> 16) & 0x7FFFu;
            }
        }
#pragma unroll
        for (int j = 0; j < EPL; j++) {
            if (first_pass) mk[j] = max(mk[j], key[j]);
            if ((key[j] >> hs) == pre[j]) {
                const int i = (int)((key[j] >> shift) & dmask) * WCH + lc + j;
                atomicAdd(&hist[i >> 1], 1u << ((i & 1) * 16));
            }
        }
    };
    if (active) {
        const uint8_t *base = x + cl * (DT == NVFP4_F32 ? 4 : 2);
        int64_t r = r0 + wid * RPW + lane / LPR;
        for (; r + (int64_t)(U - 1) * STEP < r1; r += (int64_t)U * STEP) {  // full batches
            u32x4 v[U];
#pragma unroll
            for (int u = 0; u < U; u++) v[u] = *reinterpret_cast<const u32x4 *>(base + (r + (int64_t)u * STEP) * ld_bytes);
#pragma unroll
            for (int u = 0; u < U; u++) account(v[u]);
        }
        if (r < r1) {  // last, partial batch: rows past the chunk are masked
            u32x4 v[U];
#pragma unroll
            for (int u = 0; u < U; u++) {
                const int64_t rr = r + (int64_t)u * STEP;
                v[u] = rr < r1 ? *reinterpret_cast<const u32x4 *>(base + rr * ld_bytes) : u32x4{0u, 0u, 0u, 0u};
            }
#pragma unroll
            for (int u = 0; u < U; u++)
                if (r + (int64_t)u * STEP < r1) account(v[u]);
        }
        if (first_pass) {
#pragma unroll
            for (int j = 0; j < EPL; j++) atomicMax(&maxkey[per_channel ? cl + j : 0], mk[j]);
        }
    }
    __syncthreads();
    const int nbins = 1 << dbits;
    auto count = [&](int i) { return (hist[i >> 1] >> ((i & 1) * 16)) & 0xFFFFu; };
    if (per_channel) {
        for (int i = tid; i < nbins * WCH; i += kPctThreads) {
            const uint32_t cnt = count(i);
            const int64_t ch = c0 + (i % WCH);
            if (cnt && ch < cols) atomicAdd(&ghist[ch * 256 + i / WCH], cnt);
        }
    } else {
        // the whole tensor is one channel: add up the local channels of each bin first (each lane
        // starts at its own channel, so the lanes of a wave read different banks)
        for (int b = tid; b < nbins; b += kPctThreads) {
            uint32_t cnt = 0;
            for (int c = 0; c < WCH; c++) cnt += count(b * WCH + ((c + b) & (WCH - 1)));
            if (cnt) atomicAdd(&ghist[b], cnt);
        }
    }
}

// One wave per channel: a prefix sum over the 2^d counters (4 per lane) finds the digit that holds
// the remaining rank; the counters are cleared for the next pass.  last: write key -> value of the
// selected element and of the maximum.
template <int DT>
__global__ __launch_bounds__(256) void k_pct_select(uint32_t *__restrict__ ws, int64_t nch, int dbits, int last,
                                                    float *__restrict__ out_pct, float *__restrict__ out_max,
                                                    int32_t *__restrict__ flags, const uint32_t *__restrict__ only) {
    const int64_t ch = ((int64_t)blockIdx.x * blockDim.x + threadIdx.x) >> 6;
    const int lane = threadIdx.x & 63;
    if (ch >= nch || (only && only[ch] == 0u)) return;
    uint32_t *prefix = ws, *krem = ws + nch, *maxkey = ws + 2 * nch, *h = ws + 3 * nch + ch * 256;
    const int nbins = 1 << dbits;
    uint32_t c[4];
#pragma unroll
    for (int j = 0; j < 4; j++) c[j] = (4 * lane + j < nbins) ? h[4 * lane + j] : 0u;
    const uint32_t mine = c[0] + c[1] + c[2] + c[3];
    uint32_t incl = mine;  // inclusive scan over lanes
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
        const uint32_t t = (uint32_t)__shfl_up((int)incl, o, 64);
        if (lane >= o) incl += t;
    }
    const uint32_t need = krem[ch];
    const uint32_t excl = incl - mine;
    const bool here = (excl < need) && (incl >= need);
    const uint64_t hit = __ballot(here);
    const int src = hit ? __builtin_ctzll(hit) : 63;
    int d = 4 * lane + 3;
    uint32_t before = excl;
    if (here) {
        uint32_t cum = excl;
#pragma unroll
        for (int j = 0; j < 4; j++) {
            if (cum + c[j] >= need) {
                d = 4 * lane + j;
                break;
            }
            cum += c[j];
        }
        before = cum;
    }
    d = __shfl(d, src, 64);
    before = (uint32_t)__shfl((int)before, src, 64);
#pragma unroll
    for (int j = 0; j < 4; j++)
        if (4 * lane + j < nbins) h[4 * lane + j] = 0u;
    if (lane == 0) {
        const uint32_t p = (prefix[ch] << dbits) | (uint32_t)d;
        prefix[ch] = p;
        krem[ch] = need - before;
        if (last) {
            auto to_f32 = [](uint32_t key) -> float {
                if (DT == NVFP4_F32) return u2f(key);
                if (DT == NVFP4_BF16) return u2f(key << 16);
                return (float)__builtin_bit_cast(_Float16, (uint16_t)key);
            };
            const uint32_t mk = maxkey[ch];
            const uint32_t inf_key = (DT == NVFP4_F32) ? 0x7F800000u : (DT == NVFP4_BF16 ? 0x7F80u : 0x7C00u);
            if (mk >= inf_key && flags) atomicOr(flags, 1);
            if (out_pct) out_pct[ch] = to_f32(p);
            if (out_max) out_max[ch] = to_f32(mk);
        }
    }
}


// ---------------------------------------------------------------------------------------------
// Candidate selection for ranks a little further from an end (per channel).
// ---------------------------------------------------------------------------------------------
// A sample (every kSampleStride-th row) gives, per channel, a threshold key T a safe distance past
// the wanted rank (the radix selection above, run on the sample).  One pass over all rows then
// keeps the keys on the far side of T (key >= T when the rank counts from the top, key <= T from
// the bottom) in a per-channel list, counts them and takes the maximum; the rank is selected among
// the candidates.  A channel whose list overflowed, or whose candidates are fewer than the rank (T
// fell short), is marked and goes through the exact radix passes over all rows.  Keys are oriented
// so that the wanted side is the large side: okey = key (top) or mask - key (bottom).
constexpr int kCandLds = 112;  // candidates per channel one workgroup holds in LDS (112 KB)

template <int DT, int U, bool TOP>
__global__ __launch_bounds__(kPctThreads) void k_pct_cand(const uint8_t *__restrict__ x, int64_t rows, int64_t cols,
                                                          int64_t ld_bytes, int rows_per_wg, int cap,
                                                          uint32_t *__restrict__ ws) {
    constexpr int EPL = (DT == NVFP4_F32) ? 4 : 8;
    constexpr int WCH = kPctChannels;
    constexpr int LPR = WCH / EPL;
    constexpr int RPW = 64 / LPR;
    constexpr int NW = kPctThreads / 64;
    constexpr int STEP = NW * RPW;
    constexpr uint32_t MASK = (DT == NVFP4_F32) ? 0x7FFFFFFFu : 0x7FFFu;
    __shared__ uint32_t lcount[WCH];
    __shared__ uint32_t llist[WCH * kCandLds];
    const int64_t nch = cols;
    const uint32_t *thr = ws + 262 * nch;  // the sample's threshold keys (the fallback marks' words, until set)
    uint32_t *gcnt = ws + 259 * nch, *ovf = gcnt + nch, *gmax = ovf + nch;
    uint32_t *glist = ws + 263 * nch;

    const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
    for (int i = tid; i < WCH; i += kPctThreads) lcount[i] = 0u;
    const int64_t c0 = (int64_t)blockIdx.x * WCH;
    const int64_t r0 = (int64_t)blockIdx.y * rows_per_wg;
    const int64_t r1 = (r0 + rows_per_wg) < rows ? (r0 + rows_per_wg) : rows;
    const int lc = (lane % LPR) * EPL;
    const int64_t cl = c0 + lc;
    const bool active = cl < cols;
    uint32_t t[EPL], mk[EPL];
#pragma unroll
    for (int j = 0; j < EPL; j++) {
        const uint32_t raw = active ? thr[cl + j] : MASK;
        t[j] = TOP ? raw : MASK - raw;
        mk[j] = 0u;
    }
    __syncthreads();
    auto account = [&](const u32x4 &v) {
        uint32_t key[EPL];
        if constexpr (DT == NVFP4_F32) {
#pragma unroll
            for (int j = 0; j < 4; j++) key[j] = v[j] & 0x7FFFFFFFu;
        } else {
#pragma unroll
            for (int j = 0; j < 4; j++) {
                key[2 * j] = v[j] & 0x7FFFu;
                key[2 * j + 1] = (v[j] >> 16) & 0x7FFFu;
            }
        }
        uint32_t ok[EPL], hit = 0u;
#pragma unroll
        for (int j = 0; j < EPL; j++) {
            mk[j] = max(mk[j], key[j]);
            ok[j] = TOP ? key[j] : MASK - key[j];
            hit |= (ok[j] >= t[j] ? 1u : 0u) << j;
        }
        if (hit) {  // rare: one branch per load for all of the lane's channels
#pragma unroll
            for (int j = 0; j < EPL; j++) {
                // past kCandLds + 1 the channel has overflowed whatever follows: stop counting
                if (((hit >> j) & 1u) && lcount[lc + j] <= (uint32_t)kCandLds) {
                    const uint32_t slot = atomicAdd(&lcount[lc + j], 1u);
                    if (slot < (uint32_t)kCandLds) llist[(lc + j) * kCandLds + slot] = ok[j];
                }
            }
        }
    };
    if (active) {
        const uint8_t *base = x + cl * (DT == NVFP4_F32 ? 4 : 2);
        int64_t r = r0 + wid * RPW + lane / LPR;
        for (; r + (int64_t)(U - 1) * STEP < r1; r += (int64_t)U * STEP) {
            u32x4 v[U];
#pragma unroll
            for (int u = 0; u < U; u++) v[u] = *reinterpret_cast<const u32x4 *>(base + (r + (int64_t)u * STEP) * ld_bytes);
#pragma unroll
            for (int u = 0; u < U; u++) account(v[u]);
        }
        if (r < r1) {
            u32x4 v[U];
#pragma unroll
            for (int u = 0; u < U; u++) {
                const int64_t rr = r + (int64_t)u * STEP;
                v[u] = rr < r1 ? *reinterpret_cast<const u32x4 *>(base + rr * ld_bytes) : u32x4{0u, 0u, 0u, 0u};
            }
#pragma unroll
            for (int u = 0; u < U; u++)
                if (r + (int64_t)u * STEP < r1) account(v[u]);
        }
#pragma unroll
        for (int j = 0; j < EPL; j++) atomicMax(&gmax[cl + j], mk[j]);
    }
    __syncthreads();
    // one thread per channel moves the workgroup's candidates to the channel's list
    for (int i = tid; i < WCH; i += kPctThreads) {
        const int64_t ch = c0 + i;
        const uint32_t n = lcount[i];
        if (ch >= cols || n == 0) continue;
        const uint32_t base = atomicAdd(&gcnt[ch], n);
        if (n > (uint32_t)kCandLds || base + n > (uint32_t)cap) {
            atomicOr(&ovf[ch], 1u);
            continue;
        }
        for (uint32_t q = 0; q < n; q++) glist[ch * kCandCap + base + q] = llist[i * kCandLds + q];
    }
}

// One workgroup per channel: the need-th largest oriented key among the channel's candidates, by
// radix selection in LDS; or, when the candidates cannot hold it, the fallback mark (and the radix
// state of the channel reset for the exact passes).  need: the rank counted from the wanted end.
template <int DT>
__global__ __launch_bounds__(64) void k_pct_cand_select(uint32_t *__restrict__ ws, int64_t nch, uint32_t need,
                                                         uint32_t k, int top, int cap, float *__restrict__ out_pct,
                                                         float *__restrict__ out_max, int32_t *__restrict__ flags) {
    constexpr int KEYBITS = (DT == NVFP4_F32) ? 31 : 15;
    constexpr uint32_t MASK = (DT == NVFP4_F32) ? 0x7FFFFFFFu : 0x7FFFu;
    __shared__ uint32_t keys[kCandCap];
    __shared__ uint32_t hist[256];
    __shared__ uint32_t sel_prefix, sel_need;
    const int64_t ch = blockIdx.x;
    const int tid = threadIdx.x;
    uint32_t *prefix = ws, *krem = ws + nch, *maxkey = ws + 2 * nch;
    uint32_t *gcnt = ws + 259 * nch, *ovf = gcnt + nch, *gmax = ovf + nch, *fb = gmax + nch;
    const uint32_t *glist = ws + 263 * nch + ch * kCandCap;
    const uint32_t c = gcnt[ch];
    const bool bad = ovf[ch] != 0u || c < need || c > (uint32_t)cap;
    // radix state of this channel for the exact passes (its counters held the sample's lists); the
    // threshold word becomes the fallback mark
#pragma unroll
    for (int i = 0; i < 4; i++) ws[3 * nch + ch * 256 + 64 * i + tid] = 0u;
    if (tid == 0) {
        fb[ch] = bad ? 1u : 0u;
        prefix[ch] = 0u;
        krem[ch] = k;
        maxkey[ch] = 0u;
    }
    if (bad) return;
    for (uint32_t i = tid; i < c; i += 64) keys[i] = glist[i];
    if (tid == 0) {
        sel_prefix = 0u;
        sel_need = need;
    }
    __syncthreads();
    int consumed = 0;
    while (consumed < KEYBITS) {
        const int dbits = (KEYBITS - consumed) >= 8 ? 8 : (KEYBITS - consumed);
        const int shift = KEYBITS - consumed - dbits;
        const int hs = shift + dbits;
#pragma unroll
        for (int i = 0; i < 4; i++) hist[64 * i + tid] = 0u;
        __syncthreads();
        const uint32_t pfx = sel_prefix;
        for (uint32_t i = tid; i < c; i += 64) {
            const uint32_t kk = keys[i];
            if ((kk >> hs) == pfx) atomicAdd(&hist[(kk >> shift) & ((1u << dbits) - 1u)], 1u);
        }
        __syncthreads();
        if (tid < 64) {
            // from the largest digit down: lane l holds digits top - 4 l .. top - 4 l - 3; an inclusive
            // scan over the lanes finds the digit holding the need-th largest
            const int nb = 1 << dbits, lane = tid;
            uint32_t c4[4], mine = 0;
#pragma unroll
            for (int j = 0; j < 4; j++) {
                const int d = nb - 1 - (4 * lane + j);
                c4[j] = d >= 0 ? hist[d] : 0u;
                mine += c4[j];
            }
            uint32_t incl = mine;
#pragma unroll
            for (int o = 1; o < 64; o <<= 1) {
                const uint32_t t2 = (uint32_t)__shfl_up((int)incl, o, 64);
                if (lane >= o) incl += t2;
            }
            const uint32_t nd = sel_need, excl = incl - mine;
            const bool here = excl < nd && incl >= nd;
            if (here) {
                uint32_t cum = excl;
                int j = 0;
                for (; j < 3; j++) {
                    if (cum + c4[j] >= nd) break;
                    cum += c4[j];
                }
                sel_prefix = (pfx << dbits) | (uint32_t)(nb - 1 - (4 * lane + j));
                sel_need = nd - cum;
            }
        }
        __syncthreads();
        consumed += dbits;
    }
    if (tid == 0) {
        auto to_f32 = [](uint32_t key) -> float {
            if (DT == NVFP4_F32) return u2f(key);
            if (DT == NVFP4_BF16) return u2f(key << 16);
            return (float)__builtin_bit_cast(_Float16, (uint16_t)key);
        };
        const uint32_t key = top ? sel_prefix : MASK - sel_prefix;
        const uint32_t mk = gmax[ch];
        const uint32_t inf_key = (DT == NVFP4_F32) ? 0x7F800000u : (DT == NVFP4_BF16 ? 0x7F80u : 0x7C00u);
        if (mk >= inf_key && flags) atomicOr(flags, 1);
        out_pct[ch] = to_f32(key);
        if (out_max) out_max[ch] = to_f32(mk);
    }
}

// ---------------------------------------------------------------------------------------------
// One-pass selection near either end of each channel.
// ---------------------------------------------------------------------------------------------
// Workspace per channel (uint32 words, at most 259 of them): rchunks lists of M keys, then
// rchunks maxima.
constexpr int kTopmMax = 16;

// Packed pair of 16-bit keys (bf16 / fp16 magnitudes, one channel per half) or one 31-bit key.
template <bool H>
__device__ __forceinline__ uint32_t key_max(uint32_t a, uint32_t b) {
    if constexpr (H) {
        typedef unsigned short u16x2 __attribute__((ext_vector_type(2)));
        return __builtin_bit_cast(uint32_t, __builtin_elementwise_max(__builtin_bit_cast(u16x2, a), __builtin_bit_cast(u16x2, b)));
    } else {
        return a > b ? a : b;
    }
}
template <bool H>
__device__ __forceinline__ uint32_t key_min(uint32_t a, uint32_t b) {
    if constexpr (H) {
        typedef unsigned short u16x2 __attribute__((ext_vector_type(2)));
        return __builtin_bit_cast(uint32_t, __builtin_elementwise_min(__builtin_bit_cast(u16x2, a), __builtin_bit_cast(u16x2, b)));
    } else {
        return a < b ? a : b;
    }
}
// Insert key k into the descending list L[0..M): each step keeps the larger and passes the smaller on.
template <bool H, int M>
__device__ __forceinline__ void topm_insert(uint32_t (&L)[M], uint32_t k) {
#pragma unroll
    for (int i = 0; i < M; i++) {
        const uint32_t hi = key_max<H>(L[i], k);
        k = key_min<H>(L[i], k);
        L[i] = hi;
    }
}

// One workgroup per (64 * CPL channels, row chunk); lane l owns CPL consecutive channels (one 8-byte
// load per row: four bf16 / fp16 or two fp32, kept as two words of packed or single keys), the
// eight waves take every eighth row, two batches of U rows in flight per lane.  Keys are the
// magnitude bits, XOR-complemented when `invert` (then the lists hold the smallest originals).
// The waves' lists are then merged pairwise through LDS in three rounds.
constexpr int kTopmWaves = 8;
constexpr int kTopmU = 4;

template <int DT, int M>
__global__ __launch_bounds__(64 * kTopmWaves) void k_pct_topm(const uint8_t *__restrict__ x, int64_t rows,
                                                             int64_t cols, int64_t ld_bytes, int rows_per_wg,
                                                             int invert, int rchunks, uint32_t *__restrict__ ws) {
    constexpr bool H = DT != NVFP4_F32;
    constexpr int CPL = H ? 4 : 2;  // channels per lane
    constexpr int CPW = H ? 2 : 1;  // channels per word
    constexpr int U = kTopmU;
    constexpr int NW = kTopmWaves;
    __shared__ uint32_t lst[NW / 2][M + 1][2][64];
    const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
    const int64_t c0 = ((int64_t)blockIdx.x * 64 + lane) * CPL;
    const bool active = c0 < cols;  // cols % 16 == 0: all channels of a lane are in or out
    const int64_t r0 = (int64_t)blockIdx.y * rows_per_wg;
    const int64_t r1 = (r0 + rows_per_wg) < rows ? (r0 + rows_per_wg) : rows;
    const uint32_t mask = H ? 0x7FFF7FFFu : 0x7FFFFFFFu;
    const uint32_t flip = invert ? mask : 0u;
    // the chunk's rows only: loads past its last row read zero
    const __amdgpu_buffer_rsrc_t rsrc = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint8_t *>(x + r0 * ld_bytes), (short)0, (int)((r1 - r0) * ld_bytes), 0x00020000);
    const uint32_t col_off = (uint32_t)(c0 * (H ? 2 : 4));
    uint32_t L[2][M], mx[2] = {0u, 0u};
#pragma unroll
    for (int i = 0; i < M; i++) L[0][i] = L[1][i] = 0u;
    auto load = [&](int64_t r, u32x2 (&v)[U]) {
#pragma unroll
        for (int u = 0; u < U; u++)
            v[u] = __builtin_amdgcn_raw_buffer_load_b64(rsrc, (uint32_t)((r - r0 + NW * u) * ld_bytes) + col_off, 0, 0);
    };
    // rows past the chunk enter the lists as key 0, which sorts last and never displaces a real
    // key, and the maxima as 0
    auto account = [&](int64_t r, const u32x2 (&v)[U]) {
#pragma unroll
        for (int u = 0; u < U; u++) {
            const uint32_t okm = (r + NW * u < r1) ? 0xFFFFFFFFu : 0u;
#pragma unroll
            for (int h = 0; h < 2; h++) {
                const uint32_t k = v[u][h] & mask;
                mx[h] = key_max<H>(mx[h], k);
                topm_insert<H, M>(L[h], (k ^ flip) & okm);
            }
        }
    };
    if (active) {
        u32x2 va[U], vb[U];
        int64_t r = r0 + wid;
        load(r, va);
        for (; r < r1; r += 2 * NW * U) {
            load(r + NW * U, vb);
            account(r, va);
            if (r + NW * U >= r1) break;
            load(r + 2 * NW * U, va);
            account(r + NW * U, vb);
        }
    }
    for (int half = NW / 2; half >= 1; half /= 2) {
        if (wid >= half && wid < 2 * half) {
#pragma unroll
            for (int h = 0; h < 2; h++) {
#pragma unroll
                for (int i = 0; i < M; i++) lst[wid - half][i][h][lane] = L[h][i];
                lst[wid - half][M][h][lane] = mx[h];
            }
        }
        __syncthreads();
        if (wid < half) {
#pragma unroll
            for (int h = 0; h < 2; h++) {
#pragma unroll
                for (int i = 0; i < M; i++) topm_insert<H, M>(L[h], lst[wid][i][h][lane]);
                mx[h] = key_max<H>(mx[h], lst[wid][M][h][lane]);
            }
        }
        __syncthreads();
    }
    if (wid != 0 || !active) return;
    const int64_t per_ch = (int64_t)rchunks * (M + 1);
#pragma unroll
    for (int h = 0; h < 2; h++) {
#pragma unroll
        for (int q = 0; q < CPW; q++) {
            uint32_t *p = ws + (c0 + h * CPW + q) * per_ch;
#pragma unroll
            for (int i = 0; i < M; i++) p[(int64_t)blockIdx.y * M + i] = H ? (L[h][i] >> (16 * q)) & 0xFFFFu : L[h][i];
            p[(int64_t)rchunks * M + blockIdx.y] = H ? (mx[h] >> (16 * q)) & 0xFFFFu : mx[h];
        }
    }
}

// One wave per channel: lane c holds workgroup c's descending list; m rounds each take the largest
// head across the lanes (the lowest such lane pops it); the m-th value taken is the rank sought.
// out_key not NULL: the m-th key of the lists' union is written there instead (a threshold: below or
// at the m-th of the rows the lists came from), and the channel's words clear[ch], clear[cols + ch]
// and clear[2 cols + ch] are zeroed.
template <int DT, int M>
__global__ __launch_bounds__(256) void k_pct_topm_final(const uint32_t *__restrict__ ws, int64_t cols, int rchunks,
                                                        int m, int invert, float *__restrict__ out_pct,
                                                        float *__restrict__ out_max, int32_t *__restrict__ flags,
                                                        uint32_t *__restrict__ out_key, uint32_t *__restrict__ clear) {
    const int64_t ch = ((int64_t)blockIdx.x * blockDim.x + threadIdx.x) >> 6;
    const int lane = threadIdx.x & 63;
    if (ch >= cols) return;
    const int64_t per_ch = (int64_t)rchunks * (M + 1);
    const uint32_t *p = ws + ch * per_ch;
    uint32_t L[M], mx = 0u;
#pragma unroll
    for (int i = 0; i < M; i++) L[i] = lane < rchunks ? p[lane * M + i] : 0u;
    if (lane < rchunks) mx = p[(int64_t)rchunks * M + lane];
    const uint32_t kmask = (DT == NVFP4_F32) ? 0x7FFFFFFFu : 0x7FFFu;
    if (out_key) {
        // the largest v with at least m keys >= v, bit by bit from the top
        constexpr int KB = (DT == NVFP4_F32) ? 31 : 15;
        uint32_t v = 0u;
        for (int b = KB - 1; b >= 0; b--) {
            const uint32_t c = v | (1u << b);
            uint32_t n = 0u;
#pragma unroll
            for (int i = 0; i < M; i++) n += L[i] >= c ? 1u : 0u;
            if (wave_sum_u32(n) >= (uint32_t)m) v = c;
        }
        if (lane == 0) {
            out_key[ch] = invert ? v ^ kmask : v;
            clear[ch] = 0u;
            clear[cols + ch] = 0u;
            clear[2 * cols + ch] = 0u;
        }
        return;
    }
    uint32_t key = 0u;
    for (int t = 0; t < m; t++) {
        key = wave_max_u32(L[0]);
        const uint64_t holders = __ballot(L[0] == key);
        if (lane == __builtin_ctzll(holders)) {
#pragma unroll
            for (int i = 0; i + 1 < M; i++) L[i] = L[i + 1];
            L[M - 1] = 0u;
        }
    }
    mx = wave_max_u32(mx);
    if (lane != 0) return;
    if (invert) key ^= kmask;
    auto to_f32 = [](uint32_t k) -> float {
        if (DT == NVFP4_F32) return u2f(k);
        if (DT == NVFP4_BF16) return u2f(k << 16);
        return (float)__builtin_bit_cast(_Float16, (uint16_t)k);
    };
    const uint32_t inf_key = (DT == NVFP4_F32) ? 0x7F800000u : (DT == NVFP4_BF16 ? 0x7F80u : 0x7C00u);
    if (mx >= inf_key && flags) atomicOr(flags, 1);
    out_pct[ch] = to_f32(key);
    if (out_max) out_max[ch] = to_f32(mx);
}

// Returns false (nothing launched) when a row chunk would exceed 32-bit buffer offsets.
template <int DT, int M>
static bool launch_topm(const void *x, int64_t rows, int64_t cols, int64_t ld_x, uint32_t m, int invert,
                        float *out_pct, float *out_max, int32_t *flags, uint32_t *ws, int num_cus,
                        hipStream_t stream, uint32_t *out_key = nullptr, uint32_t *clear = nullptr) {
    constexpr int CPL = DT != NVFP4_F32 ? 4 : 2;
    constexpr int EB = DT == NVFP4_F32 ? 4 : 2;
    const int64_t cgroups = (cols + 64 * CPL - 1) / (64 * CPL);
    // one round of workgroups, at most one per CU (a second partial round, or more lists for the
    // final merge, measured slower), at least 64 rows each; the lists must fit the workspace and
    // the final wave (one lane per list)
    int64_t rchunks = (int64_t)num_cus / cgroups;
    const int64_t by_rows = (rows + 63) / 64;
    int64_t by_ws = 259 / (M + 1);
    if (by_ws > 64) by_ws = 64;
    if (rchunks > by_rows) rchunks = by_rows;
    if (rchunks > by_ws) rchunks = by_ws;
    if (rchunks < 1) rchunks = 1;
    const int rows_per_wg = (int)((rows + rchunks - 1) / rchunks);
    rchunks = (rows + rows_per_wg - 1) / rows_per_wg;
    if ((int64_t)(rows_per_wg + 2 * kTopmWaves * kTopmU) * ld_x * EB >= ((int64_t)1 << 31)) return false;
    hipLaunchKernelGGL((k_pct_topm<DT, M>), dim3((unsigned)cgroups, (unsigned)rchunks), dim3(64 * kTopmWaves), 0,
                       stream, (const uint8_t *)x, rows, cols, ld_x * EB, rows_per_wg, invert, (int)rchunks, ws);
    hipLaunchKernelGGL((k_pct_topm_final<DT, M>), dim3((unsigned)((cols + 3) / 4)), dim3(256), 0, stream, ws, cols,
                       (int)rchunks, (int)m, invert, out_pct, out_max, flags, out_key, clear);
    return true;
}

// Exact radix selection of the k-th smallest |x| per channel (or of the whole tensor) over `rows`
// rows of row stride ld_x elements, with the workspace's radix state already initialized.  only:
// when not NULL, just the marked channels are wanted (the others' passes are skipped or wasted).
// out_pct NULL: the result stays in the workspace's prefix words.
template <int DT>
static void radix_passes(const void *x, int64_t rows, int64_t cols, int64_t ld_x, int per_channel, float *out_pct,
                         float *out_max, int32_t *flags, uint32_t *ws, const uint32_t *only, int num_cus,
                         hipStream_t stream, bool deep = false) {
    constexpr int EB = (DT == NVFP4_F32) ? 4 : 2;
    constexpr int WCH = kPctChannels;
    constexpr int KEYBITS = (DT == NVFP4_F32) ? 31 : 15;
    const int64_t nch = per_channel ? cols : 1;
    // A workgroup per CU (its 128 KB of counters fill most of the LDS), but at least 1024 rows each:
    // every workgroup pays for clearing and merging 256 channels x 256 counters, which few rows would
    // not amortize; and at most 65535 rows, so the 16-bit counters cannot overflow.  Long chunks keep
    // 16 rows in flight per lane, short ones 4.  Counts and maxima add up across launches, so rows
    // beyond what one grid of 65535 chunks holds go to further launches over later rows.
    const int64_t cgroups = (cols + WCH - 1) / WCH;
    const int64_t seg_max = (int64_t)kPctMaxRowsPerWg * 65535;
    auto hist_pass = [&](int shift, int dbits, int first_pass) {
        for (int64_t s0 = 0; s0 < rows; s0 += seg_max) {
            const int64_t srows = (rows - s0) < seg_max ? (rows - s0) : seg_max;
            int64_t rchunks = (int64_t)num_cus / cgroups;  // one round of workgroups: no straggler round
            const int64_t max_chunks = (srows + 1023) / 1024;
            if (rchunks > max_chunks) rchunks = max_chunks;
            const int64_t min_chunks = (srows + kPctMaxRowsPerWg - 1) / kPctMaxRowsPerWg;
            if (rchunks < min_chunks) rchunks = min_chunks;
            if (rchunks < 1) rchunks = 1;
            const int rows_per_wg = (int)((srows + rchunks - 1) / rchunks);
            rchunks = (srows + rows_per_wg - 1) / rows_per_wg;
            const uint8_t *xs = (const uint8_t *)x + s0 * ld_x * EB;
            if (rows_per_wg >= 8192 || deep)
                hipLaunchKernelGGL((k_pct_hist<DT, 16>), dim3((unsigned)cgroups, (unsigned)rchunks), dim3(kPctThreads),
                                   0, stream, xs, srows, cols, ld_x * EB, per_channel, rows_per_wg, shift, dbits,
                                   first_pass, ws, only);
            else
                hipLaunchKernelGGL((k_pct_hist<DT, 4>), dim3((unsigned)cgroups, (unsigned)rchunks), dim3(kPctThreads),
                                   0, stream, xs, srows, cols, ld_x * EB, per_channel, rows_per_wg, shift, dbits,
                                   first_pass, ws, only);
        }
    };
    int consumed = 0;
    bool first = true;
    while (consumed < KEYBITS) {
        const int dbits = (KEYBITS - consumed) >= 8 ? 8 : (KEYBITS - consumed);
        const int shift = KEYBITS - consumed - dbits;
        hist_pass(shift, dbits, first ? 1 : 0);
        consumed += dbits;
        const int last = consumed == KEYBITS;
        hipLaunchKernelGGL(k_pct_select<DT>, dim3((unsigned)((nch + 3) / 4)), dim3(256), 0, stream, ws, nch, dbits,
                           last, out_pct, out_max, flags, only);
        first = false;
    }
}

// Rank of the sample element whose key bounds the candidates: about kt / stride sample elements
// lie beyond the wanted rank kt; the bound adds 8 standard deviations of that count and 16, so that
// a threshold short of the rank is very unlikely for rows drawn alike.
static uint32_t sample_rank(uint32_t kt) {
    const uint32_t e = (kt + kSampleStride - 1) / kSampleStride;
    uint32_t r = 1;
    while (r * r < e) r++;
    return e + 8 * r + 16;
}

template <int DT>
static hipError_t launch_pct_t(const void *x, int64_t rows, int64_t cols, int64_t ld_x, uint32_t k, int per_channel,
                               float *out_pct, float *out_max, int32_t *flags, uint32_t *ws, size_t ws_bytes,
                               int num_cus, hipStream_t stream) {
    constexpr int EB = (DT == NVFP4_F32) ? 4 : 2;
    constexpr int WCH = kPctChannels;
    const int64_t nch = per_channel ? cols : 1;
    if (per_channel) {
        // rank near the top (m-th largest) or the bottom (k-th smallest): one pass
        const uint32_t n = (uint32_t)rows, mtop = n - k + 1;
        const bool top = mtop <= k;
        const uint32_t m = top ? mtop : k;
        if (m <= (uint32_t)kTopmMax) {
            const int inv = top ? 0 : 1;
            bool done;
            // lists of exactly m keys up to 6 (each key costs 2 M compare-exchange VALU), then 8, 12, 16
#define NVFP4_TOPM(M_) launch_topm<DT, (M_)>(x, rows, cols, ld_x, m, inv, out_pct, out_max, flags, ws, num_cus, stream)
            if (m <= 1) done = NVFP4_TOPM(1);
            else if (m <= 2) done = NVFP4_TOPM(2);
            else if (m <= 3) done = NVFP4_TOPM(3);
            else if (m <= 4) done = NVFP4_TOPM(4);
            else if (m <= 5) done = NVFP4_TOPM(5);
            else if (m <= 6) done = NVFP4_TOPM(6);
            else if (m <= 8) done = NVFP4_TOPM(8);
            else if (m <= 12) done = NVFP4_TOPM(12);
            else done = NVFP4_TOPM(16);
#undef NVFP4_TOPM
            if (done) return hipGetLastError();
        }
        // further from the end, on many rows: the sample threshold and one candidate pass, then the
        // exact radix passes for the channels that need them
        const uint32_t ks = sample_rank(m);
        const int64_t srows = rows / kSampleStride;
        // candidates expected beyond the threshold: ks * stride, plus 6 standard deviations
        uint32_t sd = 1;
        while (sd * sd < ks) sd++;
        const char *env = getenv("NVFP4_PCT_CAND_CAP");  // tests lower it to force the exact passes
        const long cap_env = env ? strtol(env, nullptr, 10) : kCandCap;
        const int cap = cap_env < 0 ? 0 : cap_env > kCandCap ? kCandCap : (int)cap_env;
        if (rows >= kCandMinRows && ks <= srows && ks * kSampleStride + 6 * kSampleStride * sd <= (uint32_t)kCandCap &&
            ws_bytes >= percentile_ws_bytes(cols, 1) &&
            (int64_t)(kSampleStride + 1) * ld_x * EB * 65535 < ((int64_t)1 << 62)) {
            // the threshold: the ks-th key of the union of the one-pass lists (the 8 largest, or
            // smallest, per workgroup) over the sample, which is at or beyond the sample's ks-th (a
            // workgroup rarely holds more than 8 of the sample's ks, and a few more candidates are
            // harmless); lists in the radix words, thresholds in the fallback-mark words; the
            // candidate counts, overflow marks and maxima start at zero
            if (!launch_topm<DT, 8>(x, srows, cols, ld_x * kSampleStride, ks, top ? 0 : 1, nullptr, nullptr, nullptr,
                                    ws, num_cus, stream, ws + 262 * nch, ws + 259 * nch))
                goto radix;
            // the candidate pass: chunks as in the histogram pass (one round, >= 1024 rows each), but
            // enough of them that a workgroup's share of a channel's candidates (at most the bound
            // above) fits its LDS lists
            const int64_t cgroups = (cols + WCH - 1) / WCH;
            int64_t rchunks = (int64_t)num_cus / cgroups;
            const int64_t max_chunks = (rows + 1023) / 1024;
            if (rchunks > max_chunks) rchunks = max_chunks;
            const int64_t for_lds = ((int64_t)(ks * kSampleStride + 6 * kSampleStride * sd) + kCandLds - 1) / kCandLds;
            if (rchunks < for_lds) rchunks = for_lds;
            if (rchunks < 1) rchunks = 1;
            const int64_t rpw = (rows + rchunks - 1) / rchunks;
            if (rpw < ((int64_t)1 << 31)) {
                rchunks = (rows + rpw - 1) / rpw;
                // 16 rows in flight per lane: the pass streams at close to the copy rate
                if (top)
                    hipLaunchKernelGGL((k_pct_cand<DT, 16, true>), dim3((unsigned)cgroups, (unsigned)rchunks),
                                       dim3(kPctThreads), 0, stream, (const uint8_t *)x, rows, cols, ld_x * EB,
                                       (int)rpw, cap, ws);
                else
                    hipLaunchKernelGGL((k_pct_cand<DT, 16, false>), dim3((unsigned)cgroups, (unsigned)rchunks),
                                       dim3(kPctThreads), 0, stream, (const uint8_t *)x, rows, cols, ld_x * EB,
                                       (int)rpw, cap, ws);
                hipLaunchKernelGGL(k_pct_cand_select<DT>, dim3((unsigned)nch), dim3(64), 0, stream, ws, nch, m, k,
                                   top ? 1 : 0, cap, out_pct, out_max, flags);
                // the exact passes, for the channels marked above only
                radix_passes<DT>(x, rows, cols, ld_x, 1, out_pct, out_max, flags, ws, ws + 262 * nch, num_cus,
                                 stream);
                return hipGetLastError();
            }
        }
    }
radix:
    const int64_t words = nch * 259;
    hipLaunchKernelGGL(k_pct_init, dim3((unsigned)((words + 255) / 256 < 4096 ? (words + 255) / 256 : 4096)),
                       dim3(256), 0, stream, ws, nch, k, words);
    radix_passes<DT>(x, rows, cols, ld_x, per_channel, out_pct, out_max, flags, ws, nullptr, num_cus, stream);
    return hipGetLastError();
}

hipError_t launch_percentile(const void *x, nvfp4_dtype dt, int64_t rows, int64_t cols, int64_t ld_x, uint32_t k,
                             int per_channel, float *out_pct, float *out_max, int32_t *flags, void *workspace,
                             size_t workspace_bytes, int num_cus, hipStream_t stream) {
    uint32_t *ws = reinterpret_cast<uint32_t *>(workspace);
    switch (dt) {
    case NVFP4_F32:
        return launch_pct_t<NVFP4_F32>(x, rows, cols, ld_x, k, per_channel, out_pct, out_max, flags, ws,
                                       workspace_bytes, num_cus, stream);
    case NVFP4_BF16:
        return launch_pct_t<NVFP4_BF16>(x, rows, cols, ld_x, k, per_channel, out_pct, out_max, flags, ws,
                                        workspace_bytes, num_cus, stream);
    default:
        return launch_pct_t<NVFP4_F16>(x, rows, cols, ld_x, k, per_channel, out_pct, out_max, flags, ws,
                                       workspace_bytes, num_cus, stream);
    }
}

}  // namespace nvfp4
