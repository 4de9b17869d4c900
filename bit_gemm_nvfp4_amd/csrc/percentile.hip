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
//                 channel's prefix; one workgroup per (64 x lanes' channels, row chunk), counters in
//                 LDS laid out [digit][channel] so that the 64 lanes of a wave, which hold 64
//                 different channels, never hit one address; merged into global counters with
//                 atomics (integer, so the result does not depend on the order); the first pass
//                 also takes the per-channel maximum key;
//   k_pct_select  one thread per channel scans its 2^d counters, picks the digit holding the
//                 remaining rank, narrows the prefix, and clears the counters for the next pass;
//                 the last pass writes the results.
#include <hip/hip_runtime.h>

#include "common.h"
#include "internal.h"

namespace nvfp4 {

// Workspace layout (uint32 words), nch = cols (per channel) or 1:
//   [0, nch) prefix   [nch, 2 nch) remaining rank   [2 nch, 3 nch) max key   [3 nch, 3 nch + 256 nch) counters
size_t percentile_ws_bytes(int64_t cols, int per_channel) {
    const int64_t nch = per_channel ? cols : 1;
    return (size_t)nch * (3 + 256) * 4;
}

__global__ void k_pct_init(uint32_t *ws, int64_t nch, uint32_t k) {
    const int64_t n = nch * (3 + 256);
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (int64_t)gridDim.x * blockDim.x)
        ws[i] = (i >= nch && i < 2 * nch) ? k : 0u;
}

// DT: NVFP4_F32 (31-bit keys, one channel per lane) or NVFP4_BF16 / NVFP4_F16 (15-bit keys, two
// channels per lane, one 32-bit load per lane and row).
template <int DT>
__global__ __launch_bounds__(256) void k_pct_hist(const uint8_t *__restrict__ x, int64_t rows, int64_t cols,
                                                  int64_t ld_bytes, int per_channel, int rows_per_wg, int shift,
                                                  int dbits, int first_pass, uint32_t *__restrict__ ws) {
    constexpr int CPL = (DT == NVFP4_F32) ? 1 : 2;
    constexpr int WCH = 64 * CPL;
    __shared__ uint32_t hist[256 * WCH];
    const int64_t nch = per_channel ? cols : 1;
    uint32_t *prefix = ws, *maxkey = ws + 2 * nch, *ghist = ws + 3 * nch;

    const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
    for (int i = tid; i < 256 * WCH; i += 256) hist[i] = 0u;

    const int64_t c0 = (int64_t)blockIdx.x * WCH;
    const int64_t r0 = (int64_t)blockIdx.y * rows_per_wg;
    int64_t r1 = r0 + rows_per_wg;
    if (r1 > rows) r1 = rows;
    const int64_t cl = c0 + lane * CPL;  // first channel of this lane
    const bool active = cl < cols;
    uint32_t pre[CPL], mk[CPL];
#pragma unroll
    for (int j = 0; j < CPL; j++) {
        pre[j] = (active && !first_pass) ? prefix[per_channel ? cl + j : 0] : 0u;
        mk[j] = 0u;
    }
    const uint32_t dmask = (1u << dbits) - 1u;
    const int hs = shift + dbits;  // bits above the current digit
    __syncthreads();

    if (active) {
        const uint8_t *base = x + cl * (DT == NVFP4_F32 ? 4 : 2);
        constexpr int U = 8;
        int64_t r = r0 + wid;
        auto account = [&](uint32_t key, int j) {
            if (first_pass) mk[j] = max(mk[j], key);
            if (hs >= 32 || (key >> hs) == pre[j]) atomicAdd(&hist[((key >> shift) & dmask) * WCH + lane * CPL + j], 1u);
        };
        for (; r + 4 * (U - 1) < r1; r += 4 * U) {
            uint32_t w[U];
#pragma unroll
            for (int u = 0; u < U; u++) w[u] = *reinterpret_cast<const uint32_t *>(base + (r + 4 * u) * ld_bytes);
#pragma unroll
            for (int u = 0; u < U; u++) {
                if constexpr (CPL == 1) {
                    account(w[u] & 0x7FFFFFFFu, 0);
                } else {
                    account(w[u] & 0x7FFFu, 0);
                    account((w[u] >> 16) & 0x7FFFu, 1);
                }
            }
        }
        for (; r < r1; r += 4) {
            const uint32_t w = *reinterpret_cast<const uint32_t *>(base + r * ld_bytes);
            if constexpr (CPL == 1) {
                account(w & 0x7FFFFFFFu, 0);
            } else {
                account(w & 0x7FFFu, 0);
                account((w >> 16) & 0x7FFFu, 1);
            }
        }
        if (first_pass) {
#pragma unroll
            for (int j = 0; j < CPL; j++) atomicMax(&maxkey[per_channel ? cl + j : 0], mk[j]);
        }
    }
    __syncthreads();
    const int nbins = 1 << dbits;
    for (int i = tid; i < nbins * WCH; i += 256) {
        const uint32_t cnt = hist[i];
        const int64_t ch = c0 + (i % WCH);
        if (cnt && ch < cols) atomicAdd(&ghist[(per_channel ? ch : 0) * 256 + i / WCH], cnt);
    }
}

// One thread per channel.  last: write key -> value of the selected element and of the maximum.
template <int DT>
__global__ void k_pct_select(uint32_t *__restrict__ ws, int64_t nch, int shift, int dbits, int last,
                             float *__restrict__ out_pct, float *__restrict__ out_max, int32_t *__restrict__ flags) {
    const int64_t ch = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (ch >= nch) return;
    uint32_t *prefix = ws, *krem = ws + nch, *maxkey = ws + 2 * nch, *h = ws + 3 * nch + ch * 256;
    const int nbins = 1 << dbits;
    uint32_t need = krem[ch], cum = 0;
    int d = nbins - 1;
    for (int i = 0; i < nbins; i++) {
        const uint32_t c = h[i];
        if (cum + c >= need) {
            d = i;
            break;
        }
        cum += c;
    }
    for (int i = 0; i < nbins; i++) h[i] = 0u;
    const uint32_t p = (prefix[ch] << dbits) | (uint32_t)d;
    prefix[ch] = p;
    krem[ch] = need - cum;
    if (last) {
        auto to_f32 = [](uint32_t key) -> float {
            if (DT == NVFP4_F32) return u2f(key);
            if (DT == NVFP4_BF16) return u2f(key << 16);
            return (float)__builtin_bit_cast(_Float16, (uint16_t)key);
        };
        const uint32_t mk = maxkey[ch];
        const uint32_t inf_key = (DT == NVFP4_F32) ? 0x7F800000u : (DT == NVFP4_BF16 ? 0x7F80u : 0x7C00u);
        if (mk >= inf_key && flags) atomicOr(flags, 1);
        out_pct[ch] = to_f32(p);
        if (out_max) out_max[ch] = to_f32(mk);
    }
}

template <int DT>
static hipError_t launch_pct_t(const void *x, int64_t rows, int64_t cols, int64_t ld_x, uint32_t k, int per_channel,
                               float *out_pct, float *out_max, int32_t *flags, uint32_t *ws, int num_cus,
                               hipStream_t stream) {
    constexpr int EB = (DT == NVFP4_F32) ? 4 : 2;
    constexpr int WCH = (DT == NVFP4_F32) ? 64 : 128;
    constexpr int KEYBITS = (DT == NVFP4_F32) ? 31 : 15;
    const int64_t nch = per_channel ? cols : 1;
    hipLaunchKernelGGL(k_pct_init, dim3((unsigned)((nch * 259 + 255) / 256 < 4096 ? (nch * 259 + 255) / 256 : 4096)),
                       dim3(256), 0, stream, ws, nch, k);
    const int64_t cgroups = (cols + WCH - 1) / WCH;
    int64_t target = (int64_t)num_cus * 4;
    int64_t rchunks = (target + cgroups - 1) / cgroups;
    if (rchunks > rows) rchunks = rows;
    if (rchunks < 1) rchunks = 1;
    if (rchunks > 65535) rchunks = 65535;
    const int rows_per_wg = (int)((rows + rchunks - 1) / rchunks);
    rchunks = (rows + rows_per_wg - 1) / rows_per_wg;
    int consumed = 0;
    bool first = true;
    while (consumed < KEYBITS) {
        const int dbits = (KEYBITS - consumed) >= 8 ? 8 : (KEYBITS - consumed);
        const int shift = KEYBITS - consumed - dbits;
        hipLaunchKernelGGL(k_pct_hist<DT>, dim3((unsigned)cgroups, (unsigned)rchunks), dim3(256), 0, stream,
                           (const uint8_t *)x, rows, cols, ld_x * EB, per_channel, rows_per_wg, shift, dbits,
                           first ? 1 : 0, ws);
        consumed += dbits;
        const int last = consumed == KEYBITS;
        hipLaunchKernelGGL(k_pct_select<DT>, dim3((unsigned)((nch + 255) / 256)), dim3(256), 0, stream, ws, nch, shift,
                           dbits, last, out_pct, out_max, flags);
        first = false;
    }
    return hipGetLastError();
}

hipError_t launch_percentile(const void *x, nvfp4_dtype dt, int64_t rows, int64_t cols, int64_t ld_x, uint32_t k,
                             int per_channel, float *out_pct, float *out_max, int32_t *flags, void *workspace,
                             int num_cus, hipStream_t stream) {
    uint32_t *ws = reinterpret_cast<uint32_t *>(workspace);
    switch (dt) {
    case NVFP4_F32:
        return launch_pct_t<NVFP4_F32>(x, rows, cols, ld_x, k, per_channel, out_pct, out_max, flags, ws, num_cus, stream);
    case NVFP4_BF16:
        return launch_pct_t<NVFP4_BF16>(x, rows, cols, ld_x, k, per_channel, out_pct, out_max, flags, ws, num_cus,
                                        stream);
    default:
        return launch_pct_t<NVFP4_F16>(x, rows, cols, ld_x, k, per_channel, out_pct, out_max, flags, ws, num_cus, stream);
    }
}

}  // namespace nvfp4
