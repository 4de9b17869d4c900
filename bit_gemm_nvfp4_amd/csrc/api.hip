// C ABI of libnvfp4.so: argument validation and dispatch to the gfx950 kernels.
//
// Every entry point validates all of its arguments before enqueuing anything, so an error status
// means no work was queued.  No entry point synchronizes, allocates or keeps a pointer.
#include <algorithm>
#include <hip/hip_runtime.h>

#include <atomic>
#include <cmath>
#include <cstring>

#include "internal.h"
#include "nvfp4.h"

namespace nvfp4 {

__global__ void k_fill_zero_f32(float *c, int64_t rows, int64_t cols, int64_t ld) {
    const int64_t n = rows * cols;
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (int64_t)gridDim.x * blockDim.x)
        c[(i / cols) * ld + i % cols] = 0.0f;
}

hipError_t launch_fill_zero_f32(float *c, int64_t rows, int64_t cols, int64_t ld, hipStream_t stream) {
    if (rows > 0 && cols > 0) {
        int64_t grid = (rows * cols + 255) / 256;
        if (grid > 4096) grid = 4096;
        hipLaunchKernelGGL(k_fill_zero_f32, dim3((unsigned)grid), dim3(256), 0, stream, c, rows, cols, ld);
    }
    return hipGetLastError();
}

namespace {

constexpr int kMaxDevices = 64;
// Per-device cache: 0 = not checked, 1 = gfx950, 2 = other architecture.  Also the CU count.
std::atomic<int> g_dev_state[kMaxDevices];
std::atomic<int> g_dev_cus[kMaxDevices];

// Check (once per device) that the current device is gfx950; returns its CU count or 0.
int current_device_cus() {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return 0;
    int st = g_dev_state[dev].load(std::memory_order_acquire);
    if (st == 0) {
        hipDeviceProp_t prop;
        if (hipGetDeviceProperties(&prop, dev) != hipSuccess) return 0;
        const bool ok = std::strncmp(prop.gcnArchName, "gfx950", 6) == 0;
        g_dev_cus[dev].store(prop.multiProcessorCount, std::memory_order_relaxed);
        st = ok ? 1 : 2;
        g_dev_state[dev].store(st, std::memory_order_release);
    }
    return st == 1 ? g_dev_cus[dev].load(std::memory_order_relaxed) : 0;
}

inline bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
inline bool aligned4(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 3u) == 0; }

int elem_bytes(nvfp4_dtype dt) {
    switch (dt) {
    case NVFP4_F32: return 4;
    case NVFP4_BF16:
    case NVFP4_F16: return 2;
    case NVFP4_E4M3: return 1;
    default: return 0;
    }
}

// Shape and alignment checks shared by every NVFP4 tensor argument.
// codes and scales may be NULL only for a tensor with no elements; global_scale is always required.
size_t align256(size_t b) { return (b + 255) / 256 * 256; }

constexpr int64_t kQaFusedMaxN = 512;  // widest N that nvfp4_gemm_qa runs with the fused kernel

// Workspace of the unfused form of nvfp4_gemm_qa: the NVFP4 activations (codes, scales, scale).
size_t qa_ws_bytes(int64_t M, int64_t K) {
    if (M <= 0 || K <= 0) return 0;
    return align256((size_t)M * (size_t)(K / 2)) + align256((size_t)M * (size_t)(K / 16)) + 256;
}

nvfp4_status check_qtensor(const nvfp4_tensor *t) {
    if (!t || !t->global_scale) return NVFP4_ERR_NULL;
    if (t->rows < 0 || t->cols < 0 || (t->cols % 16) != 0) return NVFP4_ERR_SHAPE;
    const bool empty = t->rows == 0 || t->cols == 0;
    if (!empty && (!t->codes || !t->scales)) return NVFP4_ERR_NULL;
    if (!aligned16(t->codes) || !aligned16(t->scales) || !aligned4(t->global_scale)) return NVFP4_ERR_ALIGN;
    return NVFP4_OK;
}

// A row-major matrix argument: ld >= cols and rows aligned to `align` bytes (16 for everything the
// kernels read with 128-bit loads; 4 for the GEMM output, written one float at a time).  The
// pointer may be NULL only when the matrix has no elements.
nvfp4_status check_matrix(const void *p, int64_t rows, int64_t cols, int64_t ld, int eb, int align = 16) {
    if (rows < 0 || cols < 0 || ld < cols) return NVFP4_ERR_SHAPE;
    if (rows == 0 || cols == 0) return NVFP4_OK;  // no element is addressed
    if (!p) return NVFP4_ERR_NULL;
    if ((reinterpret_cast<uintptr_t>(p) % align) != 0 || (rows > 1 && ((ld * eb) % align) != 0))
        return NVFP4_ERR_ALIGN;
    return NVFP4_OK;
}

// Scratch of nvfp4_quantize_noalloc: the run-time amax agreement's tag records and slots, one array
// per GPU for the life of the process.  Zero-initialized when the code object loads, which is the
// state the agreement needs before its first use; each call leaves it consistent for the next.
// The host sees only a stand-in for this name: kernels get the device address from
// hipGetSymbolAddress (scratch_address below).
static __device__ __align__(256) uint8_t scratch[kQuantizeWsBytes];

std::atomic<void *> g_scratch_ptr[kMaxDevices];

// Device address of the current device's scratch array, looked up once per device; NULL on failure.
void *scratch_address() {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
    void *p = g_scratch_ptr[dev].load(std::memory_order_acquire);
    if (p) return p;
    void *q = nullptr;
    if (hipGetSymbolAddress(&q, HIP_SYMBOL(scratch)) != hipSuccess || !q) return nullptr;
    g_scratch_ptr[dev].store(q, std::memory_order_release);
    return q;
}

}  // namespace
}  // namespace nvfp4

using namespace nvfp4;

extern "C" {

const char *nvfp4_status_string(nvfp4_status s) {
    switch (s) {
    case NVFP4_OK: return "ok";
    case NVFP4_ERR_NULL: return "a required pointer is NULL";
    case NVFP4_ERR_SHAPE: return "bad shape (negative size, cols % 16 != 0, ld < cols, or operands disagree)";
    case NVFP4_ERR_ALIGN: return "a pointer or row start is not 16-byte aligned";
    case NVFP4_ERR_DTYPE: return "dtype not accepted by this entry point";
    case NVFP4_ERR_WORKSPACE: return "workspace missing or too small";
    case NVFP4_ERR_ARG: return "bad argument";
    case NVFP4_ERR_DEVICE: return "the current device is not gfx950";
    case NVFP4_ERR_LAUNCH: return "kernel launch failed";
    default: return "unknown status";
    }
}

size_t nvfp4_workspace_size(int op, int64_t rows, int64_t cols, int64_t k) {
    switch (op) {
    case NVFP4_OP_QUANTIZE: return kQuantizeWsBytes;
    case NVFP4_OP_AMAX: return kAmaxWsBytes;
    case NVFP4_OP_PERCENTILE: return cols >= 0 ? percentile_ws_bytes(cols, k ? 1 : 0) : 0;
    case NVFP4_OP_STATS: return stats_ws_bytes();
    case NVFP4_OP_GEMM_QA: {
        // the group counters of the staged form, then the largest of the three forms' needs
        if (rows < 0 || cols < 0 || k < 0) return 0;
        const int cus = current_device_cus();
        const int c2 = cus > 0 ? cus : 256;
        const size_t fused = gemm_ws_bytes(rows, cols, k, c2, kFirstQuantTileCfg);
        const size_t two_step = qa_ws_bytes(rows, k) + gemm_ws_bytes(rows, cols, k, c2);
        const size_t staged = gemm_qa_staged_ws_bytes(rows, cols, k, c2) - kQaSyncBytes;
        return kQaSyncBytes + std::max(fused, std::max(two_step, staged));
    }
    case NVFP4_OP_LOWRANK: {
        if (rows < 0 || cols < 0 || k < 0) return 0;
        const int cus = current_device_cus();
        return lowrank_t_bytes(rows) + gemm_ws_bytes(rows, cols, k, cus > 0 ? cus : 256);
    }
    case NVFP4_OP_GEMM: {
        // planned for the current device's CU count (256, an MI355X, when none can be queried)
        const int cus = current_device_cus();
        return gemm_ws_bytes(rows, cols, k, cus > 0 ? cus : 256);
    }
    default: return 0;
    }
}

nvfp4_status nvfp4_quantize(const void *x, nvfp4_dtype x_dtype, int64_t ld_x, const float *src_scale,
                            const float *amax_in, const nvfp4_tensor *out, int32_t *flags, void *workspace,
                            size_t workspace_bytes, hipStream_t stream) {
    const int eb = elem_bytes(x_dtype);
    if (eb == 0) return NVFP4_ERR_DTYPE;
    nvfp4_status st = check_qtensor(out);
    if (st != NVFP4_OK) return st;
    st = check_matrix(x, out->rows, out->cols, ld_x, eb);
    if (st != NVFP4_OK) return st;
    if (src_scale && x_dtype != NVFP4_E4M3) return NVFP4_ERR_ARG;
    if ((src_scale && !aligned4(src_scale)) || (amax_in && !aligned4(amax_in)) || (flags && !aligned4(flags)))
        return NVFP4_ERR_ALIGN;
    if (!amax_in && (!workspace || workspace_bytes < kQuantizeWsBytes)) return NVFP4_ERR_WORKSPACE;
    if (workspace && !aligned16(workspace)) return NVFP4_ERR_ALIGN;
    const int cus = current_device_cus();
    if (cus == 0) return NVFP4_ERR_DEVICE;
    hipError_t e = launch_quantize(x, x_dtype, ld_x, src_scale, amax_in, out, flags, workspace, cus, stream);
    return e == hipSuccess ? NVFP4_OK : NVFP4_ERR_LAUNCH;
}

nvfp4_status nvfp4_quantize_batch(int count, const void *const *x, nvfp4_dtype x_dtype, const int64_t *ld_x,
                                  const float *const *src_scale, const nvfp4_tensor *out, int32_t *flags,
                                  void *workspace, size_t workspace_bytes, hipStream_t stream) {
    if (count < 0 || count > kQuantizeMaxBatch) return NVFP4_ERR_ARG;
    if (count == 0) return NVFP4_OK;
    if (!x || !ld_x || !out) return NVFP4_ERR_NULL;
    const int eb = elem_bytes(x_dtype);
    if (eb == 0) return NVFP4_ERR_DTYPE;
    for (int i = 0; i < count; i++) {
        nvfp4_status st = check_qtensor(&out[i]);
        if (st != NVFP4_OK) return st;
        st = check_matrix(x[i], out[i].rows, out[i].cols, ld_x[i], eb);
        if (st != NVFP4_OK) return st;
        const float *sc = src_scale ? src_scale[i] : nullptr;
        if (sc && x_dtype != NVFP4_E4M3) return NVFP4_ERR_ARG;
        if (sc && !aligned4(sc)) return NVFP4_ERR_ALIGN;
    }
    if (flags && !aligned4(flags)) return NVFP4_ERR_ALIGN;
    if (!workspace || workspace_bytes < kQuantizeWsBytes) return NVFP4_ERR_WORKSPACE;
    if (!aligned16(workspace)) return NVFP4_ERR_ALIGN;
    const int cus = current_device_cus();
    if (cus == 0) return NVFP4_ERR_DEVICE;
    bool batched = false;
    hipError_t e = launch_quantize_batch(count, x, x_dtype, ld_x, src_scale, out, flags, workspace, cus, stream,
                                         &batched);
    // not batched (a tensor too large to stay resident beside the others): one call per tensor,
    // in order on the stream, sharing the workspace
    for (int i = 0; e == hipSuccess && !batched && i < count; i++)
        e = launch_quantize(x[i], x_dtype, ld_x[i], src_scale ? src_scale[i] : nullptr, nullptr, &out[i], flags,
                            workspace, cus, stream);
    return e == hipSuccess ? NVFP4_OK : NVFP4_ERR_LAUNCH;
}

nvfp4_status nvfp4_quantize_noalloc(const void *x, nvfp4_dtype x_dtype, int64_t ld_x, const float *src_scale,
                                    const float *amax_in, const nvfp4_tensor *out, int32_t *flags,
                                    hipStream_t stream) {
    const int eb = elem_bytes(x_dtype);
    if (eb == 0) return NVFP4_ERR_DTYPE;
    nvfp4_status st = check_qtensor(out);
    if (st != NVFP4_OK) return st;
    st = check_matrix(x, out->rows, out->cols, ld_x, eb);
    if (st != NVFP4_OK) return st;
    if (src_scale && x_dtype != NVFP4_E4M3) return NVFP4_ERR_ARG;
    if ((src_scale && !aligned4(src_scale)) || (amax_in && !aligned4(amax_in)) || (flags && !aligned4(flags)))
        return NVFP4_ERR_ALIGN;
    // the scratch holds the run-time amax agreement of any size (the grid is capped at its slots)
    static_assert(sizeof(scratch) >= kQuantizeWsBytes, "scratch smaller than the quantize workspace");
    if (nvfp4_workspace_size(NVFP4_OP_QUANTIZE, out->rows, out->cols, 0) > sizeof(scratch)) return NVFP4_ERR_WORKSPACE;
    const int cus = current_device_cus();
    if (cus == 0) return NVFP4_ERR_DEVICE;
    void *ws = nullptr;
    if (!amax_in) {
        ws = scratch_address();
        if (!ws) return NVFP4_ERR_DEVICE;
    }
    hipError_t e = launch_quantize(x, x_dtype, ld_x, src_scale, amax_in, out, flags, ws, cus, stream);
    return e == hipSuccess ? NVFP4_OK : NVFP4_ERR_LAUNCH;
}

nvfp4_status nvfp4_tensor_amax(const void *x, nvfp4_dtype x_dtype, int64_t rows, int64_t cols, int64_t ld_x,
                               const float *src_scale, float *amax_out, int32_t *flags, void *workspace,
                               size_t workspace_bytes, hipStream_t stream) {
    const int eb = elem_bytes(x_dtype);
    if (eb == 0) return NVFP4_ERR_DTYPE;
    if (!amax_out) return NVFP4_ERR_NULL;
    if (rows < 0 || cols < 0 || (cols % 16) != 0) return NVFP4_ERR_SHAPE;
    nvfp4_status st = check_matrix(x, rows, cols, ld_x, eb);
    if (st != NVFP4_OK) return st;
    if (src_scale && x_dtype != NVFP4_E4M3) return NVFP4_ERR_ARG;
    if (!aligned4(amax_out) || (src_scale && !aligned4(src_scale)) || (flags && !aligned4(flags)))
        return NVFP4_ERR_ALIGN;
    if (!workspace || workspace_bytes < kAmaxWsBytes) return NVFP4_ERR_WORKSPACE;
    if (!aligned16(workspace)) return NVFP4_ERR_ALIGN;
    const int cus = current_device_cus();
    if (cus == 0) return NVFP4_ERR_DEVICE;
    hipError_t e = launch_amax(x, x_dtype, ld_x, rows, cols, src_scale, amax_out, flags, workspace, cus, stream);
    return e == hipSuccess ? NVFP4_OK : NVFP4_ERR_LAUNCH;
}

nvfp4_status nvfp4_quantize_fp8(const void *x, nvfp4_dtype x_dtype, int64_t rows, int64_t cols, int64_t ld_x,
                                const float *src_scale, const float *amax_in, uint8_t *out, float *out_scale,
                                int32_t *flags, void *workspace, size_t workspace_bytes, hipStream_t stream) {
    const int eb = elem_bytes(x_dtype);
    if (eb == 0) return NVFP4_ERR_DTYPE;
    if (!out_scale) return NVFP4_ERR_NULL;
    if (rows < 0 || cols < 0 || (cols % 16) != 0) return NVFP4_ERR_SHAPE;
    nvfp4_status st = check_matrix(x, rows, cols, ld_x, eb);
    if (st != NVFP4_OK) return st;
    st = check_matrix(out, rows, cols, cols, 1);
    if (st != NVFP4_OK) return st;
    if (src_scale && x_dtype != NVFP4_E4M3) return NVFP4_ERR_ARG;
    if (!aligned4(out_scale) || (src_scale && !aligned4(src_scale)) || (amax_in && !aligned4(amax_in)) ||
        (flags && !aligned4(flags)))
        return NVFP4_ERR_ALIGN;
    if (!amax_in && (!workspace || workspace_bytes < kQuantizeWsBytes)) return NVFP4_ERR_WORKSPACE;
    if (workspace && !aligned16(workspace)) return NVFP4_ERR_ALIGN;
    const int cus = current_device_cus();
    if (cus == 0) return NVFP4_ERR_DEVICE;
    hipError_t e = launch_quantize_fp8(x, x_dtype, ld_x, rows, cols, src_scale, amax_in, out, out_scale, flags,
                                       workspace, cus, stream);
    return e == hipSuccess ? NVFP4_OK : NVFP4_ERR_LAUNCH;
}

nvfp4_status nvfp4_dequantize(const nvfp4_tensor *in, void *out, nvfp4_dtype out_dtype, int64_t ld_out,
                              hipStream_t stream) {
    nvfp4_status st = check_qtensor(in);
    if (st != NVFP4_OK) return st;
    if (out_dtype != NVFP4_F32 && out_dtype != NVFP4_BF16) return NVFP4_ERR_DTYPE;
    st = check_matrix(out, in->rows, in->cols, ld_out, elem_bytes(out_dtype));
    if (st != NVFP4_OK) return st;
    const int cus = current_device_cus();
    if (cus == 0) return NVFP4_ERR_DEVICE;
    if (in->rows == 0 || in->cols == 0) return NVFP4_OK;
    hipError_t e = launch_dequantize(in, out, out_dtype, ld_out, cus, stream);
    return e == hipSuccess ? NVFP4_OK : NVFP4_ERR_LAUNCH;
}

nvfp4_status nvfp4_gemm(const void *a_bf16, const nvfp4_tensor *a_q, int64_t M, int64_t lda, const nvfp4_tensor *w,
                        float *c, int64_t ldc, void *workspace, size_t workspace_bytes, hipStream_t stream) {
    if ((a_bf16 == nullptr) == (a_q == nullptr)) return NVFP4_ERR_ARG;
    nvfp4_status st = check_qtensor(w);
    if (st != NVFP4_OK) return st;
    const int64_t N = w->rows, K = w->cols;
    if (M < 0) return NVFP4_ERR_SHAPE;
    if (a_q) {
        st = check_qtensor(a_q);
        if (st != NVFP4_OK) return st;
        if (a_q->rows != M || a_q->cols != K) return NVFP4_ERR_SHAPE;
    } else {
        st = check_matrix(a_bf16, M, K, lda, 2);
        if (st != NVFP4_OK) return st;
    }
    st = check_matrix(c, M, N, ldc, 4, 4);
    if (st != NVFP4_OK) return st;
    if (workspace && !aligned16(workspace)) return NVFP4_ERR_ALIGN;
    const int cus = current_device_cus();
    if (cus == 0) return NVFP4_ERR_DEVICE;
    hipError_t e = (K == 0) ? launch_fill_zero_f32(c, M, N, ldc, stream)
                            : launch_gemm(a_bf16, a_q, M, lda, w, c, ldc, workspace, workspace_bytes, cus, stream);
    return e == hipSuccess ? NVFP4_OK : NVFP4_ERR_LAUNCH;
}

nvfp4_status nvfp4_gemm_lowrank(const void *a_bf16, const nvfp4_tensor *a_q, int64_t M, int64_t lda,
                                const nvfp4_tensor *w, const void *lr_down, const void *lr_up, int64_t rank, float *c,
                                int64_t ldc, void *workspace, size_t workspace_bytes, hipStream_t stream) {
    nvfp4_status st = check_qtensor(w);
    if (st != NVFP4_OK) return st;
    const int64_t N = w->rows, K = w->cols;
    if (M < 0) return NVFP4_ERR_SHAPE;
    if (rank < 16 || rank > 256 || rank % 16 != 0) return NVFP4_ERR_SHAPE;
    if (!a_bf16 && M > 0 && K > 0) return NVFP4_ERR_NULL;  // the branch always takes the bf16 activations
    st = check_matrix(a_bf16, M, K, lda, 2);
    if (st != NVFP4_OK) return st;
    if (a_q) {
        st = check_qtensor(a_q);
        if (st != NVFP4_OK) return st;
        if (a_q->rows != M || a_q->cols != K) return NVFP4_ERR_SHAPE;
    }
    st = check_matrix(lr_down, rank, K, K, 2);
    if (st != NVFP4_OK) return st;
    st = check_matrix(lr_up, N, rank, rank, 2);
    if (st != NVFP4_OK) return st;
    st = check_matrix(c, M, N, ldc, 4, 4);
    if (st != NVFP4_OK) return st;
    if (M > 0 && K > 0 && (!workspace || workspace_bytes < lowrank_t_bytes(M))) return NVFP4_ERR_WORKSPACE;
    if (workspace && !aligned16(workspace)) return NVFP4_ERR_ALIGN;
    const int cus = current_device_cus();
    if (cus == 0) return NVFP4_ERR_DEVICE;
    hipError_t e = (K == 0 || M == 0) ? launch_fill_zero_f32(c, M, N, ldc, stream)
                                      : launch_gemm_lowrank(a_bf16, a_q, M, lda, w, lr_down, lr_up, (int)rank, c, ldc,
                                                  workspace, workspace_bytes, cus, stream);
    return e == hipSuccess ? NVFP4_OK : NVFP4_ERR_LAUNCH;
}

nvfp4_status nvfp4_gemm_qa(const void *a_bf16, const float *a_amax, int64_t M, int64_t lda, const nvfp4_tensor *w,
                           float *c, int64_t ldc, void *workspace, size_t workspace_bytes, hipStream_t stream) {
    nvfp4_status st = check_qtensor(w);
    if (st != NVFP4_OK) return st;
    const int64_t N = w->rows, K = w->cols;
    if (M < 0) return NVFP4_ERR_SHAPE;
    if (!a_amax) return NVFP4_ERR_NULL;
    if (!aligned4(a_amax)) return NVFP4_ERR_ALIGN;
    st = check_matrix(a_bf16, M, K, lda, 2);
    if (st != NVFP4_OK) return st;
    st = check_matrix(c, M, N, ldc, 4, 4);
    if (st != NVFP4_OK) return st;
    if (workspace && !aligned16(workspace)) return NVFP4_ERR_ALIGN;
    const int cus = current_device_cus();
    // Three forms.  Staged (one launch): where all of the W4A4 product's workgroups run in one
    // round, each quantizes a share of its A row block into the workspace, waits for the other
    // workgroups of that row block, then runs the main loop on the quantized rows.  Otherwise the
    // fused kernel, which quantizes A in its staging path once per N tile, where that is not slower
    // (measured on MI355X: equal at N = 256 .. 512, 1.1x slower at N = 1024, 1.85x at N = 3072),
    // else a quantize pass into the workspace and the W4A4 kernel.  The first kQaSyncBytes of the
    // workspace hold the staged form's group counters; the other forms use what follows.
    const bool has_sync = workspace && workspace_bytes >= kQaSyncBytes;
    const bool staged = has_sync && workspace_bytes >= gemm_qa_staged_ws_bytes(M, N, K, cus) &&
                        gemm_qa_staged_applies(M, N, K, lda, cus);
    const bool fused = !staged && gemm_qa_fusable(M, K, lda) && N <= kQaFusedMaxN;
    uint8_t *rest = has_sync ? reinterpret_cast<uint8_t *>(workspace) + kQaSyncBytes : nullptr;
    const size_t rest_bytes = has_sync ? workspace_bytes - kQaSyncBytes : 0;
    if (!staged && !fused && M > 0 && K > 0 && rest_bytes < qa_ws_bytes(M, K)) return NVFP4_ERR_WORKSPACE;
    if (cus == 0) return NVFP4_ERR_DEVICE;
    hipError_t e;
    if (K == 0 || M == 0) {
        e = launch_fill_zero_f32(c, M, N, ldc, stream);
    } else if (staged) {
        e = launch_gemm_qa_staged(a_bf16, a_amax, M, lda, w, c, ldc, workspace, workspace_bytes, cus, stream);
    } else if (fused) {
        e = launch_gemm_qa_fused(a_bf16, a_amax, M, lda, w, c, ldc, rest, rest_bytes, cus, stream);
    } else {
        // quantize A with the static amax into the workspace, then the W4A4 product
        const size_t qb = qa_ws_bytes(M, K);
        const size_t cb = align256((size_t)M * (size_t)(K / 2)), sb = align256((size_t)M * (size_t)(K / 16));
        const nvfp4_tensor aq{rest, rest + cb, reinterpret_cast<float *>(rest + cb + sb), M, K};
        e = launch_quantize(a_bf16, NVFP4_BF16, lda, nullptr, a_amax, &aq, nullptr, nullptr, cus, stream);
        if (e == hipSuccess)
            e = launch_gemm(nullptr, &aq, M, K, w, c, ldc, rest + qb, rest_bytes - qb, cus, stream);
    }
    return e == hipSuccess ? NVFP4_OK : NVFP4_ERR_LAUNCH;
}

nvfp4_status nvfp4_gemm_fp8a(const uint8_t *a_fp8, const float *a_scale, int64_t M, int64_t lda,
                             const nvfp4_tensor *w, float *c, int64_t ldc, void *workspace, size_t workspace_bytes,
                             hipStream_t stream) {
    if (!a_scale) return NVFP4_ERR_NULL;
    nvfp4_status st = check_qtensor(w);
    if (st != NVFP4_OK) return st;
    const int64_t N = w->rows, K = w->cols;
    if (M < 0) return NVFP4_ERR_SHAPE;
    st = check_matrix(a_fp8, M, K, lda, 1);
    if (st != NVFP4_OK) return st;
    st = check_matrix(c, M, N, ldc, 4, 4);
    if (st != NVFP4_OK) return st;
    if (!aligned4(a_scale)) return NVFP4_ERR_ALIGN;
    if (workspace && !aligned16(workspace)) return NVFP4_ERR_ALIGN;
    const int cus = current_device_cus();
    if (cus == 0) return NVFP4_ERR_DEVICE;
    hipError_t e = (K == 0) ? launch_fill_zero_f32(c, M, N, ldc, stream)
                            : launch_gemm_fp8(a_fp8, a_scale, M, lda, w, c, ldc, workspace, workspace_bytes, cus,
                                              stream);
    return e == hipSuccess ? NVFP4_OK : NVFP4_ERR_LAUNCH;
}

nvfp4_status nvfp4_matrix_stats(const void *w, nvfp4_dtype w_dtype, int64_t rows, int64_t cols, int64_t ld_w,
                                const nvfp4_tensor *q, double *out, void *workspace, size_t workspace_bytes,
                                hipStream_t stream) {
    if (w_dtype != NVFP4_F32 && w_dtype != NVFP4_BF16 && w_dtype != NVFP4_F16) return NVFP4_ERR_DTYPE;
    if (!out) return NVFP4_ERR_NULL;
    nvfp4_status st = check_matrix(w, rows, cols, ld_w, elem_bytes(w_dtype));
    if (st != NVFP4_OK) return st;
    if (rows < 1 || cols < 1 || (cols % 16) != 0) return NVFP4_ERR_SHAPE;
    if (rows > 1 && ld_w != cols && cols > (int64_t(1) << 30)) return NVFP4_ERR_SHAPE;  // 32-bit column split
    if (q) {
        st = check_qtensor(q);
        if (st != NVFP4_OK) return st;
        if (q->rows != rows || q->cols != cols) return NVFP4_ERR_SHAPE;
    }
    if ((reinterpret_cast<uintptr_t>(out) & 7u) != 0) return NVFP4_ERR_ALIGN;
    if (!workspace || workspace_bytes < stats_ws_bytes()) return NVFP4_ERR_WORKSPACE;
    if (!aligned16(workspace)) return NVFP4_ERR_ALIGN;
    const int cus = current_device_cus();
    if (cus == 0) return NVFP4_ERR_DEVICE;
    hipError_t e = launch_stats(w, w_dtype, rows, cols, ld_w, q, out, workspace, cus, stream);
    return e == hipSuccess ? NVFP4_OK : NVFP4_ERR_LAUNCH;
}

nvfp4_status amax_percentile(const void *x, nvfp4_dtype x_dtype, int64_t rows, int64_t cols, int64_t ld_x, double p,
                             int per_channel, float *out_pct, float *out_max, int32_t *flags, void *workspace,
                             size_t workspace_bytes, hipStream_t stream) {
    if (x_dtype != NVFP4_F32 && x_dtype != NVFP4_BF16 && x_dtype != NVFP4_F16) return NVFP4_ERR_DTYPE;
    if (!out_pct) return NVFP4_ERR_NULL;
    nvfp4_status st = check_matrix(x, rows, cols, ld_x, elem_bytes(x_dtype));
    if (st != NVFP4_OK) return st;
    if (rows < 1 || cols < 1 || (cols % 16) != 0) return NVFP4_ERR_SHAPE;
    if (!(p > 0.0 && p <= 100.0) || (per_channel != 0 && per_channel != 1)) return NVFP4_ERR_ARG;
    const int64_t n = per_channel ? rows : rows * cols;
    if (n > (int64_t)0xFFFFFFFFll) return NVFP4_ERR_SHAPE;
    if (!aligned4(out_pct) || (out_max && !aligned4(out_max)) || (flags && !aligned4(flags))) return NVFP4_ERR_ALIGN;
    if (!workspace || workspace_bytes < percentile_ws_min_bytes(cols, per_channel)) return NVFP4_ERR_WORKSPACE;
    if (!aligned16(workspace)) return NVFP4_ERR_ALIGN;
    const int cus = current_device_cus();
    if (cus == 0) return NVFP4_ERR_DEVICE;
    // nearest rank, computed once here in double
    double kk = std::ceil(p * (double)n / 100.0);
    if (kk < 1.0) kk = 1.0;
    if (kk > (double)n) kk = (double)n;
    hipError_t e = launch_percentile(x, x_dtype, rows, cols, ld_x, (uint32_t)kk, per_channel, out_pct, out_max, flags,
                                     workspace, workspace_bytes, cus, stream);
    return e == hipSuccess ? NVFP4_OK : NVFP4_ERR_LAUNCH;
}

}  // extern "C"
