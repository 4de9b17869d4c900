"""bit_gemm_nvfp4_amd -- NVFP4 quantization, expansion, NVFP4-weight GEMM and percentile
calibration on AMD Instinct MI355X (gfx950).

A thin ctypes binding over ``libnvfp4.so`` (C ABI in ``include/nvfp4.h``).  This module only
marshals arguments: every step of the computation runs in the library's HIP kernels.  PyTorch is
used for device memory and the current stream.  There is no fallback path: if the library is
missing, importing this package fails.
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libnvfp4.so")

if not os.path.exists(LIB_PATH):
    raise ImportError(f"{LIB_PATH} is not built; run `python -m bit_gemm_nvfp4_amd.build` first")

lib = ctypes.CDLL(LIB_PATH)

# ------------------------------------------------------------------------------------------------
# C ABI declarations
# ------------------------------------------------------------------------------------------------
NVFP4_F32, NVFP4_BF16, NVFP4_F16, NVFP4_E4M3 = 0, 1, 2, 3
OP_QUANTIZE, OP_DEQUANTIZE, OP_GEMM, OP_PERCENTILE, OP_STATS, OP_LOWRANK, OP_GEMM_QA = 0, 1, 2, 3, 4, 5, 6
STATUS_NAMES = ["NVFP4_OK", "NVFP4_ERR_NULL", "NVFP4_ERR_SHAPE", "NVFP4_ERR_ALIGN", "NVFP4_ERR_DTYPE",
                "NVFP4_ERR_WORKSPACE", "NVFP4_ERR_ARG", "NVFP4_ERR_DEVICE", "NVFP4_ERR_LAUNCH"]
EXPORTED = ["nvfp4_quantize", "nvfp4_quantize_fp8", "nvfp4_dequantize", "nvfp4_gemm", "nvfp4_gemm_fp8a",
            "nvfp4_matrix_stats", "nvfp4_gemm_lowrank", "nvfp4_gemm_qa", "amax_percentile", "nvfp4_workspace_size", "nvfp4_status_string"]


class CTensor(ctypes.Structure):
    """Mirror of `nvfp4_tensor`."""
    _fields_ = [("codes", ctypes.c_void_p), ("scales", ctypes.c_void_p), ("global_scale", ctypes.c_void_p),
                ("rows", ctypes.c_int64), ("cols", ctypes.c_int64)]


_P, _I64, _I32, _SZ, _D = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int, ctypes.c_size_t, ctypes.c_double
_PT = ctypes.POINTER(CTensor)
lib.nvfp4_quantize.argtypes = [_P, _I32, _I64, _P, _P, _PT, _P, _P, _SZ, _P]
lib.nvfp4_quantize.restype = _I32
lib.nvfp4_quantize_fp8.argtypes = [_P, _I32, _I64, _I64, _I64, _P, _P, _P, _P, _P, _P, _SZ, _P]
lib.nvfp4_quantize_fp8.restype = _I32
lib.nvfp4_gemm_fp8a.argtypes = [_P, _P, _I64, _I64, _PT, _P, _I64, _P, _SZ, _P]
lib.nvfp4_gemm_fp8a.restype = _I32
lib.nvfp4_matrix_stats.argtypes = [_P, _I32, _I64, _I64, _I64, _PT, _P, _P, _SZ, _P]
lib.nvfp4_matrix_stats.restype = _I32
lib.nvfp4_dequantize.argtypes = [_PT, _P, _I32, _I64, _P]
lib.nvfp4_dequantize.restype = _I32
lib.nvfp4_gemm.argtypes = [_P, _PT, _I64, _I64, _PT, _P, _I64, _P, _SZ, _P]
lib.nvfp4_gemm_lowrank.argtypes = [_P, _PT, _I64, _I64, _PT, _P, _P, _I64, _P, _I64, _P, _SZ, _P]
lib.nvfp4_gemm_lowrank.restype = _I32
lib.nvfp4_gemm_qa.argtypes = [_P, _P, _I64, _I64, _PT, _P, _I64, _P, _SZ, _P]
lib.nvfp4_gemm_qa.restype = _I32
lib.nvfp4_gemm.restype = _I32
lib.amax_percentile.argtypes = [_P, _I32, _I64, _I64, _I64, _D, _I32, _P, _P, _P, _P, _SZ, _P]
lib.amax_percentile.restype = _I32
lib.nvfp4_workspace_size.argtypes = [_I32, _I64, _I64, _I64]
lib.nvfp4_workspace_size.restype = _SZ
lib.nvfp4_status_string.argtypes = [_I32]
lib.nvfp4_status_string.restype = ctypes.c_char_p


class NVFP4Error(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        name = STATUS_NAMES[status] if 0 <= status < len(STATUS_NAMES) else str(status)
        super().__init__(f"{where}: {name} ({lib.nvfp4_status_string(status).decode()})")


def _check(status: int, where: str) -> None:
    if status != 0:
        raise NVFP4Error(status, where)


def _ptr(t: torch.Tensor | None):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(device: torch.device):
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


_DT = {torch.float32: NVFP4_F32, torch.bfloat16: NVFP4_BF16, torch.float16: NVFP4_F16,
       torch.float8_e4m3fn: NVFP4_E4M3, torch.uint8: NVFP4_E4M3}


# ------------------------------------------------------------------------------------------------
# NVFP4 tensor
# ------------------------------------------------------------------------------------------------
@dataclass
class NVFP4Tensor:
    """Packed NVFP4 tensor of logical shape [rows, cols]: codes [rows, cols/2] uint8 (element 2j
    in the low nibble of byte j), scales [rows, cols/16] uint8 (E4M3 bits), global_scale [1] fp32."""
    codes: torch.Tensor
    scales: torch.Tensor
    global_scale: torch.Tensor

    @property
    def shape(self):
        return (self.codes.shape[0], self.codes.shape[1] * 2)

    @staticmethod
    def empty(rows: int, cols: int, device) -> "NVFP4Tensor":
        return NVFP4Tensor(torch.empty((rows, cols // 2), dtype=torch.uint8, device=device),
                           torch.empty((rows, cols // 16), dtype=torch.uint8, device=device),
                           torch.empty(1, dtype=torch.float32, device=device))

    def c(self) -> CTensor:
        r, c = self.shape
        return CTensor(self.codes.data_ptr(), self.scales.data_ptr(), self.global_scale.data_ptr(), r, c)


@dataclass
class FP8Tensor:
    """FP8 E4M3 tensor with one tensor scale: data [rows, cols] uint8 (E4M3 bit patterns), scale [1]
    fp32; element value = e4m3(byte) x scale."""
    data: torch.Tensor
    scale: torch.Tensor

    @property
    def shape(self):
        return tuple(self.data.shape)

    @staticmethod
    def empty(rows: int, cols: int, device) -> "FP8Tensor":
        return FP8Tensor(torch.empty((rows, cols), dtype=torch.uint8, device=device),
                         torch.empty(1, dtype=torch.float32, device=device))


def workspace_size(op: int, rows: int, cols: int, k: int = 0) -> int:
    return int(lib.nvfp4_workspace_size(op, rows, cols, k))


def _workspace(nbytes: int, device) -> torch.Tensor | None:
    return torch.empty(max(nbytes, 1), dtype=torch.uint8, device=device) if nbytes > 0 else None


# ------------------------------------------------------------------------------------------------
# entry points
# ------------------------------------------------------------------------------------------------
def quantize(x: torch.Tensor, amax: torch.Tensor | None = None, src_scale: torch.Tensor | None = None,
             flags: torch.Tensor | None = None, out: NVFP4Tensor | None = None,
             workspace: torch.Tensor | None = None) -> NVFP4Tensor:
    """Quantize a 2-D device tensor (fp32, bf16, fp16, or float8_e4m3fn / uint8 E4M3 bytes) to NVFP4.
    amax: optional device fp32 [1] static amax; src_scale: optional device fp32 [1] per-tensor scale
    of an E4M3 source; flags: optional device int32 [1] (bit 0 = non-finite input)."""
    assert x.dim() == 2 and x.is_cuda
    rows, cols = x.shape
    if out is None:
        out = NVFP4Tensor.empty(rows, cols, x.device)
    ct = out.c()
    ct.rows, ct.cols = rows, cols
    if workspace is None and amax is None:
        workspace = _workspace(workspace_size(OP_QUANTIZE, rows, cols), x.device)
    st = lib.nvfp4_quantize(_ptr(x), _DT[x.dtype], x.stride(0) if rows > 0 else cols, _ptr(src_scale), _ptr(amax),
                            ctypes.byref(ct), _ptr(flags), _ptr(workspace),
                            0 if workspace is None else workspace.numel(), _stream(x.device))
    _check(st, "nvfp4_quantize")
    return out


def quantize_fp8(x: torch.Tensor, amax: torch.Tensor | None = None, src_scale: torch.Tensor | None = None,
                 flags: torch.Tensor | None = None, out: FP8Tensor | None = None,
                 workspace: torch.Tensor | None = None) -> FP8Tensor:
    """FP8 E4M3 tensorwise quantization of a 2-D device tensor (fp32, bf16, fp16 or E4M3 bytes):
    scale = amax / 448 (run-time amax, or the static `amax`), bytes = nearest E4M3 of x / scale."""
    assert x.dim() == 2 and x.is_cuda
    rows, cols = x.shape
    if out is None:
        out = FP8Tensor.empty(rows, cols, x.device)
    if workspace is None and amax is None:
        workspace = _workspace(workspace_size(OP_QUANTIZE, rows, cols), x.device)
    st = lib.nvfp4_quantize_fp8(_ptr(x), _DT[x.dtype], rows, cols, x.stride(0) if rows > 0 else cols, _ptr(src_scale),
                                _ptr(amax), _ptr(out.data), _ptr(out.scale), _ptr(flags), _ptr(workspace),
                                0 if workspace is None else workspace.numel(), _stream(x.device))
    _check(st, "nvfp4_quantize_fp8")
    return out


def dequantize(q: NVFP4Tensor, dtype: torch.dtype = torch.bfloat16, out: torch.Tensor | None = None) -> torch.Tensor:
    """Expand NVFP4 to bf16 or fp32: w = e2m1 x block scale x global scale."""
    rows, cols = q.shape
    if out is None:
        out = torch.empty((rows, cols), dtype=dtype, device=q.codes.device)
    ct = q.c()
    st = lib.nvfp4_dequantize(ctypes.byref(ct), _ptr(out), _DT[out.dtype], out.stride(0) if rows > 0 else cols,
                              _stream(q.codes.device))
    _check(st, "nvfp4_dequantize")
    return out


def gemm(a: torch.Tensor | NVFP4Tensor | FP8Tensor, w: NVFP4Tensor, out: torch.Tensor | None = None) -> torch.Tensor:
    """C [M, N] fp32 = A . W_hat^T.  `a` is a bf16 [M, K] tensor (W4A16), an NVFP4Tensor (W4A4) or an
    FP8Tensor (FP8 activations)."""
    n, k = w.shape
    device = w.codes.device
    if isinstance(a, FP8Tensor):
        m = a.shape[0]
        if out is None:
            out = torch.empty((m, n), dtype=torch.float32, device=device)
        ws_bytes = workspace_size(OP_GEMM, m, n, k)
        ws = _workspace(ws_bytes, device)
        wct = w.c()
        st = lib.nvfp4_gemm_fp8a(_ptr(a.data), _ptr(a.scale), m, a.data.stride(0) if m > 0 else k, ctypes.byref(wct),
                                 _ptr(out), out.stride(0) if m > 0 else n, _ptr(ws), ws_bytes, _stream(device))
        _check(st, "nvfp4_gemm_fp8a")
        return out
    if isinstance(a, NVFP4Tensor):
        m = a.shape[0]
        a_ct, a_ptr, lda = ctypes.byref(a.c()), None, k
    else:
        assert a.dtype == torch.bfloat16 and a.dim() == 2
        m = a.shape[0]
        lda = a.stride(0)
        if a.numel() == 0:  # the W4A16 form is selected by a non-NULL pointer, even with no elements
            a = torch.empty(8, dtype=torch.bfloat16, device=device)
            lda = (k + 7) // 8 * 8 or 8
        a_ct, a_ptr = None, _ptr(a)
    if out is None:
        out = torch.empty((m, n), dtype=torch.float32, device=device)
    ws_bytes = workspace_size(OP_GEMM, m, n, k)
    ws = _workspace(ws_bytes, device)
    wct = w.c()
    st = lib.nvfp4_gemm(a_ptr, a_ct, m, lda, ctypes.byref(wct), _ptr(out), out.stride(0) if m > 0 else n, _ptr(ws),
                        ws_bytes, _stream(device))
    _check(st, "nvfp4_gemm")
    return out


def gemm_qa(a: torch.Tensor, w: NVFP4Tensor, amax: torch.Tensor, out: torch.Tensor | None = None,
            workspace: torch.Tensor | None = None) -> torch.Tensor:
    """C [M, N] fp32 = A_hat . W_hat^T with A (bf16 [M, K]) quantized to NVFP4 inside the GEMM under
    the static amax (a float32 device tensor of one element)."""
    n, k = w.shape
    device = w.codes.device
    assert a.dtype == torch.bfloat16 and a.dim() == 2 and a.shape[1] == k
    assert amax.dtype == torch.float32 and amax.is_cuda and amax.numel() == 1
    m = a.shape[0]
    if out is None:
        out = torch.empty((m, n), dtype=torch.float32, device=device)
    ws_bytes = workspace_size(OP_GEMM_QA, m, n, k)
    ws = workspace if workspace is not None else _workspace(ws_bytes, device)
    wct = w.c()
    st = lib.nvfp4_gemm_qa(_ptr(a), _ptr(amax), m, a.stride(0) if m > 0 else k, ctypes.byref(wct), _ptr(out),
                           out.stride(0) if m > 0 else n, _ptr(ws), ws.numel() if workspace is not None else ws_bytes,
                           _stream(device))
    _check(st, "nvfp4_gemm_qa")
    return out


def gemm_lowrank(a: torch.Tensor, w: NVFP4Tensor, lr_down: torch.Tensor, lr_up: torch.Tensor,
                 a_q: NVFP4Tensor | None = None, out: torch.Tensor | None = None,
                 workspace: torch.Tensor | None = None) -> torch.Tensor:
    """C [M, N] fp32 = A_hat . W_hat^T + (A . V^T) . U^T: the NVFP4 product plus a bf16 low-rank branch
    of the weight.  `a` bf16 [M, K] (the branch's activations, and the main product's unless `a_q`, an
    NVFP4Tensor [M, K], is given); lr_down V bf16 [r, K], lr_up U bf16 [N, r], both contiguous."""
    n, k = w.shape
    device = w.codes.device
    assert a.dtype == torch.bfloat16 and a.dim() == 2 and a.shape[1] == k
    assert lr_down.dtype == torch.bfloat16 and lr_up.dtype == torch.bfloat16
    assert lr_down.is_contiguous() and lr_up.is_contiguous()
    m, rank = a.shape[0], lr_down.shape[0]
    if out is None:
        out = torch.empty((m, n), dtype=torch.float32, device=device)
    ws_bytes = workspace_size(OP_LOWRANK, m, n, k)
    ws = workspace if workspace is not None else _workspace(ws_bytes, device)
    wct = w.c()
    a_ct = ctypes.byref(a_q.c()) if a_q is not None else None
    st = lib.nvfp4_gemm_lowrank(_ptr(a), a_ct, m, a.stride(0) if m > 0 else k, ctypes.byref(wct), _ptr(lr_down),
                                _ptr(lr_up), rank, _ptr(out), out.stride(0) if m > 0 else n, _ptr(ws),
                                ws.numel() if workspace is not None else ws_bytes, _stream(device))
    _check(st, "nvfp4_gemm_lowrank")
    return out


def amax_percentile(x: torch.Tensor, p: float = 99.9, per_channel: bool = True,
                    flags: torch.Tensor | None = None, with_max: bool = True):
    """Nearest-rank p-th percentile (and maximum) of |x| per column, or over the whole tensor."""
    assert x.dim() == 2 and x.is_cuda
    rows, cols = x.shape
    n_out = cols if per_channel else 1
    pct = torch.empty(n_out, dtype=torch.float32, device=x.device)
    mx = torch.empty(n_out, dtype=torch.float32, device=x.device) if with_max else None
    ws_bytes = workspace_size(OP_PERCENTILE, rows, cols, 1 if per_channel else 0)
    ws = _workspace(ws_bytes, x.device)
    st = lib.amax_percentile(_ptr(x), _DT[x.dtype], rows, cols, x.stride(0), float(p), 1 if per_channel else 0,
                             _ptr(pct), _ptr(mx), _ptr(flags), _ptr(ws), ws_bytes, _stream(x.device))
    _check(st, "amax_percentile")
    return pct, mx


STAT_FIELDS = ("rel_error", "kurtosis", "block_max_over_std", "mean", "std", "max_abs", "blocks")


def matrix_stats(w: torch.Tensor, q: NVFP4Tensor | None = None, out: torch.Tensor | None = None,
                 workspace: torch.Tensor | None = None):
    """Quality statistics of a 2-D weight (fp32, bf16 or fp16) and, if given, of its NVFP4 form:
    relative error, excess kurtosis, mean block-of-64 max|w| / std, mean, std, max |w|, blocks.
    Returns a dict (synchronising), or, when out (float64, >= 7 elements, on the device) is given,
    out itself with the fields in STAT_FIELDS order and no synchronisation."""
    assert w.dim() == 2 and w.is_cuda
    rows, cols = w.shape
    ret = out
    if out is None:
        out = torch.empty(8, dtype=torch.float64, device=w.device)
    assert out.dtype == torch.float64 and out.is_contiguous() and out.numel() >= 7
    ws_bytes = workspace_size(OP_STATS, 0, 0)
    ws = workspace if workspace is not None else _workspace(ws_bytes, w.device)
    qc = q.c() if q is not None else None
    st = lib.nvfp4_matrix_stats(_ptr(w), _DT[w.dtype], rows, cols, w.stride(0), ctypes.byref(qc) if qc else None,
                                _ptr(out), _ptr(ws), ws.numel() if workspace is not None else ws_bytes,
                                _stream(w.device))
    _check(st, "nvfp4_matrix_stats")
    if ret is not None:
        return ret
    return dict(zip(STAT_FIELDS, out[:7].cpu().tolist()))
