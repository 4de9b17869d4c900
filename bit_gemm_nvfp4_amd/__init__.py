"""bit_gemm_nvfp4_amd -- NVFP4 quantization, expansion, NVFP4-weight GEMM and percentile
calibration on AMD Instinct MI355X (gfx950).

A thin ctypes binding over ``libnvfp4.so`` (C ABI in ``include/nvfp4.h``).  This module only
marshals arguments: every step of the computation runs in the library's HIP kernels.  PyTorch is
used for device memory and the current stream.  There is no fallback path: the library is loaded
at the first call (so that ``python -m bit_gemm_nvfp4_amd.build`` works in a tree where it is not
built yet), and every entry point raises if it is missing.
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libnvfp4.so")

# ------------------------------------------------------------------------------------------------
# C ABI declarations
# ------------------------------------------------------------------------------------------------
NVFP4_F32, NVFP4_BF16, NVFP4_F16, NVFP4_E4M3 = 0, 1, 2, 3
OP_QUANTIZE, OP_DEQUANTIZE, OP_GEMM, OP_PERCENTILE, OP_STATS, OP_LOWRANK, OP_GEMM_QA, OP_AMAX = 0, 1, 2, 3, 4, 5, 6, 7
STATUS_NAMES = ["NVFP4_OK", "NVFP4_ERR_NULL", "NVFP4_ERR_SHAPE", "NVFP4_ERR_ALIGN", "NVFP4_ERR_DTYPE",
                "NVFP4_ERR_WORKSPACE", "NVFP4_ERR_ARG", "NVFP4_ERR_DEVICE", "NVFP4_ERR_LAUNCH"]
EXPORTED = ["nvfp4_quantize", "nvfp4_quantize_batch", "nvfp4_quantize_noalloc", "nvfp4_quantize_fp8", "nvfp4_tensor_amax", "nvfp4_dequantize", "nvfp4_gemm",
            "nvfp4_gemm_fp8a", "nvfp4_matrix_stats", "nvfp4_gemm_lowrank", "nvfp4_gemm_qa", "amax_percentile",
            "nvfp4_workspace_size", "nvfp4_status_string"]
# bits of the quantize `flags` word
FLAG_NONFINITE, FLAG_GRID_WAIT, FLAG_BAD_WORKSPACE = 1, 2, 4


class CTensor(ctypes.Structure):
    """Mirror of `nvfp4_tensor`."""
    _fields_ = [("codes", ctypes.c_void_p), ("scales", ctypes.c_void_p), ("global_scale", ctypes.c_void_p),
                ("rows", ctypes.c_int64), ("cols", ctypes.c_int64)]


_P, _I64, _I32, _SZ, _D = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int, ctypes.c_size_t, ctypes.c_double
_PT = ctypes.POINTER(CTensor)
_SIGNATURES = {
    "nvfp4_quantize": [_P, _I32, _I64, _P, _P, _PT, _P, _P, _SZ, _P],
    "nvfp4_quantize_noalloc": [_P, _I32, _I64, _P, _P, _PT, _P, _P],
    "nvfp4_quantize_batch": [_I32, _P, _I32, _P, _P, _P, _P, _P, _SZ, _P],
    "nvfp4_quantize_fp8": [_P, _I32, _I64, _I64, _I64, _P, _P, _P, _P, _P, _P, _SZ, _P],
    "nvfp4_tensor_amax": [_P, _I32, _I64, _I64, _I64, _P, _P, _P, _P, _SZ, _P],
    "nvfp4_gemm_fp8a": [_P, _P, _I64, _I64, _PT, _P, _I64, _P, _SZ, _P],
    "nvfp4_matrix_stats": [_P, _I32, _I64, _I64, _I64, _PT, _P, _P, _SZ, _P],
    "nvfp4_dequantize": [_PT, _P, _I32, _I64, _P],
    "nvfp4_gemm": [_P, _PT, _I64, _I64, _PT, _P, _I64, _P, _SZ, _P],
    "nvfp4_gemm_lowrank": [_P, _PT, _I64, _I64, _PT, _P, _P, _I64, _P, _I64, _P, _SZ, _P],
    "nvfp4_gemm_qa": [_P, _P, _I64, _I64, _PT, _P, _I64, _P, _SZ, _P],
    "amax_percentile": [_P, _I32, _I64, _I64, _I64, _D, _I32, _P, _P, _P, _P, _SZ, _P],
    "nvfp4_workspace_size": [_I32, _I64, _I64, _I64],
    "nvfp4_status_string": [_I32],
}
_RESTYPES = {"nvfp4_workspace_size": _SZ, "nvfp4_status_string": ctypes.c_char_p}

_lib = None


def load_library() -> ctypes.CDLL:
    """The loaded ``libnvfp4.so`` with its signatures declared; raises if it is not built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is not built; run `python -m bit_gemm_nvfp4_amd.build` first "
                               "(there is no fallback path)")
        lib = ctypes.CDLL(LIB_PATH)
        for name, args in _SIGNATURES.items():
            fn = getattr(lib, name)
            fn.argtypes = args
            fn.restype = _RESTYPES.get(name, _I32)
        _lib = lib
    return _lib


def __getattr__(name):
    if name == "lib":
        return load_library()
    raise AttributeError(f"module {__name__!r} has no attribute {name!r}")


class NVFP4Error(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        name = STATUS_NAMES[status] if 0 <= status < len(STATUS_NAMES) else str(status)
        super().__init__(f"{where}: {name} ({load_library().nvfp4_status_string(status).decode()})")


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
    in the low nibble of byte j), scales [rows, cols/16] uint8 (E4M3 bits), global_scale [1] fp32.
    `flags` is the device int32 word the producing quantize call ORed its status bits into
    (FLAG_NONFINITE, FLAG_GRID_WAIT, FLAG_BAD_WORKSPACE), or None."""
    codes: torch.Tensor
    scales: torch.Tensor
    global_scale: torch.Tensor
    flags: torch.Tensor | None = None

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
        for t in (self.codes, self.scales):
            assert t.is_contiguous(), "NVFP4 codes and scales must be dense"
        return CTensor(self.codes.data_ptr(), self.scales.data_ptr(), self.global_scale.data_ptr(), r, c)


@dataclass
class FP8Tensor:
    """FP8 E4M3 tensor with one tensor scale: data [rows, cols] uint8 (E4M3 bit patterns), scale [1]
    fp32; element value = e4m3(byte) x scale.  `flags` as for NVFP4Tensor."""
    data: torch.Tensor
    scale: torch.Tensor
    flags: torch.Tensor | None = None

    @property
    def shape(self):
        return tuple(self.data.shape)

    @staticmethod
    def empty(rows: int, cols: int, device) -> "FP8Tensor":
        return FP8Tensor(torch.empty((rows, cols), dtype=torch.uint8, device=device),
                         torch.empty(1, dtype=torch.float32, device=device))


def workspace_size(op: int, rows: int, cols: int, k: int = 0) -> int:
    return int(load_library().nvfp4_workspace_size(op, rows, cols, k))


def _workspace(nbytes: int, device) -> torch.Tensor | None:
    return torch.empty(max(nbytes, 1), dtype=torch.uint8, device=device) if nbytes > 0 else None


def quantize_workspace(device) -> torch.Tensor:
    """A workspace for the one-launch run-time-amax quantizers: zeroed, as the library requires
    before its first use; afterwards it carries a call counter and needs no clearing.  Calls that
    share one must be ordered (same stream, or events)."""
    return torch.zeros(workspace_size(OP_QUANTIZE, 0, 0), dtype=torch.uint8, device=device)


def _row_stride(t: torch.Tensor, what: str, cols: int | None = None) -> int:
    """Row stride (elements) of a 2-D row-major tensor whose elements within a row are contiguous
    (the C ABI takes a row stride only); checks the column count when given."""
    assert t.dim() == 2, f"{what}: a 2-D tensor is required"
    if cols is not None:
        assert t.shape[1] == cols, f"{what}: {t.shape[1]} columns, expected {cols}"
    if t.numel() == 0:
        return t.shape[1]
    assert t.shape[1] <= 1 or t.stride(1) == 1, f"{what}: elements of a row must be contiguous (stride(1) == 1)"
    return t.stride(0) if t.shape[0] > 1 else t.shape[1]


def _rows(t: torch.Tensor, what: str, cols: int | None = None) -> int:
    assert t.is_cuda, f"{what}: a device tensor is required"
    return _row_stride(t, what, cols)


def check_flags(flags: torch.Tensor | None, where: str = "quantize") -> None:
    """Synchronise on a quantize `flags` word and raise if any status bit is set."""
    if flags is None:
        return
    f = int(flags.item())
    if f:
        what = [n for b, n in ((FLAG_NONFINITE, "non-finite input"),
                               (FLAG_GRID_WAIT, "run-time amax not agreed within the bounded wait "
                                                "(other kernels held compute units; use two_pass=True)"),
                               (FLAG_BAD_WORKSPACE, "workspace not zeroed before first use, or shared by "
                                                    "overlapping calls")) if f & b]
        raise RuntimeError(f"{where}: flags {f:#x}: " + "; ".join(what) + " -- the outputs are invalid")


# ------------------------------------------------------------------------------------------------
# entry points
# ------------------------------------------------------------------------------------------------
def tensor_amax(x: torch.Tensor, src_scale: torch.Tensor | None = None, flags: torch.Tensor | None = None,
                out: torch.Tensor | None = None, workspace: torch.Tensor | None = None) -> torch.Tensor:
    """amax = max |x| (fp32 [1] on the device; E4M3 bytes times src_scale) in a pass of its own:
    the first launch of the two-launch run-time quantize."""
    ld = _rows(x, "x")
    rows, cols = x.shape
    if out is None:
        out = torch.empty(1, dtype=torch.float32, device=x.device)
    ws_bytes = workspace_size(OP_AMAX, rows, cols)
    ws = workspace if workspace is not None else _workspace(ws_bytes, x.device)
    st = load_library().nvfp4_tensor_amax(_ptr(x), _DT[x.dtype], rows, cols, ld, _ptr(src_scale), _ptr(out),
                                          _ptr(flags), _ptr(ws), ws.numel(), _stream(x.device))
    _check(st, "nvfp4_tensor_amax")
    return out


def _run_time_setup(x, amax, flags, workspace, two_pass, src_scale):
    """Shared by the two quantizers: a flags word (allocated, zeroed, when the caller gives none)
    and, for the run-time amax, either a zeroed workspace (one launch) or the amax pass (two)."""
    if flags is None:
        flags = torch.zeros(1, dtype=torch.int32, device=x.device)
    if amax is None and two_pass:
        amax = tensor_amax(x, src_scale=src_scale, flags=flags)
    elif amax is None and workspace is None:
        workspace = quantize_workspace(x.device)
    return amax, flags, (workspace if amax is None else None)


def quantize(x: torch.Tensor, amax: torch.Tensor | None = None, src_scale: torch.Tensor | None = None,
             flags: torch.Tensor | None = None, out: NVFP4Tensor | None = None,
             workspace: torch.Tensor | None = None, two_pass: bool = False, check: bool = False) -> NVFP4Tensor:
    """Quantize a 2-D device tensor (fp32, bf16, fp16, or float8_e4m3fn / uint8 E4M3 bytes) to NVFP4.
    amax: optional device fp32 [1] static amax; src_scale: optional device fp32 [1] per-tensor scale
    of an E4M3 source.  flags: device int32 [1] that the call ORs its status into (bit 0 non-finite
    input, bit 1 run-time amax not agreed within the bounded wait, bit 2 workspace not in the state
    the last call left it in); allocated and zeroed when not given, and returned as `out.flags`.
    workspace: for the one-launch run-time amax, a buffer from quantize_workspace() (zeroed before
    its first use); a fresh one is made when not given.  two_pass: take the run-time amax in a pass
    of its own first (no requirement that the grid be resident at once; identical outputs).
    check: synchronise and raise if any flag bit is set."""
    ld = _rows(x, "x")
    rows, cols = x.shape
    if out is None:
        out = NVFP4Tensor.empty(rows, cols, x.device)
    amax, flags, workspace = _run_time_setup(x, amax, flags, workspace, two_pass, src_scale)
    ct = out.c()
    ct.rows, ct.cols = rows, cols
    st = load_library().nvfp4_quantize(_ptr(x), _DT[x.dtype], ld, _ptr(src_scale), _ptr(amax), ctypes.byref(ct),
                                       _ptr(flags), _ptr(workspace), 0 if workspace is None else workspace.numel(),
                                       _stream(x.device))
    _check(st, "nvfp4_quantize")
    out.flags = flags
    if check:
        check_flags(flags, "nvfp4_quantize")
    return out


QUANTIZE_MAX_BATCH = 8


def quantize_batch(xs, src_scales=None, outs=None, flags: torch.Tensor | None = None,
                   workspace: torch.Tensor | None = None, check: bool = False) -> list:
    """Quantize up to 8 device tensors of one dtype to NVFP4, each with its own run-time amax, in one
    launch where they fit on chip together (else one launch each): the results of quantize() on
    each.  src_scales: None, or one device fp32 [1] tensor (or None) per tensor (E4M3 sources).
    flags: one int32 word for the whole batch (allocated and zeroed when not given; returned as the
    `flags` of every output).  workspace: as for quantize()."""
    xs = list(xs)
    n = len(xs)
    assert n <= QUANTIZE_MAX_BATCH, f"at most {QUANTIZE_MAX_BATCH} tensors per batch"
    if n == 0:
        return []
    dev = xs[0].device
    assert all(x.dtype == xs[0].dtype and x.device == dev for x in xs), "one dtype and device per batch"
    lds = [_rows(x, f"xs[{i}]") for i, x in enumerate(xs)]
    if outs is None:
        outs = [NVFP4Tensor.empty(x.shape[0], x.shape[1], dev) for x in xs]
    if flags is None:
        flags = torch.zeros(1, dtype=torch.int32, device=dev)
    if workspace is None:
        workspace = quantize_workspace(dev)
    cts = (CTensor * n)()
    for i, (x, o) in enumerate(zip(xs, outs)):
        cts[i] = o.c()
        cts[i].rows, cts[i].cols = x.shape
    xp = (ctypes.c_void_p * n)(*[x.data_ptr() for x in xs])
    ldp = (ctypes.c_int64 * n)(*lds)
    scp = None
    if src_scales is not None:
        assert len(src_scales) == n
        scp = (ctypes.c_void_p * n)(*[None if s is None else s.data_ptr() for s in src_scales])
    st = load_library().nvfp4_quantize_batch(n, xp, _DT[xs[0].dtype], ldp, scp, cts, _ptr(flags), _ptr(workspace),
                                             workspace.numel(), _stream(dev))
    _check(st, "nvfp4_quantize_batch")
    for o in outs:
        o.flags = flags
    if check:
        check_flags(flags, "nvfp4_quantize_batch")
    return outs


def quantize_noalloc(x: torch.Tensor, out: NVFP4Tensor, amax: torch.Tensor | None = None,
                     src_scale: torch.Tensor | None = None, flags: torch.Tensor | None = None) -> NVFP4Tensor:
    """quantize() for callers that cannot allocate: the outputs (and the optional flags word) come
    from the caller, and the run-time amax agreement uses the library's own per-GPU scratch instead of
    a workspace.  Nothing is allocated.  Calls that overlap on one GPU race on that scratch."""
    ld = _rows(x, "x")
    rows, cols = x.shape
    assert out.shape == (rows, cols), f"out: shape {out.shape}, expected {(rows, cols)}"
    ct = out.c()
    st = load_library().nvfp4_quantize_noalloc(_ptr(x), _DT[x.dtype], ld, _ptr(src_scale), _ptr(amax),
                                               ctypes.byref(ct), _ptr(flags), _stream(x.device))
    _check(st, "nvfp4_quantize_noalloc")
    out.flags = flags
    return out


def quantize_fp8(x: torch.Tensor, amax: torch.Tensor | None = None, src_scale: torch.Tensor | None = None,
                 flags: torch.Tensor | None = None, out: FP8Tensor | None = None,
                 workspace: torch.Tensor | None = None, two_pass: bool = False, check: bool = False) -> FP8Tensor:
    """FP8 E4M3 tensorwise quantization of a 2-D device tensor (fp32, bf16, fp16 or E4M3 bytes):
    scale = amax / 448 (run-time amax, or the static `amax`), bytes = nearest E4M3 of x / scale.
    flags, workspace, two_pass and check as for quantize()."""
    ld = _rows(x, "x")
    rows, cols = x.shape
    if out is None:
        out = FP8Tensor.empty(rows, cols, x.device)
    assert out.data.is_contiguous() and tuple(out.data.shape) == (rows, cols)
    amax, flags, workspace = _run_time_setup(x, amax, flags, workspace, two_pass, src_scale)
    st = load_library().nvfp4_quantize_fp8(_ptr(x), _DT[x.dtype], rows, cols, ld, _ptr(src_scale), _ptr(amax),
                                           _ptr(out.data), _ptr(out.scale), _ptr(flags), _ptr(workspace),
                                           0 if workspace is None else workspace.numel(), _stream(x.device))
    _check(st, "nvfp4_quantize_fp8")
    out.flags = flags
    if check:
        check_flags(flags, "nvfp4_quantize_fp8")
    return out


def dequantize(q: NVFP4Tensor, dtype: torch.dtype = torch.bfloat16, out: torch.Tensor | None = None) -> torch.Tensor:
    """Expand NVFP4 to bf16 or fp32: w = e2m1 x block scale x global scale."""
    rows, cols = q.shape
    if out is None:
        out = torch.empty((rows, cols), dtype=dtype, device=q.codes.device)
    assert out.shape[0] == rows
    ld = _rows(out, "out", cols)
    ct = q.c()
    st = load_library().nvfp4_dequantize(ctypes.byref(ct), _ptr(out), _DT[out.dtype], ld, _stream(q.codes.device))
    _check(st, "nvfp4_dequantize")
    return out


def _gemm_out(out, m, n, device):
    if out is None:
        out = torch.empty((m, n), dtype=torch.float32, device=device)
    assert out.dtype == torch.float32 and out.shape[0] == m
    return out, _rows(out, "out", n)


def gemm(a: torch.Tensor | NVFP4Tensor | FP8Tensor, w: NVFP4Tensor, out: torch.Tensor | None = None) -> torch.Tensor:
    """C [M, N] fp32 = A . W_hat^T.  `a` is a bf16 [M, K] tensor (W4A16), an NVFP4Tensor (W4A4) or an
    FP8Tensor (FP8 activations)."""
    n, k = w.shape
    device = w.codes.device
    lib = load_library()
    if isinstance(a, FP8Tensor):
        m = a.shape[0]
        lda = _rows(a.data, "a", k)
        out, ldc = _gemm_out(out, m, n, device)
        ws_bytes = workspace_size(OP_GEMM, m, n, k)
        ws = _workspace(ws_bytes, device)
        wct = w.c()
        st = lib.nvfp4_gemm_fp8a(_ptr(a.data), _ptr(a.scale), m, lda, ctypes.byref(wct), _ptr(out), ldc, _ptr(ws),
                                 ws_bytes, _stream(device))
        _check(st, "nvfp4_gemm_fp8a")
        return out
    if isinstance(a, NVFP4Tensor):
        m = a.shape[0]
        assert a.shape[1] == k, f"a: {a.shape[1]} columns, expected {k}"
        a_ct, a_ptr, lda = ctypes.byref(a.c()), None, k
    else:
        assert a.dtype == torch.bfloat16
        lda = _rows(a, "a", k)
        m = a.shape[0]
        if a.numel() == 0:  # the W4A16 form is selected by a non-NULL pointer, even with no elements
            a = torch.empty(8, dtype=torch.bfloat16, device=device)
            lda = (k + 7) // 8 * 8 or 8
        a_ct, a_ptr = None, _ptr(a)
    out, ldc = _gemm_out(out, m, n, device)
    ws_bytes = workspace_size(OP_GEMM, m, n, k)
    ws = _workspace(ws_bytes, device)
    wct = w.c()
    st = lib.nvfp4_gemm(a_ptr, a_ct, m, lda, ctypes.byref(wct), _ptr(out), ldc, _ptr(ws), ws_bytes, _stream(device))
    _check(st, "nvfp4_gemm")
    return out


def gemm_qa_workspace(m: int, n: int, k: int, device) -> torch.Tensor:
    """A workspace for gemm_qa on [m, k] activations and an [n, k] weight: zeroed, as the library
    requires of its first bytes (the staged form's group counters) before their first use; every
    call leaves them zero, so it can be reused for any shape it is large enough for.  Calls that
    share one must be ordered (same stream, or events)."""
    return torch.zeros(max(workspace_size(OP_GEMM_QA, m, n, k), 1), dtype=torch.uint8, device=device)


def gemm_qa(a: torch.Tensor, w: NVFP4Tensor, amax: torch.Tensor, out: torch.Tensor | None = None,
            workspace: torch.Tensor | None = None) -> torch.Tensor:
    """C [M, N] fp32 = A_hat . W_hat^T with A (bf16 [M, K]) quantized to NVFP4 inside the GEMM under
    the static amax (a float32 device tensor of one element)."""
    n, k = w.shape
    device = w.codes.device
    assert a.dtype == torch.bfloat16
    lda = _rows(a, "a", k)
    assert amax.dtype == torch.float32 and amax.is_cuda and amax.numel() == 1
    m = a.shape[0]
    out, ldc = _gemm_out(out, m, n, device)
    ws_bytes = workspace_size(OP_GEMM_QA, m, n, k)
    ws = workspace if workspace is not None else gemm_qa_workspace(m, n, k, device)
    wct = w.c()
    st = load_library().nvfp4_gemm_qa(_ptr(a), _ptr(amax), m, lda, ctypes.byref(wct), _ptr(out), ldc, _ptr(ws),
                                      ws.numel() if workspace is not None else ws_bytes, _stream(device))
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
    assert a.dtype == torch.bfloat16
    lda = _rows(a, "a", k)
    assert lr_down.dtype == torch.bfloat16 and lr_up.dtype == torch.bfloat16
    assert lr_down.is_contiguous() and lr_up.is_contiguous()
    m, rank = a.shape[0], lr_down.shape[0]
    assert tuple(lr_down.shape) == (rank, k) and tuple(lr_up.shape) == (n, rank)
    out, ldc = _gemm_out(out, m, n, device)
    ws_bytes = workspace_size(OP_LOWRANK, m, n, k)
    ws = workspace if workspace is not None else _workspace(ws_bytes, device)
    wct = w.c()
    a_ct = ctypes.byref(a_q.c()) if a_q is not None else None
    st = load_library().nvfp4_gemm_lowrank(_ptr(a), a_ct, m, lda, ctypes.byref(wct), _ptr(lr_down), _ptr(lr_up),
                                           rank, _ptr(out), ldc, _ptr(ws),
                                           ws.numel() if workspace is not None else ws_bytes, _stream(device))
    _check(st, "nvfp4_gemm_lowrank")
    return out


def amax_percentile(x: torch.Tensor, p: float = 99.9, per_channel: bool = True,
                    flags: torch.Tensor | None = None, with_max: bool = True):
    """Nearest-rank p-th percentile (and maximum) of |x| per column, or over the whole tensor."""
    ld = _rows(x, "x")
    rows, cols = x.shape
    n_out = cols if per_channel else 1
    pct = torch.empty(n_out, dtype=torch.float32, device=x.device)
    mx = torch.empty(n_out, dtype=torch.float32, device=x.device) if with_max else None
    ws_bytes = workspace_size(OP_PERCENTILE, rows, cols, 1 if per_channel else 0)
    ws = _workspace(ws_bytes, x.device)
    st = load_library().amax_percentile(_ptr(x), _DT[x.dtype], rows, cols, ld, float(p), 1 if per_channel else 0,
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
    ld = _rows(w, "w")
    rows, cols = w.shape
    ret = out
    if out is None:
        out = torch.empty(8, dtype=torch.float64, device=w.device)
    assert out.dtype == torch.float64 and out.is_contiguous() and out.numel() >= 7
    ws_bytes = workspace_size(OP_STATS, 0, 0)
    ws = workspace if workspace is not None else _workspace(ws_bytes, w.device)
    qc = q.c() if q is not None else None
    st = load_library().nvfp4_matrix_stats(_ptr(w), _DT[w.dtype], rows, cols, ld,
                                           ctypes.byref(qc) if qc else None, _ptr(out), _ptr(ws),
                                           ws.numel() if workspace is not None else ws_bytes, _stream(w.device))
    _check(st, "nvfp4_matrix_stats")
    if ret is not None:
        return ret
    return dict(zip(STAT_FIELDS, out[:7].cpu().tolist()))
