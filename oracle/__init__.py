"""CPU oracle for NVFP4 quantization, expansion, the NVFP4-weight GEMM and percentile calibration.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package.  The product path (``bit_gemm_nvfp4_amd``) never imports it
and shares no code with it.

The codec arithmetic lives in ``nvfp4_oracle.c`` (plain scalar C, built without fused multiply-add);
this module only marshals numpy arrays into it.  The GEMM reference is the plain definition
C = A_hat . W_hat^T evaluated in float64 with numpy's matmul over the exactly expanded operands
("Qwen-Image NVFP4 on a 16 GB Ada GPU", section "Running the NVFP4 weights on Ada": the weights are
expanded before each multiply; activations are bf16, or NVFP4 for the W4A4 form named in section
"What NVFP4 is and how it differs from NF4").  With a low-rank branch (reading R10: "Qwen Image 2.1:
INT4 + FP4", "What I quantized", FP4 weights with BF16 rank-128 branches) the same plain definition
gains the term (A . V^T) . U^T, also in float64.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "nvfp4_oracle.c")
_LIB_PATH = os.path.join(_HERE, "liboracle.so")

F32, BF16, F16, E4M3 = 0, 1, 2, 3
_DTYPE_OF = {np.dtype(np.float32): F32}

_lib = None


def build_library() -> str:
    """Compile the oracle with gcc (no fast-math, no FMA contraction)."""
    cmd = ["gcc", "-O2", "-std=c99", "-fPIC", "-shared", "-fno-fast-math", "-ffp-contract=off",
           "-Wall", "-Wextra", "-o", _LIB_PATH + ".tmp", _SRC, "-lm"]
    subprocess.check_call(cmd)
    os.replace(_LIB_PATH + ".tmp", _LIB_PATH)
    return _LIB_PATH


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        build_library()
    lib = ctypes.CDLL(_LIB_PATH)
    P, I64, D, I = ctypes.c_void_p, ctypes.c_int64, ctypes.c_double, ctypes.c_int
    lib.ref_e2m1_value.argtypes, lib.ref_e2m1_value.restype = [I], D
    lib.ref_e2m1_index.argtypes, lib.ref_e2m1_index.restype = [D], I
    lib.ref_e4m3_value.argtypes, lib.ref_e4m3_value.restype = [I], D
    lib.ref_e4m3_encode.argtypes, lib.ref_e4m3_encode.restype = [ctypes.c_float], I
    lib.ref_global_scale.argtypes, lib.ref_global_scale.restype = [ctypes.c_float], ctypes.c_float
    lib.ref_block_scale_byte.argtypes, lib.ref_block_scale_byte.restype = [ctypes.c_float, ctypes.c_float], I
    lib.ref_element_code.argtypes = [ctypes.c_float, ctypes.c_float, ctypes.c_float]
    lib.ref_element_code.restype = I
    lib.ref_widen.argtypes, lib.ref_widen.restype = [P, I, I64, I64, I64, P, P], None
    lib.ref_quantize_f32.argtypes, lib.ref_quantize_f32.restype = [P, I64, I64, P, P, P, P], I
    lib.ref_dequantize_f64.argtypes = [P, P, ctypes.c_float, I64, I64, P]
    lib.ref_dequantize_f32.argtypes = [P, P, ctypes.c_float, I64, I64, P]
    lib.ref_dequantize_bf16.argtypes = [P, P, ctypes.c_float, I64, I64, P]
    lib.ref_f32_to_bf16.argtypes, lib.ref_f32_to_bf16.restype = [ctypes.c_float], ctypes.c_uint16
    lib.ref_rank.argtypes, lib.ref_rank.restype = [D, I64], I64
    lib.ref_amax_percentile.argtypes = [P, I64, I64, D, I, P, P]
    lib.ref_e2m1_index_array.argtypes = [P, I64, P]
    lib.ref_e4m3_encode_array.argtypes = [P, I64, P]
    lib.ref_f32_to_bf16_array.argtypes = [P, I64, P]
    lib.ref_matrix_stats.argtypes = [P, I64, I64, P, P, ctypes.c_float, I, P]
    lib.ref_fp8_scale.argtypes, lib.ref_fp8_scale.restype = [ctypes.c_float], ctypes.c_float
    lib.ref_fp8_byte.argtypes, lib.ref_fp8_byte.restype = [ctypes.c_float, ctypes.c_float], I
    lib.ref_quantize_fp8_f32.argtypes, lib.ref_quantize_fp8_f32.restype = [P, I64, I64, P, P, P], I
    _lib = lib
    return lib


def _ptr(a: np.ndarray):
    return a.ctypes.data_as(ctypes.c_void_p)


# ------------------------------------------------------------------------------------------------
# scalar codec pieces
# ------------------------------------------------------------------------------------------------
def e2m1_value(code: int) -> float:
    return _load().ref_e2m1_value(int(code))


def e2m1_index(y: float) -> int:
    return _load().ref_e2m1_index(float(y))


def e4m3_value(b: int) -> float:
    return _load().ref_e4m3_value(int(b))


def e4m3_encode(t: float) -> int:
    return _load().ref_e4m3_encode(float(t))


def global_scale(amax: float) -> np.float32:
    return np.float32(_load().ref_global_scale(float(amax)))


def block_scale_byte(bamax: float, g: float) -> int:
    return _load().ref_block_scale_byte(float(bamax), float(g))


def element_code(v: float, s: float, g: float) -> int:
    return _load().ref_element_code(float(v), float(s), float(g))


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round-to-nearest-even fp32 -> bf16 bit patterns (uint16), elementwise."""
    flat = np.ascontiguousarray(x, dtype=np.float32).ravel()
    out = np.empty(flat.shape, dtype=np.uint16)
    _load().ref_f32_to_bf16_array(_ptr(flat), flat.size, _ptr(out))
    return out.reshape(np.shape(x))


def e2m1_index_array(y: np.ndarray) -> np.ndarray:
    """Nearest E2M1 magnitude index (0..7) of each non-negative fp32 value."""
    flat = np.ascontiguousarray(y, dtype=np.float32).ravel()
    out = np.empty(flat.shape, dtype=np.uint8)
    _load().ref_e2m1_index_array(_ptr(flat), flat.size, _ptr(out))
    return out.reshape(np.shape(y))


def e4m3_encode_array(t: np.ndarray) -> np.ndarray:
    """Nearest saturating E4M3 byte of each non-negative fp32 value."""
    flat = np.ascontiguousarray(t, dtype=np.float32).ravel()
    out = np.empty(flat.shape, dtype=np.uint8)
    _load().ref_e4m3_encode_array(_ptr(flat), flat.size, _ptr(out))
    return out.reshape(np.shape(t))


# ------------------------------------------------------------------------------------------------
# array operations
# ------------------------------------------------------------------------------------------------
def widen(x: np.ndarray, dtype: int, src_scale: float | None = None) -> np.ndarray:
    """Source values -> fp32 [rows, cols].  dtype F32 (float32), BF16/F16 (uint16 bit patterns) or
    E4M3 (uint8 bytes, multiplied by src_scale, 1.0 when None)."""
    x = np.ascontiguousarray(x)
    rows, cols = x.shape
    out = np.empty((rows, cols), dtype=np.float32)
    sc = np.array([src_scale], dtype=np.float32) if src_scale is not None else None
    _load().ref_widen(_ptr(x), dtype, rows, cols, cols, _ptr(sc) if sc is not None else None, _ptr(out))
    return out


class QTensor:
    """An NVFP4 tensor: codes [rows, cols/2] uint8, scales [rows, cols/16] uint8, g float32."""

    def __init__(self, codes: np.ndarray, scales: np.ndarray, g: np.float32):
        self.codes, self.scales, self.g = codes, scales, np.float32(g)

    @property
    def shape(self):
        return (self.codes.shape[0], self.codes.shape[1] * 2)


def quantize(x: np.ndarray, dtype: int = F32, src_scale: float | None = None,
             amax: float | None = None) -> tuple[QTensor, int]:
    """Quantize [rows, cols] (cols % 16 == 0) to NVFP4.  Returns (QTensor, flags)."""
    v = widen(x, dtype, src_scale)
    rows, cols = v.shape
    assert cols % 16 == 0
    codes = np.zeros((rows, cols // 2), dtype=np.uint8)
    scales = np.zeros((rows, cols // 16), dtype=np.uint8)
    g = np.zeros(1, dtype=np.float32)
    a = np.array([amax], dtype=np.float32) if amax is not None else None
    flags = _load().ref_quantize_f32(_ptr(v), rows, cols, _ptr(a) if a is not None else None,
                                     _ptr(codes), _ptr(scales), _ptr(g))
    return QTensor(codes, scales, g[0]), int(flags)


def fp8_scale(amax: float) -> np.float32:
    return np.float32(_load().ref_fp8_scale(float(amax)))


def fp8_byte(v: float, scale: float) -> int:
    return _load().ref_fp8_byte(float(v), float(scale))


def quantize_fp8(x: np.ndarray, dtype: int = F32, src_scale: float | None = None,
                 amax: float | None = None) -> tuple[np.ndarray, np.float32, int]:
    """FP8 E4M3 tensorwise quantization ("Qwen3-VL-8B-Instruct-heretic-NVFP4", "Quantization
    Details" and "Runtime / hardware"): scale = fl(amax / 448) (1 when amax = 0), byte = sign |
    nearest E4M3 (ties to even, saturating) of fl(|v| / scale).  Returns (bytes [rows, cols] uint8,
    scale, flags)."""
    v = widen(x, dtype, src_scale)
    rows, cols = v.shape
    out = np.zeros((rows, cols), dtype=np.uint8)
    sc = np.zeros(1, dtype=np.float32)
    a = np.array([amax], dtype=np.float32) if amax is not None else None
    flags = _load().ref_quantize_fp8_f32(_ptr(v), rows, cols, _ptr(a) if a is not None else None, _ptr(out),
                                         _ptr(sc))
    return out, sc[0], int(flags)


def fp8_values(b: np.ndarray, scale: float) -> np.ndarray:
    """Exact values e4m3(b) * scale of FP8 bytes, in float64."""
    lut = np.array([_load().ref_e4m3_value(i & 0x7F) * (-1.0 if i & 0x80 else 1.0) for i in range(256)])
    return lut[np.asarray(b, dtype=np.uint8)] * float(np.float32(scale))


def dequantize(q: QTensor, out: str = "f32") -> np.ndarray:
    """Expand NVFP4 to 'f32', 'bf16' (uint16 bit patterns) or 'f64' (exact values)."""
    rows, cols = q.shape
    codes = np.ascontiguousarray(q.codes)
    scales = np.ascontiguousarray(q.scales)
    lib = _load()
    if out == "f64":
        o = np.empty((rows, cols), dtype=np.float64)
        lib.ref_dequantize_f64(_ptr(codes), _ptr(scales), float(q.g), rows, cols, _ptr(o))
    elif out == "f32":
        o = np.empty((rows, cols), dtype=np.float32)
        lib.ref_dequantize_f32(_ptr(codes), _ptr(scales), float(q.g), rows, cols, _ptr(o))
    elif out == "bf16":
        o = np.empty((rows, cols), dtype=np.uint16)
        lib.ref_dequantize_bf16(_ptr(codes), _ptr(scales), float(q.g), rows, cols, _ptr(o))
    else:
        raise ValueError(out)
    return o


def bf16_bits_to_f64(a_bits: np.ndarray) -> np.ndarray:
    return widen(np.ascontiguousarray(a_bits, dtype=np.uint16), BF16).astype(np.float64)


def gemm_f64(a_hat: np.ndarray, w_hat: np.ndarray) -> np.ndarray:
    """C[m, n] = sum_k A_hat[m, k] * W_hat[n, k] in float64 (the plain definition)."""
    return np.asarray(a_hat, dtype=np.float64) @ np.asarray(w_hat, dtype=np.float64).T


def gemm_w4a16(a_bits: np.ndarray, w: QTensor) -> np.ndarray:
    """Reference for the W4A16 GEMM: bf16 activations (uint16 bits) against expanded NVFP4 W."""
    return gemm_f64(bf16_bits_to_f64(a_bits), dequantize(w, "f64"))


def gemm_w4a4(a: QTensor, w: QTensor) -> np.ndarray:
    """Reference for the W4A4 GEMM: both operands expanded exactly from NVFP4."""
    return gemm_f64(dequantize(a, "f64"), dequantize(w, "f64"))


def gemm_w4a8(a_fp8: np.ndarray, a_scale: float, w: QTensor) -> np.ndarray:
    """Reference for the GEMM with FP8 activations ("Qwen3-VL-8B-Instruct-heretic-NVFP4", "Runtime /
    hardware": FP4 weight times dynamically quantized FP8 activation): both operands expanded
    exactly, contraction in float64."""
    return gemm_f64(fp8_values(a_fp8, a_scale), dequantize(w, "f64"))


def gemm_lowrank(a_bits: np.ndarray, w: QTensor, v_bits: np.ndarray, u_bits: np.ndarray,
                 a_q: QTensor | None = None) -> np.ndarray:
    """Reference for the NVFP4 GEMM with a bf16 low-rank branch ("Qwen Image 2.1: INT4 + FP4",
    "What I quantized": FP4 weights with BF16 rank-128 branches; reading R10): the weight is
    W ~ W_hat + U . V with U [N x r] and V [r x K] kept in bf16, and the layer computes
    C = A_hat . W_hat^T + (A . V^T) . U^T.  The branch takes the bf16 activations A (uint16 bits);
    the main product takes A itself (W4A16) or its NVFP4 form a_q (W4A4).  Every product and sum in
    float64 over the exact operand values."""
    a = bf16_bits_to_f64(a_bits)
    main = gemm_f64(dequantize(a_q, "f64") if a_q is not None else a, dequantize(w, "f64"))
    t = gemm_f64(a, bf16_bits_to_f64(v_bits))  # T = A . V^T, [M x r]
    return main + gemm_f64(t, bf16_bits_to_f64(u_bits))


def gemm_error(c: np.ndarray, cref: np.ndarray) -> float:
    """max_{m,n} |C - Cref| / max(|Cref[m,n]|, 1e-2 * max_n' |Cref[m,n']|): relative error with a
    per-row floor so that outputs near zero by cancellation do not dominate."""
    c = np.asarray(c, dtype=np.float64)
    cref = np.asarray(cref, dtype=np.float64)
    if cref.size == 0:
        return 0.0
    floor = 1e-2 * np.max(np.abs(cref), axis=1, keepdims=True)
    denom = np.maximum(np.abs(cref), floor)
    denom = np.where(denom == 0, 1.0, denom)
    return float(np.max(np.abs(c - cref) / denom))


STAT_FIELDS = ("rel_error", "kurtosis", "block_max_over_std", "mean", "std", "max_abs", "blocks")


def matrix_stats(w: np.ndarray, q: QTensor | None = None, dtype: int = F32) -> dict:
    """Quality statistics of one matrix ("Qwen-Image NVFP4 on a 16 GB Ada GPU", section "Quality:
    the error of each matrix"): the relative error ||W - W_hat|| / ||W|| (Frobenius, W_hat the exact
    expansion of q), the excess kurtosis (population moments), and the mean over blocks of 64
    consecutive elements of max|w| / std (population std of the block; blocks with std 0 left out)."""
    v = widen(w, dtype)
    rows, cols = v.shape
    out = np.zeros(7, dtype=np.float64)
    if q is not None:
        codes, scales = np.ascontiguousarray(q.codes), np.ascontiguousarray(q.scales)
        _load().ref_matrix_stats(_ptr(v), rows, cols, _ptr(codes), _ptr(scales), float(q.g), 1, _ptr(out))
    else:
        _load().ref_matrix_stats(_ptr(v), rows, cols, None, None, 0.0, 0, _ptr(out))
    return dict(zip(STAT_FIELDS, out.tolist()))


def rank(p: float, n: int) -> int:
    return int(_load().ref_rank(float(p), int(n)))


def amax_percentile(x: np.ndarray, p: float, per_channel: bool = True, dtype: int = F32):
    """Nearest-rank p-th percentile and max of |x| per column (or over the whole tensor)."""
    v = widen(x, dtype)
    rows, cols = v.shape
    n_out = cols if per_channel else 1
    pct = np.empty(n_out, dtype=np.float32)
    mx = np.empty(n_out, dtype=np.float32)
    _load().ref_amax_percentile(_ptr(v), rows, cols, float(p), 1 if per_channel else 0, _ptr(pct), _ptr(mx))
    return pct, mx
