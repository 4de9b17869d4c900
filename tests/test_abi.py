"""The C ABI library on the CPU: it loads, exports every function include/nvfp4.h declares, and
rejects bad arguments before touching the GPU (no compute call is made here)."""
import ctypes
import os
import re
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "nvfp4.h")


def _declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\s*\*?\s*(\w+)\s*\(", text, flags=re.M)))


@pytest.fixture(scope="module")
def nv():
    import bit_gemm_nvfp4_amd as m
    return m


def test_header_declares_the_entry_points():
    assert _declared_functions() == sorted(["nvfp4_quantize", "nvfp4_quantize_batch", "nvfp4_quantize_noalloc",
                                            "nvfp4_quantize_fp8",
                                            "nvfp4_tensor_amax",
                                            "nvfp4_dequantize", "nvfp4_gemm",
                                            "nvfp4_gemm_fp8a", "nvfp4_matrix_stats", "nvfp4_gemm_lowrank", "nvfp4_gemm_qa",
                                            "amax_percentile",
                                            "nvfp4_workspace_size", "nvfp4_status_string"])


def test_library_exports_every_declared_symbol(nv):
    out = subprocess.run(["nm", "-D", "--defined-only", nv.LIB_PATH], capture_output=True, text=True).stdout
    exported = set(re.findall(r"\bT (\w+)$", out, flags=re.M))
    for name in _declared_functions():
        assert name in exported, name
        assert getattr(nv.lib, name) is not None
    assert sorted(nv.EXPORTED) == _declared_functions()


def test_status_strings_and_workspace(nv):
    for s in range(9):
        assert nv.lib.nvfp4_status_string(s)
    assert nv.lib.nvfp4_status_string(99) == b"unknown status"
    assert nv.workspace_size(nv.OP_QUANTIZE, 10, 32) >= 4
    # per channel: the radix state (259 words), the candidate path's 4 words and 2048-key list
    assert nv.workspace_size(nv.OP_PERCENTILE, 100, 3072, 1) == 3072 * (259 + 4 + 2048) * 4
    assert nv.workspace_size(nv.OP_PERCENTILE, 100, 3072, 0) == 259 * 4
    assert nv.workspace_size(nv.OP_GEMM, 4096, 3072, 3072) == 0


FAKE = 0x10000  # a 16-byte aligned address that is never dereferenced: validation fails first


def _qt(nv, rows, cols, codes=FAKE, scales=FAKE, g=FAKE):
    return nv.CTensor(codes, scales, g, rows, cols)


def test_quantize_validation(nv):
    q = nv.lib.nvfp4_quantize
    t = _qt(nv, 4, 32)
    P = ctypes.c_void_p
    assert q(P(FAKE), 9, 32, None, None, ctypes.byref(t), None, P(FAKE), 256, None) == 4  # dtype
    assert q(None, 0, 32, None, None, ctypes.byref(t), None, P(FAKE), 256, None) == 1  # NULL x
    assert q(P(FAKE), 0, 32, None, None, None, None, P(FAKE), 256, None) == 1  # NULL out
    bad = _qt(nv, 4, 24)
    assert q(P(FAKE), 0, 24, None, None, ctypes.byref(bad), None, P(FAKE), 256, None) == 2  # cols % 16
    assert q(P(FAKE), 0, 16, None, None, ctypes.byref(t), None, P(FAKE), 256, None) == 2  # ld < cols
    neg = _qt(nv, -1, 32)
    assert q(P(FAKE), 0, 32, None, None, ctypes.byref(neg), None, P(FAKE), 256, None) == 2
    assert q(P(FAKE + 4), 0, 32, None, None, ctypes.byref(t), None, P(FAKE), 256, None) == 3  # align
    assert q(P(FAKE), 1, 36, None, None, ctypes.byref(t), None, P(FAKE), 256, None) == 3  # row start 72 B
    assert q(P(FAKE), 0, 32, P(FAKE), None, ctypes.byref(t), None, P(FAKE), 256, None) == 6  # scale w/o e4m3
    assert q(P(FAKE), 0, 32, None, None, ctypes.byref(t), None, None, 0, None) == 5  # workspace
    assert q(P(FAKE), 0, 32, None, None, ctypes.byref(t), None, P(FAKE), 8, None) == 5
    ws = nv.workspace_size(nv.OP_QUANTIZE, 4, 32)
    assert q(P(FAKE), 0, 32, None, None, ctypes.byref(t), None, P(FAKE), ws - 1, None) == 5
    unal = _qt(nv, 4, 32, codes=FAKE + 8)
    assert q(P(FAKE), 0, 32, None, None, ctypes.byref(unal), None, P(FAKE), 256, None) == 3


def test_quantize_noalloc_validation(nv):
    q = nv.lib.nvfp4_quantize_noalloc
    t = _qt(nv, 4, 32)
    P = ctypes.c_void_p
    assert q(P(FAKE), 9, 32, None, None, ctypes.byref(t), None, None) == 4  # dtype
    assert q(None, 0, 32, None, None, ctypes.byref(t), None, None) == 1  # NULL x
    assert q(P(FAKE), 0, 32, None, None, None, None, None) == 1  # NULL out
    assert q(P(FAKE), 0, 16, None, None, ctypes.byref(t), None, None) == 2  # ld < cols
    assert q(P(FAKE + 4), 0, 32, None, None, ctypes.byref(t), None, None) == 3  # align
    assert q(P(FAKE), 0, 32, P(FAKE), None, ctypes.byref(t), None, None) == 6  # scale without e4m3
    assert q(P(FAKE), 0, 32, None, None, ctypes.byref(t), P(FAKE + 2), None) == 3  # flags align


def test_quantize_batch_validation(nv):
    q = nv.lib.nvfp4_quantize_batch
    P = ctypes.c_void_p
    ws = nv.workspace_size(nv.OP_QUANTIZE, 4, 32)

    def arrays(n, xs=None, lds=None, outs=None, scs=None):
        xa = (ctypes.c_void_p * n)(*(xs or [FAKE] * n))
        la = (ctypes.c_int64 * n)(*(lds or [32] * n))
        oa = (nv.CTensor * n)(*(outs or [_qt(nv, 4, 32) for _ in range(n)]))
        sa = None if scs is None else (ctypes.c_void_p * n)(*scs)
        return xa, la, oa, sa

    x, ld, o, _ = arrays(2)
    assert q(0, None, 0, None, None, None, None, P(FAKE), ws, None) == 0  # nothing to do
    assert q(9, x, 0, ld, None, o, None, P(FAKE), ws, None) == 6  # more than 8 tensors
    assert q(-1, x, 0, ld, None, o, None, P(FAKE), ws, None) == 6
    assert q(2, None, 0, ld, None, o, None, P(FAKE), ws, None) == 1  # NULL arrays
    assert q(2, x, 0, None, None, o, None, P(FAKE), ws, None) == 1
    assert q(2, x, 0, ld, None, None, None, P(FAKE), ws, None) == 1
    assert q(2, x, 9, ld, None, o, None, P(FAKE), ws, None) == 4  # dtype
    x2, ld2, o2, _ = arrays(2, xs=[FAKE, 0])
    assert q(2, x2, 0, ld2, None, o2, None, P(FAKE), ws, None) == 1  # NULL second tensor
    x3, ld3, o3, _ = arrays(2, lds=[32, 16])
    assert q(2, x3, 0, ld3, None, o3, None, P(FAKE), ws, None) == 2  # second ld < cols
    x4, ld4, o4, _ = arrays(2, outs=[_qt(nv, 4, 32), _qt(nv, 4, 24)])
    assert q(2, x4, 0, ld4, None, o4, None, P(FAKE), ws, None) == 2  # second cols % 16
    x5, ld5, o5, sc5 = arrays(2, scs=[None, FAKE])
    assert q(2, x5, 0, ld5, sc5, o5, None, P(FAKE), ws, None) == 6  # source scale without e4m3
    x6, ld6, o6, sc6 = arrays(2, scs=[None, FAKE + 2])
    assert q(2, x6, 3, ld6, sc6, o6, None, P(FAKE), ws, None) == 3  # source scale alignment
    assert q(2, x, 0, ld, None, o, None, None, 0, None) == 5  # workspace
    assert q(2, x, 0, ld, None, o, None, P(FAKE), ws - 1, None) == 5
    assert q(2, x, 0, ld, None, o, P(FAKE + 2), P(FAKE), ws, None) == 3  # flags alignment


def test_tensor_amax_validation(nv):
    f = nv.lib.nvfp4_tensor_amax
    P = ctypes.c_void_p
    ws = nv.workspace_size(nv.OP_AMAX, 4, 32)
    assert ws >= 4 * 256
    assert f(P(FAKE), 9, 4, 32, 32, None, P(FAKE), None, P(FAKE), ws, None) == 4  # dtype
    assert f(None, 0, 4, 32, 32, None, P(FAKE), None, P(FAKE), ws, None) == 1  # NULL x
    assert f(P(FAKE), 0, 4, 32, 32, None, None, None, P(FAKE), ws, None) == 1  # NULL amax_out
    assert f(P(FAKE), 0, 4, 24, 24, None, P(FAKE), None, P(FAKE), ws, None) == 2  # cols % 16
    assert f(P(FAKE), 0, 4, 32, 16, None, P(FAKE), None, P(FAKE), ws, None) == 2  # ld < cols
    assert f(P(FAKE), 0, -1, 32, 32, None, P(FAKE), None, P(FAKE), ws, None) == 2
    assert f(P(FAKE + 4), 0, 4, 32, 32, None, P(FAKE), None, P(FAKE), ws, None) == 3  # x align
    assert f(P(FAKE), 0, 4, 32, 32, None, P(FAKE + 2), None, P(FAKE), ws, None) == 3  # amax align
    assert f(P(FAKE), 0, 4, 32, 32, P(FAKE), P(FAKE), None, P(FAKE), ws, None) == 6  # src_scale w/o e4m3
    assert f(P(FAKE), 0, 4, 32, 32, None, P(FAKE), None, None, ws, None) == 5  # workspace
    assert f(P(FAKE), 0, 4, 32, 32, None, P(FAKE), None, P(FAKE), ws - 1, None) == 5


def test_dequantize_validation(nv):
    d = nv.lib.nvfp4_dequantize
    t = _qt(nv, 4, 32)
    P = ctypes.c_void_p
    assert d(None, P(FAKE), 0, 32, None) == 1
    assert d(ctypes.byref(t), None, 0, 32, None) == 1
    assert d(ctypes.byref(t), P(FAKE), 3, 32, None) == 4  # E4M3 output not offered
    assert d(ctypes.byref(t), P(FAKE), 1, 20, None) == 2  # ld < cols
    assert d(ctypes.byref(t), P(FAKE), 1, 36, None) == 3  # bf16 rows of 72 bytes
    nog = _qt(nv, 4, 32, g=0)
    assert d(ctypes.byref(nog), P(FAKE), 0, 32, None) == 1


def test_gemm_validation(nv):
    g = nv.lib.nvfp4_gemm
    w = _qt(nv, 64, 128)
    a = _qt(nv, 8, 128)
    P = ctypes.c_void_p
    assert g(None, None, 8, 128, ctypes.byref(w), P(FAKE), 64, None, 0, None) == 6  # neither form
    assert g(P(FAKE), ctypes.byref(a), 8, 128, ctypes.byref(w), P(FAKE), 64, None, 0, None) == 6  # both
    assert g(P(FAKE), None, 8, 128, None, P(FAKE), 64, None, 0, None) == 1
    assert g(P(FAKE), None, 8, 64, ctypes.byref(w), P(FAKE), 64, None, 0, None) == 2  # lda < K
    a_bad = _qt(nv, 8, 256)
    assert g(None, ctypes.byref(a_bad), 8, 0, ctypes.byref(w), P(FAKE), 64, None, 0, None) == 2  # K mismatch
    assert g(None, ctypes.byref(a), 9, 0, ctypes.byref(w), P(FAKE), 64, None, 0, None) == 2  # M mismatch
    assert g(P(FAKE), None, 8, 128, ctypes.byref(w), P(FAKE), 32, None, 0, None) == 2  # ldc < N
    assert g(P(FAKE), None, 8, 128, ctypes.byref(w), None, 64, None, 0, None) == 1  # NULL C
    assert g(P(FAKE), None, -1, 128, ctypes.byref(w), P(FAKE), 64, None, 0, None) == 2
    assert g(P(FAKE), None, 8, 132, ctypes.byref(w), P(FAKE), 64, None, 0, None) == 3  # A rows 264 B
    assert g(P(FAKE), None, 8, 128, ctypes.byref(w), P(FAKE + 2), 64, None, 0, None) == 3  # C not 4-aligned


def test_quantize_fp8_validation(nv):
    q = nv.lib.nvfp4_quantize_fp8
    P = ctypes.c_void_p
    ws = nv.workspace_size(nv.OP_QUANTIZE, 4, 32)
    assert q(P(FAKE), 9, 4, 32, 32, None, None, P(FAKE), P(FAKE), None, P(FAKE), ws, None) == 4  # dtype
    assert q(None, 0, 4, 32, 32, None, None, P(FAKE), P(FAKE), None, P(FAKE), ws, None) == 1  # NULL x
    assert q(P(FAKE), 0, 4, 32, 32, None, None, None, P(FAKE), None, P(FAKE), ws, None) == 1  # NULL out
    assert q(P(FAKE), 0, 4, 32, 32, None, None, P(FAKE), None, None, P(FAKE), ws, None) == 1  # NULL scale out
    assert q(P(FAKE), 0, 4, 24, 24, None, None, P(FAKE), P(FAKE), None, P(FAKE), ws, None) == 2  # cols % 16
    assert q(P(FAKE), 0, 4, 32, 16, None, None, P(FAKE), P(FAKE), None, P(FAKE), ws, None) == 2  # ld < cols
    assert q(P(FAKE), 0, -1, 32, 32, None, None, P(FAKE), P(FAKE), None, P(FAKE), ws, None) == 2
    assert q(P(FAKE + 4), 0, 4, 32, 32, None, None, P(FAKE), P(FAKE), None, P(FAKE), ws, None) == 3  # x align
    assert q(P(FAKE), 0, 4, 32, 32, None, None, P(FAKE + 8), P(FAKE), None, P(FAKE), ws, None) == 3  # out align
    assert q(P(FAKE), 0, 4, 32, 32, None, None, P(FAKE), P(FAKE + 2), None, P(FAKE), ws, None) == 3
    assert q(P(FAKE), 0, 4, 32, 32, P(FAKE), None, P(FAKE), P(FAKE), None, P(FAKE), ws, None) == 6  # src_scale
    assert q(P(FAKE), 0, 4, 32, 32, None, None, P(FAKE), P(FAKE), None, None, 0, None) == 5  # workspace
    assert q(P(FAKE), 0, 4, 32, 32, None, None, P(FAKE), P(FAKE), None, P(FAKE), ws - 1, None) == 5


def test_gemm_fp8a_validation(nv):
    g = nv.lib.nvfp4_gemm_fp8a
    w = _qt(nv, 64, 128)
    P = ctypes.c_void_p
    assert g(P(FAKE), None, 8, 128, ctypes.byref(w), P(FAKE), 64, None, 0, None) == 1  # NULL a_scale
    assert g(None, P(FAKE), 8, 128, ctypes.byref(w), P(FAKE), 64, None, 0, None) == 1  # NULL a
    assert g(P(FAKE), P(FAKE), 8, 128, None, P(FAKE), 64, None, 0, None) == 1  # NULL w
    assert g(P(FAKE), P(FAKE), 8, 64, ctypes.byref(w), P(FAKE), 64, None, 0, None) == 2  # lda < K
    assert g(P(FAKE), P(FAKE), -1, 128, ctypes.byref(w), P(FAKE), 64, None, 0, None) == 2
    assert g(P(FAKE), P(FAKE), 8, 136, ctypes.byref(w), P(FAKE), 64, None, 0, None) == 3  # A rows 136 B
    assert g(P(FAKE), P(FAKE + 2), 8, 128, ctypes.byref(w), P(FAKE), 64, None, 0, None) == 3  # scale align
    assert g(P(FAKE), P(FAKE), 8, 128, ctypes.byref(w), P(FAKE), 32, None, 0, None) == 2  # ldc < N
    assert g(P(FAKE), P(FAKE), 8, 128, ctypes.byref(w), None, 64, None, 0, None) == 1  # NULL C


def test_matrix_stats_validation(nv):
    f = nv.lib.nvfp4_matrix_stats
    P = ctypes.c_void_p
    ws = nv.workspace_size(nv.OP_STATS, 0, 0)
    assert ws > 0
    q = _qt(nv, 4, 32)
    assert f(P(FAKE), 3, 4, 32, 32, None, P(FAKE), P(FAKE), ws, None) == 4  # e4m3 input
    assert f(P(FAKE), 0, 4, 32, 32, None, None, P(FAKE), ws, None) == 1  # NULL out
    assert f(None, 0, 4, 32, 32, None, P(FAKE), P(FAKE), ws, None) == 1  # NULL w
    assert f(P(FAKE), 0, 4, 24, 24, None, P(FAKE), P(FAKE), ws, None) == 2  # cols % 16
    assert f(P(FAKE), 0, 0, 32, 32, None, P(FAKE), P(FAKE), ws, None) == 2  # no rows
    bad = _qt(nv, 5, 32)
    assert f(P(FAKE), 0, 4, 32, 32, ctypes.byref(bad), P(FAKE), P(FAKE), ws, None) == 2  # q shape
    assert f(P(FAKE), 0, 4, 32, 32, ctypes.byref(q), P(FAKE + 4), P(FAKE), ws, None) == 3  # out align
    assert f(P(FAKE), 0, 4, 32, 32, ctypes.byref(q), P(FAKE), P(FAKE), ws - 1, None) == 5  # workspace
    assert f(P(FAKE), 0, 4, 32, 32, ctypes.byref(q), P(FAKE), None, ws, None) == 5


def test_gemm_lowrank_validation(nv):
    f = nv.lib.nvfp4_gemm_lowrank
    P = ctypes.c_void_p
    w = _qt(nv, 64, 32)
    ws = nv.workspace_size(nv.OP_LOWRANK, 8, 64, 32)
    assert ws >= 8 * 1024  # T at rank 256: 8 rows x 1 KiB
    ok = dict(a=P(FAKE), aq=None, M=8, lda=32, w=ctypes.byref(w), v=P(FAKE), u=P(FAKE), r=16, c=P(FAKE), ldc=64,
              ws=P(FAKE), wsb=ws)

    def call(**kw):
        d = dict(ok, **kw)
        return f(d["a"], d["aq"], d["M"], d["lda"], d["w"], d["v"], d["u"], d["r"], d["c"], d["ldc"], d["ws"],
                 d["wsb"], None)
    assert call(r=0) == 2 and call(r=24) == 2 and call(r=272) == 2  # rank: 16 .. 256, multiple of 16
    assert call(a=None) == 1                                          # the branch needs the bf16 activations
    assert call(v=None) == 1 and call(u=None) == 1                    # V, U NULL with elements
    assert call(lda=16) == 2                                          # lda < K
    assert call(v=P(FAKE + 8)) == 3                                   # alignment of V
    assert call(ws=None) == 5 and call(wsb=8 * 1024 - 1) == 5         # T does not fit
    bad = _qt(nv, 9, 32)
    assert call(aq=ctypes.byref(bad)) == 2                            # a_q rows != M
    assert call(M=-1) == 2


def test_gemm_qa_validation(nv):
    f = nv.lib.nvfp4_gemm_qa
    P = ctypes.c_void_p
    w = _qt(nv, 64, 128)
    w_odd = _qt(nv, 64, 48)  # K % 64 != 0: the unfused form, which needs the workspace
    ws = nv.workspace_size(nv.OP_GEMM_QA, 8, 64, 48)
    assert ws >= 8 * 24 + 8 * 3  # codes and scales of the quantized activations
    assert f(P(FAKE), None, 8, 128, ctypes.byref(w), P(FAKE), 64, None, 0, None) == 1        # amax NULL
    assert f(P(FAKE), P(FAKE + 2), 8, 128, ctypes.byref(w), P(FAKE), 64, None, 0, None) == 3  # amax align
    assert f(None, P(FAKE), 8, 128, ctypes.byref(w), P(FAKE), 64, None, 0, None) == 1        # A NULL
    assert f(P(FAKE), P(FAKE), 8, 64, ctypes.byref(w), P(FAKE), 64, None, 0, None) == 2      # lda < K
    assert f(P(FAKE), P(FAKE), 8, 128, ctypes.byref(w), P(FAKE), 32, None, 0, None) == 2     # ldc < N
    assert f(P(FAKE), P(FAKE), -1, 128, ctypes.byref(w), P(FAKE), 64, None, 0, None) == 2
    assert f(P(FAKE), P(FAKE), 8, 48, ctypes.byref(w_odd), P(FAKE), 64, None, 0, None) == 5  # unfused, no ws
    assert f(P(FAKE), P(FAKE), 8, 48, ctypes.byref(w_odd), P(FAKE), 64, P(FAKE), 8, None) == 5


def test_percentile_validation(nv):
    f = nv.lib.amax_percentile
    P = ctypes.c_void_p
    ws = 3072 * 259 * 4
    assert f(P(FAKE), 3, 10, 32, 32, 99.9, 1, P(FAKE), None, None, P(FAKE), ws, None) == 4  # e4m3 input
    assert f(P(FAKE), 1, 10, 32, 32, 0.0, 1, P(FAKE), None, None, P(FAKE), ws, None) == 6  # p = 0
    assert f(P(FAKE), 1, 10, 32, 32, 100.5, 1, P(FAKE), None, None, P(FAKE), ws, None) == 6
    assert f(P(FAKE), 1, 10, 32, 32, float("nan"), 1, P(FAKE), None, None, P(FAKE), ws, None) == 6
    assert f(P(FAKE), 1, 10, 32, 32, 99.9, 2, P(FAKE), None, None, P(FAKE), ws, None) == 6  # mode
    assert f(P(FAKE), 1, 0, 32, 32, 99.9, 1, P(FAKE), None, None, P(FAKE), ws, None) == 2  # no rows
    assert f(P(FAKE), 1, 10, 40, 40, 99.9, 1, P(FAKE), None, None, P(FAKE), ws, None) == 2  # cols % 16
    assert f(P(FAKE), 1, 10, 32, 32, 99.9, 1, None, None, None, P(FAKE), ws, None) == 1
    assert f(P(FAKE), 1, 10, 32, 32, 99.9, 1, P(FAKE), None, None, P(FAKE), 100, None) == 5
    assert f(P(FAKE), 1, 10, 32, 32, 99.9, 1, P(FAKE), None, None, None, ws, None) == 5


def test_binding_rejects_column_strided_views(nv):
    # the C ABI takes a row stride only, so the binding refuses views whose rows are not contiguous
    import torch
    x = torch.zeros((4, 64), dtype=torch.float32)
    with pytest.raises(AssertionError):
        nv._row_stride(x[:, ::2], "x")
    with pytest.raises(AssertionError):
        nv._row_stride(x, "x", cols=32)
    assert nv._row_stride(x[1:3], "x") == 64 and nv._row_stride(x[:1], "x") == 64
    assert nv._row_stride(torch.zeros((8, 128))[:, :64], "x") == 128


def test_valid_call_without_gpu_reports_device(nv):
    # A fully valid call on a machine without a gfx950 device is refused with NVFP4_ERR_DEVICE
    # before anything is enqueued.
    import torch
    if torch.cuda.is_available():
        pytest.skip("a GPU is present")
    t = _qt(nv, 4, 32)
    P = ctypes.c_void_p
    ws = nv.workspace_size(nv.OP_QUANTIZE, 4, 32)
    assert nv.lib.nvfp4_quantize(P(FAKE), 0, 32, None, None, ctypes.byref(t), None, P(FAKE), ws, None) == 7
    assert nv.lib.nvfp4_quantize_noalloc(P(FAKE), 0, 32, None, None, ctypes.byref(t), None, None) == 7
