"""nvfp4_quantize_noalloc (the quantize entry point that allocates nothing, for callers that cannot
allocate: its run-time amax agreement uses a scratch array inside the library) against
nvfp4_quantize with a workspace: identical codes, scale bytes and global scale, bit for bit, on two
calls in a row with the second on a smaller input, for each source type, and with a static amax."""
import ctypes
import sys

import numpy as np
import pytest
import torch

import synth
from gpu_util import DEV, padded, to_dev_bf16, to_dev_f32, to_dev_u8

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def nv():
    import bit_gemm_nvfp4_amd as m
    return m


def _same(a, b, what):
    assert torch.equal(a.global_scale.view(torch.int32), b.global_scale.view(torch.int32)), what
    assert torch.equal(a.scales, b.scales), what
    assert torch.equal(a.codes, b.codes), what


def _noalloc(nv, x, out, flags, amax=None, src_scale=None):
    """The entry point called through the C ABI directly (ctypes), with caller-owned outputs."""
    ct = out.c()
    st = nv.lib.nvfp4_quantize_noalloc(ctypes.c_void_p(x.data_ptr()), nv._DT[x.dtype], nv._rows(x, "x"),
                                       None if src_scale is None else ctypes.c_void_p(src_scale.data_ptr()),
                                       None if amax is None else ctypes.c_void_p(amax.data_ptr()),
                                       ctypes.byref(ct), ctypes.c_void_p(flags.data_ptr()),
                                       ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    assert st == 0, nv.lib.nvfp4_status_string(st)
    return out


def _inputs(kind):
    rng = np.random.default_rng(17)
    big = (rng.standard_normal((3072, 3072)) * 0.02).astype(np.float32)
    small = (rng.standard_normal((300, 272)) * 3.0).astype(np.float32)
    if kind == "f32":
        return [(to_dev_f32(big), None), (to_dev_f32(small), None)]
    if kind == "bf16":
        return [(to_dev_bf16(synth.bf16_bits(big)), None), (padded(to_dev_bf16(synth.bf16_bits(small)), 16), None)]
    out = []
    for w in (big, small):
        b, sc = synth.fp8_tensorwise(w)
        out.append((to_dev_u8(b), torch.tensor([sc], dtype=torch.float32, device=DEV)))
    return out


@pytest.mark.parametrize("kind", ["f32", "bf16", "e4m3"])
def test_noalloc_matches_workspace_form_on_two_calls(nv, kind):
    print(f"quantize_noalloc {kind}", flush=True)
    sys.stdout.flush()
    flags = torch.zeros(1, dtype=torch.int32, device=DEV)
    for i, (x, sc) in enumerate(_inputs(kind)):  # the second call is the smaller input
        rows, cols = x.shape
        ref = nv.quantize(x, src_scale=sc, check=True)
        got = _noalloc(nv, x, nv.NVFP4Tensor.empty(rows, cols, DEV), flags, src_scale=sc)
        torch.cuda.synchronize()
        assert int(flags.item()) == 0, f"call {i}: flags {int(flags.item()):#x}"
        _same(got, ref, f"{kind} call {i} {rows}x{cols}")
        # static amax: no scratch involved, same outputs as the workspace form
        amax = torch.tensor([0.5], dtype=torch.float32, device=DEV)
        got_s = _noalloc(nv, x, nv.NVFP4Tensor.empty(rows, cols, DEV), flags, amax=amax, src_scale=sc)
        _same(got_s, nv.quantize(x, amax=amax, src_scale=sc), f"{kind} static amax call {i}")
        # and through the binding's wrapper
        got_b = nv.quantize_noalloc(x, nv.NVFP4Tensor.empty(rows, cols, DEV), src_scale=sc, flags=flags)
        torch.cuda.synchronize()
        assert int(flags.item()) == 0
        _same(got_b, ref, f"{kind} binding call {i}")
