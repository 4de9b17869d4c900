"""GPU tests of the run-time amax protocols of the quantizers.

The one-launch form agrees on the tensor amax across its workgroups through a workspace that
carries a call tag from one call to the next; the two-launch form takes the amax in a pass of its
own (nvfp4_tensor_amax) and then encodes with it as a static amax.  Both must give exactly the
oracle's codes, scale bytes and global scale ("Qwen3-VL-8B-Instruct-heretic-NVFP4", "Quantization
Details": per-tensor amax at run time), and a workspace left in a state the protocol did not
leave it in must be reported in flags bit 2, not trusted.
"""
import sys

import numpy as np
import pytest
import torch

import oracle
import synth
from gpu_util import DEV, padded, to_dev_bf16, to_dev_f16, to_dev_f32, to_dev_u8

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def nv():
    import bit_gemm_nvfp4_amd as m
    return m


def _note(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def _assert_q(q, ref, what):
    assert q.global_scale.cpu().numpy().view(np.uint32)[0] == np.float32(ref.g).view(np.uint32), what
    assert np.array_equal(q.scales.cpu().numpy(), ref.scales), what
    assert np.array_equal(q.codes.cpu().numpy(), ref.codes), what


def _input(dtype, shape, seed):
    rng = np.random.default_rng(seed)
    x = (rng.standard_normal(shape) * 0.03).astype(np.float32)
    if x.size:
        x.reshape(-1)[rng.integers(0, x.size)] = 1.7
    if dtype == "f32":
        return to_dev_f32(x), x, oracle.F32, None
    if dtype == "bf16":
        b = synth.bf16_bits(x)
        return to_dev_bf16(b), b, oracle.BF16, None
    if dtype == "f16":
        h = x.astype(np.float16).view(np.uint16)
        return to_dev_f16(h), h, oracle.F16, None
    if x.size == 0:
        b, sc = np.zeros(shape, np.uint8), np.float32(1.0)
    else:
        b, sc = synth.fp8_tensorwise(x)
    return to_dev_u8(b), b, oracle.E4M3, float(sc)


@pytest.mark.parametrize("shape", [(0, 64), (1, 16), (5, 48), (300, 272), (1024, 3072), (4099, 1040)])
@pytest.mark.parametrize("dtype", ["f32", "bf16", "f16", "e4m3"])
def test_two_pass_quantize_matches_oracle_and_one_launch(nv, dtype, shape):
    xd, xh, odt, sc = _input(dtype, shape, shape[0] * 31 + shape[1])
    _note(f"two-pass quantize {dtype} {shape}")
    s = None if sc is None else torch.tensor([sc], dtype=torch.float32, device=DEV)
    q2 = nv.quantize(xd, src_scale=s, two_pass=True, check=True)
    q1 = nv.quantize(xd, src_scale=s, check=True)
    ref, _ = oracle.quantize(xh, odt, sc)
    _assert_q(q2, ref, f"two-pass {dtype} {shape}")
    _assert_q(q1, ref, f"one-launch {dtype} {shape}")
    amax = nv.tensor_amax(xd, src_scale=s).cpu().numpy()
    want = np.abs(oracle.widen(xh, odt, sc)).max() if xh.size else np.float32(0)
    assert amax.view(np.uint32)[0] == np.float32(want).view(np.uint32)
    if shape[0] > 1 and dtype != "e4m3":
        _assert_q(nv.quantize(padded(xd, 16), src_scale=s, two_pass=True, check=True), ref, "strided")
    # the FP8 tensorwise quantizer in its two-launch form
    f2 = nv.quantize_fp8(xd, src_scale=s, two_pass=True, check=True)
    rb, rs, _ = oracle.quantize_fp8(xh, odt, sc)
    assert f2.scale.cpu().numpy().view(np.uint32)[0] == np.float32(rs).view(np.uint32)
    assert np.array_equal(f2.data.cpu().numpy(), rb)


def test_tensor_amax_nonfinite_flag(nv):
    for bad in [np.nan, np.inf]:
        x = np.ones((64, 256), np.float32)
        x[40, 100] = bad
        flags = torch.zeros(1, dtype=torch.int32, device=DEV)
        nv.tensor_amax(to_dev_f32(x), flags=flags)
        assert int(flags.item()) & 1
    b = np.full((8, 32), 0x38, np.uint8)
    b[3, 3] = 0x7F  # E4M3 NaN
    flags = torch.zeros(1, dtype=torch.int32, device=DEV)
    nv.tensor_amax(to_dev_u8(b), flags=flags)
    assert int(flags.item()) & 1


def test_modulation_two_pass_full(nv):
    _note("two-pass quantize of the 18432x3072 fp32 modulation weight")
    w = synth.modulation_weight()
    ref, _ = oracle.quantize(w)
    _assert_q(nv.quantize(to_dev_f32(w), two_pass=True, check=True), ref, "modulation two-pass")


def test_workspace_reused_over_calls_of_changing_size(nv):
    # one zeroed workspace, calls of different sizes (different grids) in a row: the call tag moves
    # on after every call, and no flag is raised
    ws = nv.quantize_workspace(DEV)
    flags = torch.zeros(1, dtype=torch.int32, device=DEV)
    for i, shape in enumerate([(4096, 3072), (3, 32), (1024, 4096), (1, 16), (2048, 2048), (4096, 3072)]):
        xd, xh, odt, _ = _input("f32", shape, 900 + i)
        q = nv.quantize(xd, workspace=ws, flags=flags)
        f8 = nv.quantize_fp8(xd, workspace=ws, flags=flags)
        _assert_q(q, oracle.quantize(xh)[0], f"call {i}")
        rb, _, _ = oracle.quantize_fp8(xh)
        assert np.array_equal(f8.data.cpu().numpy(), rb)
    nv.check_flags(flags)
    records = ws.view(torch.int32).cpu().numpy()[16:16 + 1360]
    assert records.max() == 12  # the tag records count the calls


def test_stale_workspace_is_reported(nv):
    # a workspace whose slots already carry the next call's tag (never zeroed, or shared by calls
    # that overlapped): the call ends (every slot looks published), and flags bit 2 says that its
    # outputs cannot be trusted
    rows, cols = 2048, 3072
    xd, xh, _, _ = _input("f32", (rows, cols), 77)
    # workspace layout: 16 reserved words, 1360 tag records, then the 64-bit slots
    def records(w):
        return w[64:64 + 4 * 1360].view(torch.int32)

    def slots(w):
        return w[5504:].view(torch.int64)
    ws = nv.quantize_workspace(DEV)
    records(ws).fill_(1000)
    slots(ws).fill_(1001 << 32)  # every slot tagged for the next call, payload 0
    flags = torch.zeros(1, dtype=torch.int32, device=DEV)
    nv.quantize(xd, workspace=ws, flags=flags)
    torch.cuda.synchronize()
    assert int(flags.item()) & 4
    with pytest.raises(RuntimeError):
        nv.check_flags(flags)
    # one stale slot in an otherwise consistent workspace is enough to be reported
    ws = nv.quantize_workspace(DEV)
    records(ws)[3] = 7
    slots(ws)[1] = 8 << 32
    flags.zero_()
    nv.quantize(xd, workspace=ws, flags=flags)
    torch.cuda.synchronize()
    assert int(flags.item()) & 4
    # a zeroed workspace is fine, and the result is the oracle's
    flags.zero_()
    q = nv.quantize(xd, workspace=nv.quantize_workspace(DEV), flags=flags)
    torch.cuda.synchronize()
    assert int(flags.item()) == 0
    _assert_q(q, oracle.quantize(xh)[0], "zeroed workspace")
