"""GPU parity: the HIP path (through the C ABI via the binding) against the CPU oracle.

Codes, scale bytes, global scales, expanded values and percentiles are compared bit for bit;
GEMM outputs within the floored max relative error 2e-3 of the FP64 definition.  Shapes span
several tiles with ragged tails; the large workloads are covered at full size.
"""
import math
import sys

import numpy as np
import pytest
import torch

import oracle
import synth
from gpu_util import DEV, bits16, padded, to_dev_bf16, to_dev_f16, to_dev_f32, to_dev_u8

pytestmark = pytest.mark.gpu

GEMM_TOL = 2e-3


@pytest.fixture(scope="module")
def nv():
    import bit_gemm_nvfp4_amd as m
    return m


def _note(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def _quant(nv, x, **kw):
    """nvfp4_quantize with a flags word that must stay clear: no non-finite input and no
    incomplete grid agreement on amax."""
    flags = torch.zeros(1, dtype=torch.int32, device=DEV)
    q = nv.quantize(x, flags=flags, **kw)
    f = int(flags.item())
    assert f == 0, f"quantize flags {f:#x}"
    return q


def _assert_q_equal(q, ref, what=""):
    codes = q.codes.cpu().numpy()
    scales = q.scales.cpu().numpy()
    g = q.global_scale.cpu().numpy()[0]
    assert g.view(np.uint32) == np.float32(ref.g).view(np.uint32), f"{what} global scale {g} vs {ref.g}"
    bad_s = np.nonzero(scales != ref.scales)
    assert bad_s[0].size == 0, f"{what} {bad_s[0].size} scale bytes differ, first at {bad_s[0][0]},{bad_s[1][0]}"
    bad_c = np.nonzero(codes != ref.codes)
    assert bad_c[0].size == 0, (f"{what} {bad_c[0].size} code bytes differ, first at {bad_c[0][0]},{bad_c[1][0]}: "
                                f"{codes[bad_c[0][0], bad_c[1][0]]:#x} vs {ref.codes[bad_c[0][0], bad_c[1][0]]:#x}")


# ------------------------------------------------------------------------------------------------
# quantize
# ------------------------------------------------------------------------------------------------
def test_tiny_quantize_expand(nv):
    d = synth.tiny()
    _note("tiny 64x256 fp32")
    q = _quant(nv, to_dev_f32(d["w"]))
    ref, flags = oracle.quantize(d["w"])
    _assert_q_equal(q, ref, "tiny")
    f32 = nv.dequantize(q, torch.float32).cpu().numpy()
    assert np.array_equal(f32.view(np.uint32), oracle.dequantize(ref, "f32").view(np.uint32))
    bf = bits16(nv.dequantize(q, torch.bfloat16))
    assert np.array_equal(bf, oracle.dequantize(ref, "bf16"))


SHAPES = [(1, 16), (3, 48), (64, 256), (65, 1040), (7, 4096), (300, 272), (129, 2048)]


@pytest.mark.parametrize("shape", SHAPES)
@pytest.mark.parametrize("dtype", ["f32", "bf16", "f16"])
def test_quantize_shapes_dtypes(nv, shape, dtype):
    rows, cols = shape
    _note(f"quantize {dtype} {shape}")
    rng = np.random.default_rng(rows * 7919 + cols)
    x = (rng.standard_t(4, size=shape) * 10.0 ** rng.uniform(-3, 1)).astype(np.float32)
    x[rng.random(shape) < 0.05] = 0.0
    x[rng.random(shape) < 0.02] *= -0.0
    if dtype == "f32":
        xd, ref = to_dev_f32(x), oracle.quantize(x)[0]
    elif dtype == "bf16":
        b = synth.bf16_bits(x)
        xd, ref = to_dev_bf16(b), oracle.quantize(b, oracle.BF16)[0]
    else:
        h = x.astype(np.float16).view(np.uint16)
        xd, ref = to_dev_f16(h), oracle.quantize(h, oracle.F16)[0]
    _assert_q_equal(_quant(nv, xd), ref, f"{dtype} {shape}")
    # the same matrix with a larger row stride
    if rows > 1:
        _assert_q_equal(_quant(nv, padded(xd, 16)), ref, f"{dtype} {shape} strided")


def test_quantize_static_amax_clips(nv):
    _note("static amax")
    rng = np.random.default_rng(5)
    x = rng.standard_normal((128, 512)).astype(np.float32)
    for amax in [0.5, 1.0, 3.0, 1e6]:
        ref, _ = oracle.quantize(x, amax=amax)
        q = _quant(nv, to_dev_f32(x), amax=torch.tensor([amax], dtype=torch.float32, device=DEV))
        _assert_q_equal(q, ref, f"amax {amax}")


def test_quantize_zero_negzero_tiny(nv):
    _note("zero / -0 / tiny magnitudes")
    for x in [np.zeros((4, 64), np.float32), -np.zeros((4, 64), np.float32),
              np.full((4, 64), 1e-40, np.float32), np.full((2, 32), 3e-45, np.float32)]:
        ref, _ = oracle.quantize(x)
        _assert_q_equal(_quant(nv, to_dev_f32(x)), ref, f"const {x.ravel()[0]}")
    # blocks far below the tensor amax: scale byte 0, all magnitudes 0
    x = np.ones((2, 64), np.float32) * 1e-9
    x[0, 0] = 1e3
    ref, _ = oracle.quantize(x)
    _assert_q_equal(_quant(nv, to_dev_f32(x)), ref, "dynamic range")
    # very small tensors: g denormal, s * g tiny, reciprocal overflow
    rng = np.random.default_rng(6)
    for scale in [1e-38, 1e-40, 1e-42, 1e-44]:
        x = (rng.standard_normal((8, 64)) * scale).astype(np.float32)
        ref, _ = oracle.quantize(x)
        _assert_q_equal(_quant(nv, to_dev_f32(x)), ref, f"scale {scale}")


def test_quantize_nonfinite_sets_flag(nv):
    _note("non-finite flag")
    for bad in [np.nan, np.inf, -np.inf]:
        x = np.ones((4, 64), np.float32)
        x[2, 17] = bad
        flags = torch.zeros(1, dtype=torch.int32, device=DEV)
        nv.quantize(to_dev_f32(x), flags=flags)
        assert flags.item() & 1
        flags.zero_()
        nv.quantize(to_dev_f32(x), amax=torch.tensor([1.0], device=DEV), flags=flags)
        assert flags.item() & 1
    flags = torch.zeros(1, dtype=torch.int32, device=DEV)
    nv.quantize(to_dev_f32(np.ones((4, 64), np.float32)), flags=flags)
    assert flags.item() == 0


def test_requantize_all_e4m3_bytes(nv):
    _note("E4M3 source, all bytes")
    b = np.arange(256, dtype=np.uint32).astype(np.uint8)
    b = b[(b & 0x7F) != 0x7F]  # NaN bytes are checked by the flag test
    x = np.tile(b, 16).reshape(-1, 16 * 2)[:, :32]
    x = np.ascontiguousarray(np.concatenate([x, x[::-1]], axis=0))
    for sc in [None, 0.0123, 1e-30, 3.7e3]:
        ref, _ = oracle.quantize(x, oracle.E4M3, sc)
        s = None if sc is None else torch.tensor([sc], dtype=torch.float32, device=DEV)
        q = _quant(nv, to_dev_u8(x).view(torch.float8_e4m3fn), src_scale=s)
        _assert_q_equal(q, ref, f"e4m3 scale {sc}")
    x2 = x.copy()
    x2[3, 5] = 0xFF
    flags = torch.zeros(1, dtype=torch.int32, device=DEV)
    nv.quantize(to_dev_u8(x2), flags=flags)
    assert flags.item() & 1


def test_requantize_modulation_fp8(nv):
    _note("requantize one 18432x3072 FP8 modulation weight")
    b, sc = synth.modulation_fp8(0)
    ref, _ = oracle.quantize(b, oracle.E4M3, float(sc))
    q = _quant(nv, to_dev_u8(b), src_scale=torch.tensor([sc], dtype=torch.float32, device=DEV))
    _assert_q_equal(q, ref, "modulation fp8")


@pytest.mark.parametrize("shape", [(64, 256), (1000, 3072), (18432, 3072)])
def test_requantize_partial_range_fp8(nv, shape):
    # E4M3 sources whose largest magnitude byte is below 0x7E (448), and an all-zero one: the
    # kernel's full-range guess of the global scale fails and the agreed scale re-encodes every
    # resident tile; codes and scales must still equal the oracle's bit for bit
    _note(f"requantize, partial-range FP8 {shape}")
    rows, cols = shape
    x = synth.normal_f32((rows, cols), 0.01, 77)
    b, sc = synth.fp8_tensorwise(x)
    mag = b & 0x7F
    b = np.where(mag > 0x77, (b & 0x80) | 0x77, b).astype(np.uint8)  # largest magnitude byte 0x77 (240)
    ref, _ = oracle.quantize(b, oracle.E4M3, float(sc))
    assert (ref.codes != 0).any()
    q = _quant(nv, to_dev_u8(b), src_scale=torch.tensor([sc], dtype=torch.float32, device=DEV))
    _assert_q_equal(q, ref, f"partial-range fp8 {shape}")
    if rows <= 1000:
        z = np.zeros_like(b)
        ref0, _ = oracle.quantize(z, oracle.E4M3, float(sc))
        _assert_q_equal(_quant(nv, to_dev_u8(z), src_scale=torch.tensor([sc], dtype=torch.float32, device=DEV)),
                        ref0, f"zero fp8 {shape}")


def test_quantize_replayed_from_hip_graph(nv):
    # run-time amax quantizes (NVFP4 and FP8) captured once in a HIP graph and replayed on new
    # inputs whose amax differs each time: the replays reuse the kernel arguments, so each call's
    # grid agreement must be told apart through its workspace, not its arguments
    rows, cols = 1024, 3072
    _note(f"quantize + quantize_fp8 replayed from a HIP graph, {rows}x{cols}")
    x = torch.zeros((rows, cols), dtype=torch.float32, device=DEV)
    q = nv.NVFP4Tensor.empty(rows, cols, DEV)
    q8 = nv.FP8Tensor.empty(rows, cols, DEV)
    ws = nv.quantize_workspace(DEV)
    ws8 = nv.quantize_workspace(DEV)
    flags = torch.zeros(1, dtype=torch.int32, device=DEV)
    nv.quantize(x, out=q, workspace=ws, flags=flags)
    nv.quantize_fp8(x, out=q8, workspace=ws8, flags=flags)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        nv.quantize(x, out=q, workspace=ws, flags=flags)
        nv.quantize_fp8(x, out=q8, workspace=ws8, flags=flags)
    for i in range(5):
        xi = (np.random.default_rng(700 + i).standard_normal((rows, cols)) * 10.0 ** (i - 2)).astype(np.float32)
        xi[i * 100, 7 * i] = 40.0 * 10.0 ** (i - 2)
        x.copy_(torch.from_numpy(xi))
        flags.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert int(flags.item()) == 0, f"replay {i}"
        _assert_q_equal(q, oracle.quantize(xi)[0], f"replay {i}")
        rb, rs, _ = oracle.quantize_fp8(xi)
        _assert_fp8_equal(q8, rb, rs, f"fp8 replay {i}")


def test_whole_path_replayed_from_hip_graph(nv):
    # every entry point captured once in one HIP graph and replayed on new inputs (written between
    # replays by ordinary stream work); each replay's outputs equal, bit for bit, those of eager
    # calls on the same inputs
    n, k, m, r = 384, 1024, 200, 64
    _note("whole path replayed from a HIP graph")
    w = torch.zeros((n, k), dtype=torch.float32, device=DEV)
    w8 = torch.zeros((n, k), dtype=torch.uint8, device=DEV)
    a = torch.zeros((m, k), dtype=torch.bfloat16, device=DEV)
    sc = torch.tensor([0.01], dtype=torch.float32, device=DEV)
    amax = torch.tensor([4.0], dtype=torch.float32, device=DEV)
    gl = torch.Generator(device="cpu").manual_seed(11)
    v_lr = (torch.randn((r, k), generator=gl) * 0.05).to(torch.bfloat16).to(DEV)
    u_lr = (torch.randn((n, r), generator=gl) * 0.05).to(torch.bfloat16).to(DEV)
    st_out = torch.zeros(8, dtype=torch.float64, device=DEV)  # matrix_stats syncs unless given `out`

    def path():
        qw = nv.quantize(w)
        qw8 = nv.quantize(w8, src_scale=sc)
        qa = nv.quantize(a)
        a8 = nv.quantize_fp8(a)
        pct, mx = nv.amax_percentile(a, 99.9)
        return [qw.codes, qw.scales, qw.global_scale, qw8.codes, qw8.scales, qw8.global_scale,
                qa.codes, qa.scales, qa.global_scale, a8.data, a8.scale, nv.dequantize(qw),
                nv.gemm(a, qw), nv.gemm(qa, qw), nv.gemm(a[:2], qw), nv.gemm(a8, qw), nv.gemm(a8.__class__(
                    a8.data[:3], a8.scale), qw), pct, mx, nv.matrix_stats(w, qw, out=st_out)[:7],
                nv.gemm_lowrank(a, qw, v_lr, u_lr), nv.gemm_qa(a, qw, amax)]

    def refill(seed):
        g = torch.Generator(device="cpu").manual_seed(seed)
        w.copy_(torch.randn((n, k), generator=g) * 0.02)
        b = torch.randint(0, 256, (n, k), generator=g, dtype=torch.int32).to(torch.uint8)
        w8.copy_(torch.where((b & 0x7F) == 0x7F, b - 1, b))
        a.copy_((torch.randn((m, k), generator=g) * (1 + seed % 3)).to(torch.bfloat16))

    refill(0)
    path()
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        outs = path()
    for seed in (1, 2, 3):
        refill(seed)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        got = [t.clone() for t in outs]
        want = path()
        torch.cuda.synchronize()
        for i, (x, y) in enumerate(zip(got, want)):
            assert torch.equal(x, y), f"replay {seed}: output {i} differs from the eager call"


def test_quantize_attention_weight_full(nv):
    _note("quantize 3072x3072 fp32 attention weight")
    w = synth.attn_proj_weight()
    ref, _ = oracle.quantize(w)
    q = _quant(nv, to_dev_f32(w))
    _assert_q_equal(q, ref, "attn weight")
    f32 = nv.dequantize(q, torch.float32).cpu().numpy()
    assert np.array_equal(f32.view(np.uint32), oracle.dequantize(ref, "f32").view(np.uint32))


# Tall tensors whose tile counts (64 blocks per tile, 3 tiles per 3072-wide row) give the
# single-pass kernel 2, 4, 5, 8 and 12 resident tiles per wave at four waves per SIMD on a
# 256-CU part, the largest register residency for fp32, bf16, f16 and e4m3 sources respectively;
# then part of the tiles in LDS (fp32 7000, bf16 9000, f16 14000, e4m3 22000 rows); then more than
# registers and LDS hold, the rest streamed (fp32 18432, bf16 12000, f16 17000, e4m3 24000 rows).
@pytest.mark.parametrize("dtype,rows", [("f32", 2000), ("f32", 5000), ("bf16", 6000), ("f16", 10000),
                                        ("e4m3", 15000), ("f32", 7000), ("bf16", 9000), ("f16", 14000),
                                        ("e4m3", 22000), ("f32", 18432), ("bf16", 12000), ("f16", 17000),
                                        ("e4m3", 24000)])
def test_quantize_resident_tiles_per_wave(nv, dtype, rows):
    cols = 3072
    _note(f"quantize {dtype} {rows}x{cols}")
    g = synth.rng(rows + 31)
    x = (g.standard_t(5, size=(rows, cols)) * 0.02).astype(np.float32)
    x[g.random((rows, cols)) < 0.01] = 0.0
    if dtype == "f32":
        xd, ref = to_dev_f32(x), oracle.quantize(x)[0]
        _assert_q_equal(_quant(nv, xd), ref, f"{dtype} {rows}")
    elif dtype == "bf16":
        b = synth.bf16_bits(x)
        _assert_q_equal(_quant(nv, to_dev_bf16(b)), oracle.quantize(b, oracle.BF16)[0], f"{dtype} {rows}")
    elif dtype == "f16":
        h = x.astype(np.float16).view(np.uint16)
        _assert_q_equal(_quant(nv, to_dev_f16(h)), oracle.quantize(h, oracle.F16)[0], f"{dtype} {rows}")
    else:
        b, sc = synth.fp8_tensorwise(x)
        ref, _ = oracle.quantize(b, oracle.E4M3, float(sc))
        q = _quant(nv, to_dev_u8(b), src_scale=torch.tensor([sc], dtype=torch.float32, device=DEV))
        _assert_q_equal(q, ref, f"{dtype} {rows}")


# ------------------------------------------------------------------------------------------------
# dequantize
# ------------------------------------------------------------------------------------------------
@pytest.mark.parametrize("shape", [(1, 16), (5, 48), (33, 1024), (257, 272)])
def test_dequantize_random_codes(nv, shape):
    _note(f"dequantize {shape}")
    rows, cols = shape
    rng = np.random.default_rng(rows + cols)
    codes = rng.integers(0, 256, (rows, cols // 2), dtype=np.uint8)
    scales = rng.integers(0, 0x7F, (rows, cols // 16), dtype=np.uint8)
    for g in [np.float32(0.0017439), np.float32(2.5e-39), np.float32(1e30)]:
        ref = oracle.QTensor(codes, scales, g)
        import bit_gemm_nvfp4_amd as nvm
        q = nvm.NVFP4Tensor(to_dev_u8(codes), to_dev_u8(scales), torch.tensor([g], dtype=torch.float32, device=DEV))
        f32 = nv.dequantize(q, torch.float32).cpu().numpy()
        assert np.array_equal(f32.view(np.uint32), oracle.dequantize(ref, "f32").view(np.uint32))
        bf = bits16(nv.dequantize(q, torch.bfloat16))
        assert np.array_equal(bf, oracle.dequantize(ref, "bf16"))
        if rows > 1:
            out = padded(torch.empty((rows, cols), dtype=torch.bfloat16, device=DEV), 8)
            nv.dequantize(q, out=out)
            assert np.array_equal(bits16(out.contiguous()), oracle.dequantize(ref, "bf16"))


# ------------------------------------------------------------------------------------------------
# GEMM
# ------------------------------------------------------------------------------------------------
def _rand_q(nv, rows, cols, seed, sigma=0.02):
    w = synth.normal_f32((rows, cols), sigma, seed)
    ref, _ = oracle.quantize(w)
    q = _quant(nv, to_dev_f32(w))
    _assert_q_equal(q, ref, f"weight {rows}x{cols}")
    return q, ref


# M <= 4 take the register GEMV up to K = 4096 and the LDS form beyond (6144, 8192); 5 <= M <= 16 with
# K a multiple of 32 up to 4096 the matrix-core GEMV; other M = 5 the LDS GEMV; the rest the tiled
# kernels
@pytest.mark.parametrize("mnk", [(16, 64, 256), (1, 64, 128), (2, 100, 48), (3, 33, 4096), (4, 17, 16),
                                 (5, 70, 80), (37, 129, 272), (130, 257, 1024), (256, 128, 64), (300, 200, 3072),
                                 (2, 300, 8192), (4, 129, 6144), (6, 1000, 3072), (7, 65, 4096), (8, 300, 4096),
                                 (8, 64, 8192), (9, 100, 1024)])
def test_gemm_w4a16(nv, mnk):
    m, n, k = mnk
    _note(f"gemm w4a16 {mnk}")
    q, ref = _rand_q(nv, n, k, seed=m * 31 + n)
    a_bits = synth.bf16_bits(np.random.default_rng(m + k).standard_normal((m, k)).astype(np.float32))
    c = nv.gemm(to_dev_bf16(a_bits), q).cpu().numpy()
    err = oracle.gemm_error(c, oracle.gemm_w4a16(a_bits, ref))
    assert err <= GEMM_TOL, err
    if m > 1:  # strided A and C
        a = padded(to_dev_bf16(a_bits), 8)
        out = padded(torch.empty((m, n), dtype=torch.float32, device=DEV), 4)
        nv.gemm(a, q, out=out)
        assert np.array_equal(out.cpu().numpy(), c)


@pytest.mark.parametrize("mnk", [(16, 64, 256), (2, 300, 1024), (4, 64, 16), (64, 96, 112), (200, 300, 512),
                                 (2, 100, 8192), (5, 200, 2048), (8, 100, 4096)])
def test_gemm_w4a4(nv, mnk):
    m, n, k = mnk
    _note(f"gemm w4a4 {mnk}")
    q, ref = _rand_q(nv, n, k, seed=m * 17 + n)
    a_bits = synth.bf16_bits(np.random.default_rng(m * 3 + k).standard_normal((m, k)).astype(np.float32))
    aq = _quant(nv, to_dev_bf16(a_bits))
    aref, _ = oracle.quantize(a_bits, oracle.BF16)
    _assert_q_equal(aq, aref, "activations")
    c = nv.gemm(aq, q).cpu().numpy()
    err = oracle.gemm_error(c, oracle.gemm_w4a4(aref, ref))
    assert err <= GEMM_TOL, err


def test_gemm_one_hot_reproduces_expansion(nv):
    _note("gemm one-hot")
    q, ref = _rand_q(nv, 192, 320, seed=99)
    eye = np.zeros((320, 320), np.float32)
    eye[np.arange(320), np.arange(320)] = 1.0
    # exact equality of values (a -0 weight times 1 summed with +0 products gives +0)
    c = nv.gemm(to_dev_bf16(synth.bf16_bits(eye)), q).cpu().numpy()
    assert np.array_equal(c, oracle.dequantize(ref, "f32").T)
    for m in [1, 2, 3, 4]:  # the GEMV path
        cm = nv.gemm(to_dev_bf16(synth.bf16_bits(eye[:m])), q).cpu().numpy()
        assert np.array_equal(cm, oracle.dequantize(ref, "f32").T[:m])


def test_gemm_zero_weight_and_empty(nv):
    _note("gemm zero weight / empty")
    z = _quant(nv, to_dev_f32(np.zeros((64, 128), np.float32)))
    a = to_dev_bf16(synth.bf16_bits(np.ones((8, 128), np.float32)))
    assert not nv.gemm(a, z).cpu().numpy().any()
    # K = 0: C = 0
    import bit_gemm_nvfp4_amd as nvm
    w0 = nvm.NVFP4Tensor(torch.zeros((5, 0), dtype=torch.uint8, device=DEV),
                         torch.zeros((5, 0), dtype=torch.uint8, device=DEV), torch.ones(1, device=DEV))
    a0 = torch.zeros((3, 0), dtype=torch.bfloat16, device=DEV)
    out = torch.full((3, 5), 7.0, device=DEV)
    nv.gemm(a0, w0, out=out)
    assert not out.cpu().numpy().any()


def test_gemm_attention_projection_full(nv):
    _note("gemm w4a16 4096x3072x3072 (full) + w4a4")
    w = synth.attn_proj_weight()
    a_bits = synth.attn_proj_activations()
    ref, _ = oracle.quantize(w)
    q = _quant(nv, to_dev_f32(w))
    _assert_q_equal(q, ref, "attn weight")
    c = nv.gemm(to_dev_bf16(a_bits), q).cpu().numpy()
    cref = oracle.gemm_w4a16(a_bits, ref)
    err = oracle.gemm_error(c, cref)
    # informational: the NVFP4 product against the unquantized one (fp32 W, bf16 A) in fp64
    cu = oracle.gemm_f64(oracle.bf16_bits_to_f64(a_bits[:256]), w.astype(np.float64))
    qerr = np.linalg.norm(c[:256] - cu) / np.linalg.norm(cu)
    _note(f"  W4A16 floored max rel err {err:.3e}, normwise {np.abs(c - cref).max() / np.abs(cref).max():.3e}, "
          f"vs unquantized (256 rows, Frobenius) {qerr:.3e}")
    assert err <= GEMM_TOL
    aq = _quant(nv, to_dev_bf16(a_bits))
    aref, _ = oracle.quantize(a_bits, oracle.BF16)
    _assert_q_equal(aq, aref, "activations")
    rows = np.random.default_rng(1).choice(4096, 256, replace=False)
    c4 = nv.gemm(aq, q).cpu().numpy()[rows]
    c4ref = oracle.gemm_f64(oracle.dequantize(aref, "f64")[rows], oracle.dequantize(ref, "f64"))
    assert oracle.gemm_error(c4, c4ref) <= GEMM_TOL


def test_mlp_w4a4_chain_full(nv):
    # the Qwen3-VL-8B text MLP at full size: gate / up 12288 x 4096 and down 4096 x 12288 NVFP4
    # weights, 512 tokens of bf16 activations quantized with their run-time amax, W4A4 products.
    # The intermediate between the projections (SiLU(gate) * up, rounded to bf16) is test glue,
    # formed from the oracle's gate and up outputs; both sides quantize and project it.
    _note("Qwen3-VL MLP chain 512 x 4096 -> 12288 -> 4096, W4A4")
    wg, wu, wd = synth.mlp_weights()
    qs, refs = [], []
    for w in (wg, wu, wd):
        ref, _ = oracle.quantize(w)
        q = _quant(nv, to_dev_f32(w))
        _assert_q_equal(q, ref, f"mlp weight {w.shape}")
        qs.append(q)
        refs.append(ref)
    a_bits = synth.mlp_activations()
    aq = _quant(nv, to_dev_bf16(a_bits))
    aref, _ = oracle.quantize(a_bits, oracle.BF16)
    _assert_q_equal(aq, aref, "mlp activations")
    gate_ref = oracle.gemm_w4a4(aref, refs[0])
    up_ref = oracle.gemm_w4a4(aref, refs[1])
    assert oracle.gemm_error(nv.gemm(aq, qs[0]).cpu().numpy(), gate_ref) <= GEMM_TOL
    assert oracle.gemm_error(nv.gemm(aq, qs[1]).cpu().numpy(), up_ref) <= GEMM_TOL
    h_bits = synth.bf16_bits((gate_ref / (1.0 + np.exp(-gate_ref)) * up_ref).astype(np.float32))
    hq = _quant(nv, to_dev_bf16(h_bits))
    href, _ = oracle.quantize(h_bits, oracle.BF16)
    _assert_q_equal(hq, href, "mlp intermediate")
    down = nv.gemm(hq, qs[2]).cpu().numpy()
    assert oracle.gemm_error(down, oracle.gemm_w4a4(href, refs[2])) <= GEMM_TOL


# one block of the 60-block layer stack: its six FP8 weights requantized (bit-exact), then each
# one's W4A16 product at M = 4096, checked on 64 sampled rows
@pytest.mark.parametrize("j", range(6))
def test_stack_block_requantize_and_gemm(nv, j):
    block = 37
    _note(f"stack block {block} weight {j}")
    b, sc = synth.stack_weight_fp8(block, j)
    ref, _ = oracle.quantize(b, oracle.E4M3, float(sc))
    q = _quant(nv, to_dev_u8(b), src_scale=torch.tensor([sc], dtype=torch.float32, device=DEV))
    _assert_q_equal(q, ref, f"stack {block}.{j}")
    k = b.shape[1]
    a_bits = synth.bf16_bits(synth.rng(5500 + j).standard_normal((4096, k)).astype(np.float32))
    c = nv.gemm(to_dev_bf16(a_bits), q)
    rows = np.sort(synth.rng(5600 + j).choice(4096, 64, replace=False))
    cs = c[torch.from_numpy(rows).to(DEV)].cpu().numpy()
    assert oracle.gemm_error(cs, oracle.gemm_w4a16(a_bits[rows], ref)) <= GEMM_TOL


def test_gemv_fp8a_modulation_full(nv):
    # the modulation GEMV with its two activation rows as FP8 (dynamic tensor scale)
    _note("gemv fp8a M=2 over 18432x3072")
    w = synth.modulation_weight()
    ref, _ = oracle.quantize(w)
    q = _quant(nv, to_dev_f32(w))
    a_bits = synth.modulation_activations()
    a8 = _quant_fp8(nv, to_dev_bf16(a_bits))
    rb, rs, _ = oracle.quantize_fp8(a_bits, oracle.BF16)
    _assert_fp8_equal(a8, rb, rs, "activations")
    c = nv.gemm(a8, q).cpu().numpy()
    assert oracle.gemm_error(c, oracle.gemm_w4a8(rb, rs, ref)) <= GEMM_TOL


def test_gemv_modulation_full(nv):
    _note("gemv M=2 over 18432x3072")
    w = synth.modulation_weight()
    ref, _ = oracle.quantize(w)
    q = _quant(nv, to_dev_f32(w))
    _assert_q_equal(q, ref, "modulation weight")
    a_bits = synth.modulation_activations()
    c = nv.gemm(to_dev_bf16(a_bits), q).cpu().numpy()
    assert oracle.gemm_error(c, oracle.gemm_w4a16(a_bits, ref)) <= GEMM_TOL


# ------------------------------------------------------------------------------------------------
# percentile
# ------------------------------------------------------------------------------------------------
@pytest.mark.parametrize("dtype", ["bf16", "f32", "f16"])
@pytest.mark.parametrize("shape", [(1, 16), (7, 48), (1000, 272), (4097, 64)])
def test_percentile(nv, dtype, shape):
    _note(f"percentile {dtype} {shape}")
    rng = np.random.default_rng(shape[0] + shape[1])
    x = rng.standard_t(3, size=shape).astype(np.float32)
    x[rng.random(shape) < 0.01] = -0.0
    if dtype == "bf16":
        src, xd, odt = synth.bf16_bits(x), None, oracle.BF16
        xd = to_dev_bf16(src)
    elif dtype == "f16":
        src, odt = x.astype(np.float16).view(np.uint16), oracle.F16
        xd = to_dev_f16(src)
    else:
        src, odt = x, oracle.F32
        xd = to_dev_f32(src)
    # 99.9 / 100 / 1e-6 and 99.63 / 0.3 take the one-pass path near either end of a channel (up
    # to 16 from the end), 50 the radix path
    for p in [99.9, 50.0, 100.0, 1e-6, 99.63, 0.3]:
        for per_channel in [True, False]:
            pct, mx = nv.amax_percentile(xd, p, per_channel)
            rp, rm = oracle.amax_percentile(src, p, per_channel, dtype=odt)
            assert np.array_equal(pct.cpu().numpy(), rp), (p, per_channel)
            assert np.array_equal(mx.cpu().numpy(), rm), (p, per_channel)
    if shape[0] > 1:
        pct, mx = nv.amax_percentile(padded(xd, 16), 99.9)
        rp, rm = oracle.amax_percentile(src, 99.9, dtype=odt)
        assert np.array_equal(pct.cpu().numpy(), rp)


# the m-th largest and m-th smallest of 4096-row channels for m = 1..17: every list length of the
# one-pass path (1-6, 8, 12, 16) at and just past its bucket edge, and the radix path beyond 16
@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("m", [1, 2, 3, 4, 5, 6, 7, 8, 9, 12, 13, 16, 17])
def test_percentile_rank_near_ends(nv, dtype, m):
    rows, cols = 4096, 64
    _note(f"percentile {dtype} rank {m} from either end")
    x = np.random.default_rng(900 + m).standard_t(3, size=(rows, cols)).astype(np.float32)
    if dtype == "bf16":
        src, odt = synth.bf16_bits(x), oracle.BF16
        xd = to_dev_bf16(src)
    else:
        src, odt = x, oracle.F32
        xd = to_dev_f32(src)
    for k in (rows - m + 1, m):
        p = 100.0 * (k - 0.5) / rows  # nearest rank k
        pct, mx = nv.amax_percentile(xd, p)
        rp, rm = oracle.amax_percentile(src, p, dtype=odt)
        assert np.array_equal(pct.cpu().numpy(), rp), (m, k)
        assert np.array_equal(mx.cpu().numpy(), rm), (m, k)


def _pct_input(dtype, x):
    if dtype == "bf16":
        src = synth.bf16_bits(x)
        return src, to_dev_bf16(src), oracle.BF16
    if dtype == "f16":
        src = x.astype(np.float16).view(np.uint16)
        return src, to_dev_f16(src), oracle.F16
    return x, to_dev_f32(x), oracle.F32


# ranks 17 .. about 250 from an end on at least 32768 rows take the candidate path: a threshold
# from every 16th row, one pass keeping the keys beyond it, the rank selected among them
@pytest.mark.parametrize("dtype", ["bf16", "f16", "f32"])
@pytest.mark.parametrize("cols", [64, 272])
def test_percentile_candidate_path(nv, dtype, cols):
    rows = 40000
    _note(f"percentile candidate path {dtype} {rows}x{cols}")
    rng = np.random.default_rng(4000 + cols)
    x = rng.standard_t(3, size=(rows, cols)).astype(np.float32)
    x[rng.random(x.shape) < 0.01] = -0.0
    src, xd, odt = _pct_input(dtype, x)
    for m in (17, 201, 250):
        for k in (rows - m + 1, m):  # the m-th largest, then the m-th smallest
            p = 100.0 * (k - 0.5) / rows
            pct, mx = nv.amax_percentile(xd, p)
            rp, rm = oracle.amax_percentile(src, p, dtype=odt)
            assert np.array_equal(pct.cpu().numpy(), rp), (m, k)
            assert np.array_equal(mx.cpu().numpy(), rm), (m, k)


def test_percentile_candidate_fallbacks(nv, monkeypatch):
    # channels the candidates cannot settle go through the exact passes: (a) a sample that
    # overstates the tail (every 16th row, the sampled ones, is 8x larger in channels 0-31), (b)
    # equal values (every candidate list overflows), (c) a list capacity of one (every channel)
    rows, cols = 40000, 64
    _note("percentile candidate fallbacks")
    rng = np.random.default_rng(77)
    x = rng.standard_t(3, size=(rows, cols)).astype(np.float32)
    x[0::16, :32] *= 8.0
    x[:, 40:48] = 1.5
    src, xd, odt = _pct_input("bf16", x)
    for p in (99.5, 0.5):
        rp, rm = oracle.amax_percentile(src, p, dtype=odt)
        pct, mx = nv.amax_percentile(xd, p)
        assert np.array_equal(pct.cpu().numpy(), rp), p
        assert np.array_equal(mx.cpu().numpy(), rm), p
        monkeypatch.setenv("NVFP4_PCT_CAND_CAP", "1")
        pct, mx = nv.amax_percentile(xd, p)
        monkeypatch.delenv("NVFP4_PCT_CAND_CAP")
        assert np.array_equal(pct.cpu().numpy(), rp), p
        assert np.array_equal(mx.cpu().numpy(), rm), p


def test_percentile_attention_activations_full(nv):
    # the activations of the attention projection, per-channel p99.9 (the 5th largest of 4096)
    _note("percentile 4096 x 3072 bf16")
    a_bits = synth.attn_proj_activations(4096, 3072)
    pct, mx = nv.amax_percentile(to_dev_bf16(a_bits), 99.9)
    rp, rm = oracle.amax_percentile(a_bits, 99.9, dtype=oracle.BF16)
    assert np.array_equal(pct.cpu().numpy(), rp) and np.array_equal(mx.cpu().numpy(), rm)


def test_percentile_calibration_full_rows(nv):
    # 53 x 4096 rows of Student-t(3) at the calibration size, on 128 of the 3072 channels
    _note("percentile 217088 x 128 bf16")
    x = synth.calib_activations(cols=128)
    pct, mx = nv.amax_percentile(to_dev_bf16(x), 99.9)
    rp, rm = oracle.amax_percentile(x, 99.9, dtype=oracle.BF16)
    assert np.array_equal(pct.cpu().numpy(), rp) and np.array_equal(mx.cpu().numpy(), rm)


def test_percentile_long_row_chunks(nv):
    # 2.1 M rows on 16 channels: the histogram pass gives each workgroup over 8192 rows (16 rows in
    # flight per lane), with a ragged last chunk
    _note("percentile 2100000 x 16 bf16")
    x = synth.calib_activations(rows=2_100_000, cols=16, seed=5001)
    xd = to_dev_bf16(x)
    for p, per_channel in [(99.9, True), (50.0, True), (99.9, False)]:
        pct, mx = nv.amax_percentile(xd, p, per_channel)
        rp, rm = oracle.amax_percentile(x, p, per_channel, dtype=oracle.BF16)
        assert np.array_equal(pct.cpu().numpy(), rp), (p, per_channel)
        assert np.array_equal(mx.cpu().numpy(), rm), (p, per_channel)


def test_percentile_counter_capacity(nv):
    # 65535 x 256 + 1000 rows that are all 1.0 but for +-2.0 in the last 100 rows: with 256 row
    # chunks a chunk would count more than 65535 equal keys of one channel, so the launch must cut
    # the rows finer.  The answer is known in closed form: the m-th largest |x| of a channel is 2.0
    # for m <= 100 and 1.0 beyond (m > 16 keeps it on the histogram path).
    rows, cols = 65535 * 256 + 1000, 16
    _note(f"percentile {rows} x {cols} bf16, counter capacity")
    x = torch.full((rows, cols), 1.0, dtype=torch.bfloat16, device=DEV)
    x[-100:, 0::2] = -2.0
    x[-100:, 1::2] = 2.0
    for n, per_channel, m_two in [(rows, True, 100), (rows * cols, False, 100 * cols)]:
        for m in [m_two // 2, m_two, m_two + 1, 3 * m_two]:
            p = 100.0 * (n - m + 0.5) / n  # nearest rank n - m + 1: the m-th largest
            pct, mx = nv.amax_percentile(x, p, per_channel)
            want = 2.0 if m <= m_two else 1.0
            assert torch.all(pct == want).item(), (per_channel, m, pct[:4].tolist())
            assert torch.all(mx == 2.0).item(), (per_channel, m)
    del x


# shapes that select each of the GEMM kernel's tile configurations (256x256, 256x192, 128x256,
# 128x128, 128x192), with aligned and ragged K and ragged M / N edges
@pytest.mark.parametrize("mnk", [(576, 16384, 64), (448, 16512, 64), (390, 16300, 128), (704, 10880, 128),
                                 (130, 1000, 128), (3000, 5000, 80), (250, 12400, 48), (700, 10800, 80)])
def test_gemm_tile_configs(nv, mnk):
    m, n, k = mnk
    _note(f"gemm tile configs {mnk}")
    q, ref = _rand_q(nv, n, k, seed=m + n + k)
    a_bits = synth.bf16_bits(np.random.default_rng(m * 7 + k).standard_normal((m, k)).astype(np.float32))
    c = nv.gemm(to_dev_bf16(a_bits), q).cpu().numpy()
    assert oracle.gemm_error(c, oracle.gemm_w4a16(a_bits, ref)) <= GEMM_TOL
    aq = _quant(nv, to_dev_bf16(a_bits))
    aref, _ = oracle.quantize(a_bits, oracle.BF16)
    _assert_q_equal(aq, aref, "activations")
    c4 = nv.gemm(aq, q).cpu().numpy()
    assert oracle.gemm_error(c4, oracle.gemm_w4a4(aref, ref)) <= GEMM_TOL


# few output tiles and a long K: the product is split along K (partial planes in the workspace,
# summed in slice order); ragged M and N edges, and the Qwen3-VL MLP down projection
@pytest.mark.parametrize("mnk", [(100, 1000, 4096), (512, 4096, 12288)])
def test_gemm_split_k(nv, mnk):
    m, n, k = mnk
    _note(f"gemm split-K {mnk}")
    assert nv.workspace_size(nv.OP_GEMM, m, n, k) > 0
    q, ref = _rand_q(nv, n, k, seed=m + n + k, sigma=0.015)
    a_bits = synth.bf16_bits(np.random.default_rng(m + 5).standard_normal((m, k)).astype(np.float32))
    c = nv.gemm(to_dev_bf16(a_bits), q).cpu().numpy()
    assert oracle.gemm_error(c, oracle.gemm_w4a16(a_bits, ref)) <= GEMM_TOL
    aq = _quant(nv, to_dev_bf16(a_bits))
    aref, _ = oracle.quantize(a_bits, oracle.BF16)
    _assert_q_equal(aq, aref, "activations")
    c4 = nv.gemm(aq, q).cpu().numpy()
    assert oracle.gemm_error(c4, oracle.gemm_w4a4(aref, ref)) <= GEMM_TOL


def test_quantize_large_tensor_overflow_path(nv):
    # more tiles than the single-pass kernel holds in registers: part of the input is read twice
    _note("quantize 16384 x 8192 fp32 (128 M elements)")
    rng = np.random.default_rng(77)
    x = (rng.standard_normal((16384, 8192)) * 0.01).astype(np.float32)
    x[123, 4567] = 0.75
    q = _quant(nv, to_dev_f32(x))
    ref, _ = oracle.quantize(x)
    _assert_q_equal(q, ref, "large")


# ------------------------------------------------------------------------------------------------
# FP8 tensorwise quantizer and the GEMM with FP8 activations
# ------------------------------------------------------------------------------------------------
def _quant_fp8(nv, x, **kw):
    flags = torch.zeros(1, dtype=torch.int32, device=DEV)
    q = nv.quantize_fp8(x, flags=flags, **kw)
    f = int(flags.item())
    assert f == 0, f"quantize_fp8 flags {f:#x}"
    return q


def _assert_fp8_equal(q, ref_bytes, ref_scale, what=""):
    s = q.scale.cpu().numpy()[0]
    assert s.view(np.uint32) == np.float32(ref_scale).view(np.uint32), f"{what} scale {s} vs {ref_scale}"
    b = q.data.cpu().numpy()
    bad = np.nonzero(b != ref_bytes)
    assert bad[0].size == 0, (f"{what} {bad[0].size} bytes differ, first at {bad[0][0]},{bad[1][0]}: "
                              f"{b[bad[0][0], bad[1][0]]:#x} vs {ref_bytes[bad[0][0], bad[1][0]]:#x}")


def _fp8_case(x, dtype):
    """(device tensor, oracle bytes, oracle scale) for fp32 values x given as dtype."""
    if dtype == "f32":
        return to_dev_f32(x), *oracle.quantize_fp8(x)[:2]
    if dtype == "bf16":
        b = synth.bf16_bits(x)
        return to_dev_bf16(b), *oracle.quantize_fp8(b, oracle.BF16)[:2]
    h = x.astype(np.float16).view(np.uint16)
    return to_dev_f16(h), *oracle.quantize_fp8(h, oracle.F16)[:2]


@pytest.mark.parametrize("shape", SHAPES + [(2000, 3072), (4096, 3072)])
@pytest.mark.parametrize("dtype", ["f32", "bf16", "f16"])
def test_quantize_fp8_shapes_dtypes(nv, shape, dtype):
    rows, cols = shape
    _note(f"quantize_fp8 {dtype} {shape}")
    rng = np.random.default_rng(rows * 131 + cols)
    x = (rng.standard_t(4, size=shape) * 10.0 ** rng.uniform(-3, 1)).astype(np.float32)
    x[rng.random(shape) < 0.05] = 0.0
    x[rng.random(shape) < 0.02] *= -0.0
    xd, rb, rs = _fp8_case(x, dtype)
    _assert_fp8_equal(_quant_fp8(nv, xd), rb, rs, f"{dtype} {shape}")
    if rows > 1:
        _assert_fp8_equal(_quant_fp8(nv, padded(xd, 16)), rb, rs, f"{dtype} {shape} strided")


def test_quantize_fp8_from_fp8_static_zero_and_flags(nv):
    _note("quantize_fp8: E4M3 source, static amax, zeros, non-finite")
    rng = np.random.default_rng(8)
    w = (rng.standard_normal((96, 512)) * 0.02).astype(np.float32)
    b8, sc = synth.fp8_tensorwise(w)
    rb, rs, _ = oracle.quantize_fp8(b8, oracle.E4M3, float(sc))
    q = _quant_fp8(nv, to_dev_u8(b8), src_scale=torch.tensor([sc], dtype=torch.float32, device=DEV))
    _assert_fp8_equal(q, rb, rs, "e4m3 source")
    amax = np.float32(0.01)
    rb, rs, _ = oracle.quantize_fp8(w, amax=float(amax))
    q = nv.quantize_fp8(to_dev_f32(w), amax=torch.tensor([amax], dtype=torch.float32, device=DEV))
    _assert_fp8_equal(q, rb, rs, "static amax")
    z = np.zeros((33, 64), np.float32)
    rb, rs, _ = oracle.quantize_fp8(z)
    _assert_fp8_equal(_quant_fp8(nv, to_dev_f32(z)), rb, rs, "zeros")
    w[5, 7] = np.inf
    flags = torch.zeros(1, dtype=torch.int32, device=DEV)
    nv.quantize_fp8(to_dev_f32(w), flags=flags)
    assert flags.item() & 1
    flags.zero_()
    nv.quantize_fp8(to_dev_f32(w), amax=torch.tensor([1.0], device=DEV), flags=flags)
    assert flags.item() & 1


@pytest.mark.parametrize("dtype,rows", [("f32", 6000), ("bf16", 12000)])
def test_quantize_fp8_lds_and_streamed_tiles(nv, dtype, rows):
    # the FP8 output of the single-pass kernel with part of the tiles in LDS (fp32 6000 rows), and
    # with the rest streamed (bf16 12000 rows)
    _note(f"quantize_fp8 {dtype} {rows}x3072")
    x = (np.random.default_rng(rows).standard_normal((rows, 3072)) * 0.02).astype(np.float32)
    if dtype == "f32":
        xd, xh, odt = to_dev_f32(x), x, oracle.F32
    else:
        xh = synth.bf16_bits(x)
        xd, odt = to_dev_bf16(xh), oracle.BF16
    rb, rs, _ = oracle.quantize_fp8(xh, odt)
    _assert_fp8_equal(_quant_fp8(nv, xd), rb, rs, f"{dtype} {rows}")


def test_quantize_fp8_streamed_tensor(nv):
    _note("quantize_fp8 16384 x 8192 fp32 (streaming path)")
    rng = np.random.default_rng(78)
    x = (rng.standard_normal((16384, 8192)) * 0.01).astype(np.float32)
    x[99, 4321] = -0.5
    rb, rs, _ = oracle.quantize_fp8(x)
    _assert_fp8_equal(_quant_fp8(nv, to_dev_f32(x)), rb, rs, "large")


# K % 64 != 0 takes k_gemm_tile; M <= 4 the GEMV forms (A in registers for K <= 4096, in LDS beyond)
@pytest.mark.parametrize("mnk", [(16, 64, 256), (1, 64, 128), (4, 100, 48), (5, 70, 80), (37, 129, 272),
                                 (130, 257, 1024), (300, 200, 3072), (576, 16384, 64), (130, 1000, 128),
                                 (2, 300, 4608), (3, 1000, 3072), (4, 257, 8192), (6, 300, 3072), (8, 129, 4096)])
def test_gemm_fp8a(nv, mnk):
    m, n, k = mnk
    _note(f"gemm fp8a {mnk}")
    q, ref = _rand_q(nv, n, k, seed=m * 13 + n)
    x = np.random.default_rng(m * 7 + k).standard_normal((m, k)).astype(np.float32)
    a8 = _quant_fp8(nv, to_dev_f32(x))
    rb, rs, _ = oracle.quantize_fp8(x)
    _assert_fp8_equal(a8, rb, rs, "activations")
    c = nv.gemm(a8, q).cpu().numpy()
    err = oracle.gemm_error(c, oracle.gemm_w4a8(rb, rs, ref))
    assert err <= GEMM_TOL, err
    if m > 1:  # strided A and C
        import bit_gemm_nvfp4_amd as nvm
        a = nvm.FP8Tensor(padded(a8.data, 16), a8.scale)
        out = padded(torch.empty((m, n), dtype=torch.float32, device=DEV), 4)
        nv.gemm(a, q, out=out)
        assert np.array_equal(out.cpu().numpy(), c)


# The matrix-core GEMV (5 <= M <= 16, K % 32 == 0, K <= 4096): K ending inside a 128-element chunk
# (32, 96, 160, 4064), N not a multiple of 16, and the three activation forms
@pytest.mark.parametrize("form", ["w4a16", "w4a4", "fp8a"])
@pytest.mark.parametrize("mnk", [(5, 17, 32), (5, 100, 96), (11, 33, 160), (16, 1000, 4064), (16, 37, 3072),
                                 (7, 250, 4096), (12, 129, 1024)])
def test_gemv_mfma(nv, form, mnk):
    m, n, k = mnk
    _note(f"gemv mfma {form} {mnk}")
    q, ref = _rand_q(nv, n, k, seed=m * 19 + n + k)
    x = np.random.default_rng(m * 5 + k).standard_normal((m, k)).astype(np.float32)
    if form == "w4a16":
        a_bits = synth.bf16_bits(x)
        c = nv.gemm(to_dev_bf16(a_bits), q).cpu().numpy()
        want = oracle.gemm_w4a16(a_bits, ref)
    elif form == "w4a4":
        a_bits = synth.bf16_bits(x)
        aq = _quant(nv, to_dev_bf16(a_bits))
        aref, _ = oracle.quantize(a_bits, oracle.BF16)
        _assert_q_equal(aq, aref, "activations")
        c = nv.gemm(aq, q).cpu().numpy()
        want = oracle.gemm_w4a4(aref, ref)
    else:
        a8 = _quant_fp8(nv, to_dev_f32(x))
        rb, rs, _ = oracle.quantize_fp8(x)
        _assert_fp8_equal(a8, rb, rs, "activations")
        c = nv.gemm(a8, q).cpu().numpy()
        want = oracle.gemm_w4a8(rb, rs, ref)
    err = oracle.gemm_error(c, want)
    assert err <= GEMM_TOL, err


# the matrix-core GEMV at the modulation shape (18432 x 3072) with 16 rows of A: every output
def test_gemv_mfma_modulation_full(nv):
    n, k, m = 18432, 3072, 16
    _note("gemv mfma 16 x 18432 x 3072")
    q, ref = _rand_q(nv, n, k, seed=4242)
    a_bits = synth.bf16_bits(np.random.default_rng(4243).standard_normal((m, k)).astype(np.float32))
    c = nv.gemm(to_dev_bf16(a_bits), q).cpu().numpy()
    err = oracle.gemm_error(c, oracle.gemm_w4a16(a_bits, ref))
    assert err <= GEMM_TOL, err


def test_gemm_fp8a_one_hot_all_bytes(nv):
    # every finite E4M3 byte times a one-hot row: C reproduces the exact products e4m3 x w_hat x scale
    _note("gemm fp8a one-hot over all E4M3 bytes")
    q, ref = _rand_q(nv, 64, 256, seed=7)
    import bit_gemm_nvfp4_amd as nvm
    bts = np.array([b for b in range(256) if (b & 0x7F) != 0x7F], dtype=np.uint8)
    a = np.zeros((bts.size, 256), dtype=np.uint8)
    a[np.arange(bts.size), np.arange(bts.size) % 256] = bts
    sc = np.float32(0.5)
    a8 = nvm.FP8Tensor(to_dev_u8(a), torch.tensor([sc], dtype=torch.float32, device=DEV))
    c = nv.gemm(a8, q).cpu().numpy()
    cref = oracle.gemm_w4a8(a, sc, ref)
    assert np.array_equal(c.astype(np.float64), cref.astype(np.float32).astype(np.float64))
    # the same rows four at a time through the GEMV form
    cv = np.concatenate([nv.gemm(nvm.FP8Tensor(to_dev_u8(np.ascontiguousarray(a[i:i + 4])), a8.scale), q).cpu().numpy()
                         for i in range(0, bts.size, 4)])
    assert np.array_equal(cv.astype(np.float64), cref.astype(np.float32).astype(np.float64))


def test_gemm_fp8a_split_k_and_full(nv):
    _note("gemm fp8a split-K 512x4096x12288, attention projection 4096x3072x3072 (sampled rows)")
    m, n, k = 512, 4096, 12288
    assert nv.workspace_size(nv.OP_GEMM, m, n, k) > 0
    q, ref = _rand_q(nv, n, k, seed=5, sigma=0.015)
    x = np.random.default_rng(6).standard_normal((m, k)).astype(np.float32)
    a8 = _quant_fp8(nv, to_dev_f32(x))
    rb, rs, _ = oracle.quantize_fp8(x)
    _assert_fp8_equal(a8, rb, rs, "split-K activations")
    assert oracle.gemm_error(nv.gemm(a8, q).cpu().numpy(), oracle.gemm_w4a8(rb, rs, ref)) <= GEMM_TOL
    w = synth.attn_proj_weight()
    ref, _ = oracle.quantize(w)
    q = _quant(nv, to_dev_f32(w))
    a_bits = synth.attn_proj_activations()
    a8 = _quant_fp8(nv, to_dev_bf16(a_bits))
    rb, rs, _ = oracle.quantize_fp8(a_bits, oracle.BF16)
    _assert_fp8_equal(a8, rb, rs, "attention activations")
    rows = np.random.default_rng(2).choice(4096, 256, replace=False)
    c = nv.gemm(a8, q).cpu().numpy()[rows]
    cref = oracle.gemm_f64(oracle.fp8_values(rb[rows], rs), oracle.dequantize(ref, "f64"))
    assert oracle.gemm_error(c, cref) <= GEMM_TOL


# ------------------------------------------------------------------------------------------------
# per-matrix quality statistics
# ------------------------------------------------------------------------------------------------
# Both sides sum in double, in different orders; the oracle's sequential sums over n <= 6e7 terms
# carry a relative error below n * 2^-53 < 1e-8, the kernel's tree sums far less.  The moments
# behind the kurtosis are formed about the first element on the GPU and about the mean in the
# oracle; for the inputs here the extra cancellation is a few units in the last place.  Maximum
# and block count are exact; the ratio of a constant block is left out on both sides exactly.
STAT_RTOL = 1e-8


def _dev_q(nv, ref):
    return nv.NVFP4Tensor(to_dev_u8(ref.codes), to_dev_u8(ref.scales),
                          torch.tensor([ref.g], dtype=torch.float32, device=DEV))


def _assert_stats(got, ref, what=""):
    for k in ("max_abs", "blocks"):
        assert got[k] == ref[k] or (math.isnan(got[k]) and math.isnan(ref[k])), f"{what} {k} {got[k]} vs {ref[k]}"
    for k in ("rel_error", "block_max_over_std", "std"):
        a, b = got[k], ref[k]
        if math.isnan(b):
            assert math.isnan(a), f"{what} {k} {a} vs NaN"
        else:
            assert abs(a - b) <= STAT_RTOL * abs(b), f"{what} {k} {a!r} vs {b!r}"
    a, b = got["kurtosis"] + 3.0, ref["kurtosis"] + 3.0
    if math.isnan(b):
        assert math.isnan(a), f"{what} kurtosis {a} vs NaN"
    else:
        assert abs(a - b) <= STAT_RTOL * abs(b), f"{what} kurtosis {got['kurtosis']!r} vs {ref['kurtosis']!r}"
    scale = abs(ref["mean"]) + ref["std"]
    assert abs(got["mean"] - ref["mean"]) <= STAT_RTOL * scale, f"{what} mean {got['mean']!r} vs {ref['mean']!r}"


def _stats_case(nv, x, dtype, with_q=True, pad=0):
    """x: fp32 values; returns (device tensor in dtype, oracle source array, oracle dtype code)."""
    if dtype == "f32":
        src, code, dev = x, oracle.F32, to_dev_f32(x)
    elif dtype == "bf16":
        src = synth.bf16_bits(x)
        code, dev = oracle.BF16, to_dev_bf16(src)
    else:
        src = x.astype(np.float16).view(np.uint16)
        code, dev = oracle.F16, to_dev_f16(src)
    if pad:
        dev = padded(dev, pad)
    ref_q = oracle.quantize(src, code)[0] if with_q else None
    ref = oracle.matrix_stats(src, ref_q, code)
    got = nv.matrix_stats(dev, _dev_q(nv, ref_q) if with_q else None)
    return got, ref


@pytest.mark.parametrize("shape", [(1, 16), (3, 48), (65, 1040), (300, 272), (129, 2048), (1000, 3072)])
@pytest.mark.parametrize("dtype", ["f32", "bf16", "f16"])
def test_matrix_stats_shapes_dtypes(nv, shape, dtype):
    _note(f"matrix stats {dtype} {shape}")
    g = synth.rng(shape[0] * 7 + shape[1])
    x = (g.standard_t(4, size=shape) * 0.02).astype(np.float32)
    got, ref = _stats_case(nv, x, dtype)
    _assert_stats(got, ref, f"{dtype} {shape}")
    got, ref = _stats_case(nv, x, dtype, with_q=False, pad=16)
    assert math.isnan(got["rel_error"]) and math.isnan(ref["rel_error"])
    _assert_stats(got, ref, f"{dtype} {shape} no q, strided")


def test_matrix_stats_offset_constant_blocks_and_degenerate(nv):
    _note("matrix stats: offset mean, constant blocks, constant matrix")
    g = synth.rng(77)
    # mean far from 0 relative to the spread (a norm-gain-like vector), and zero rows
    x = (1.0 + 0.01 * g.standard_normal((257, 320))).astype(np.float32)
    x[5] = 0.0
    x[100:103] = 0.25
    for dt in ("f32", "bf16"):
        got, ref = _stats_case(nv, x, dt)
        assert ref["blocks"] < 257 * 320 / 64
        _assert_stats(got, ref, f"offset {dt}")
    # a matrix whose first element is an outlier: the shift is far from the mean
    y = (g.standard_normal((64, 512)) * 0.02).astype(np.float32)
    y[0, 0] = 40.0
    got, ref = _stats_case(nv, y, "f32")
    _assert_stats(got, ref, "outlier first")
    # constant matrix: no block counts, the moments are 0/0
    z = np.full((8, 64), 0.5, dtype=np.float32)
    got, ref = _stats_case(nv, z, "f32")
    assert got["blocks"] == 0 and math.isnan(got["block_max_over_std"]) and math.isnan(got["kurtosis"])
    _assert_stats(got, ref, "constant")
    assert got["mean"] == 0.5 and got["std"] == 0.0


def test_matrix_stats_full_sizes(nv):
    _note("matrix stats: 18432x3072 bf16 modulation weight, 3072x3072 fp32 attention weight")
    w = synth.modulation_weight()
    got, ref = _stats_case(nv, w, "bf16")
    _assert_stats(got, ref, "modulation bf16")
    w = synth.attn_proj_weight()
    got, ref = _stats_case(nv, w, "f32")
    _assert_stats(got, ref, "attention f32")


# ------------------------------------------------------------------------------------------------
# NVFP4 GEMM with a bf16 low-rank branch: C = A_hat . W_hat^T + (A . V^T) . U^T
# ------------------------------------------------------------------------------------------------
def _lowrank_operands(m, n, k, r, seed):
    g = synth.rng(seed)
    a_bits = synth.bf16_bits(g.standard_normal((m, k)).astype(np.float32))
    v_bits = synth.bf16_bits((g.standard_normal((r, k)) * 0.05).astype(np.float32))
    u_bits = synth.bf16_bits((g.standard_normal((n, r)) * 0.05).astype(np.float32))
    return a_bits, v_bits, u_bits


# paths: fused epilogue of the tiled kernel (K % 64 == 0, unsplit), the GEMV for M <= 4, the
# K % 64 != 0 kernel and split-K (the last three add the branch in a second pass); ranks 16 .. 256
# including r % 32 == 16 and r > 128 (two column blocks of T)
LOWRANK_SHAPES = [(16, 64, 256, 16), (1, 64, 128, 32), (3, 100, 4096, 128), (64, 96, 112, 48),
                  (200, 300, 512, 128), (130, 1000, 128, 64), (256, 192, 1024, 256), (100, 1000, 4096, 128),
                  (300, 520, 640, 144), (7, 300, 3072, 128)]


@pytest.mark.parametrize("mnkr", LOWRANK_SHAPES)
@pytest.mark.parametrize("form", ["w4a16", "w4a4"])
def test_gemm_lowrank(nv, mnkr, form):
    m, n, k, r = mnkr
    _note(f"gemm lowrank {form} {mnkr}")
    q, ref = _rand_q(nv, n, k, seed=m * 13 + n + r)
    a_bits, v_bits, u_bits = _lowrank_operands(m, n, k, r, seed=m + k + r)
    a, v, u = to_dev_bf16(a_bits), to_dev_bf16(v_bits), to_dev_bf16(u_bits)
    aq = aref = None
    if form == "w4a4":
        aq = _quant(nv, a)
        aref, _ = oracle.quantize(a_bits, oracle.BF16)
        _assert_q_equal(aq, aref, "activations")
    c = nv.gemm_lowrank(a, q, v, u, a_q=aq).cpu().numpy()
    cref = oracle.gemm_lowrank(a_bits, ref, v_bits, u_bits, a_q=aref)
    err = oracle.gemm_error(c, cref)
    assert err <= GEMM_TOL, err
    if m > 1:  # strided A and C, and a workspace that holds T only (the product runs unsplit)
        t_bytes = (m * 1024 + 255) // 256 * 256
        ws = torch.empty(t_bytes, dtype=torch.uint8, device=DEV)
        out = padded(torch.empty((m, n), dtype=torch.float32, device=DEV), 4)
        nv.gemm_lowrank(padded(a, 8), q, v, u, a_q=aq, out=out, workspace=ws)
        err2 = oracle.gemm_error(out.cpu().numpy(), cref)
        assert err2 <= GEMM_TOL, err2


def test_gemm_lowrank_zero_branch_is_plain_product(nv):
    _note("gemm lowrank: zero branch, one-hot branch")
    m, n, k, r = 300, 200, 1024, 128
    q, ref = _rand_q(nv, n, k, seed=5)
    a_bits, v_bits, u_bits = _lowrank_operands(m, n, k, r, seed=6)
    a, v = to_dev_bf16(a_bits), to_dev_bf16(v_bits)
    zu = torch.zeros((n, r), dtype=torch.bfloat16, device=DEV)
    assert np.array_equal(nv.gemm_lowrank(a, q, v, zu).cpu().numpy(), nv.gemm(a, q).cpu().numpy())
    # one-hot branch: V = e_k (row 0), U = e_0 for output column 7: adds A[:, 3] to column 7 exactly
    v1 = np.zeros((r, k), np.uint16)
    v1[0, 3] = 0x3F80
    u1 = np.zeros((n, r), np.uint16)
    u1[7, 0] = 0x3F80
    d = nv.gemm_lowrank(a, q, to_dev_bf16(v1), to_dev_bf16(u1)).cpu().numpy() - nv.gemm(a, q).cpu().numpy()
    want = np.zeros((m, n))
    want[:, 7] = oracle.bf16_bits_to_f64(a_bits)[:, 3]
    assert np.allclose(d, want, rtol=1e-6, atol=1e-6 * np.abs(nv.gemm(a, q).cpu().numpy()).max())


def test_gemm_lowrank_attention_projection_full(nv):
    m, n, k, r = 4096, 3072, 3072, 128
    _note(f"gemm lowrank w4a16 {m}x{n}x{k} rank {r} (full)")
    w = synth.attn_proj_weight()
    a_bits = synth.attn_proj_activations()
    ref, _ = oracle.quantize(w)
    q = _quant(nv, to_dev_f32(w))
    _assert_q_equal(q, ref, "attn weight")
    _, v_bits, u_bits = _lowrank_operands(8, n, k, r, seed=2024)
    c = nv.gemm_lowrank(to_dev_bf16(a_bits), q, to_dev_bf16(v_bits), to_dev_bf16(u_bits)).cpu().numpy()
    err = oracle.gemm_error(c, oracle.gemm_lowrank(a_bits, ref, v_bits, u_bits))
    _note(f"  floored max rel err {err:.3e}")
    assert err <= GEMM_TOL


# ------------------------------------------------------------------------------------------------
# W4A4 with the activation quantization inside the GEMM (static amax)
# ------------------------------------------------------------------------------------------------
# With its full workspace the call runs the staged form wherever the W4A4 product's workgroups fit
# in one round (every shape below but M <= 4 and K % 64 != 0, where A is quantized into the
# workspace first): both are bit-identical to the separate static-amax quantize + W4A4 product.
# The reference quantizes A with the same static amax in the oracle and contracts the exact
# operands in float64.
QA_SHAPES = [(16, 64, 256), (2, 300, 1024), (64, 96, 112), (200, 300, 512), (100, 500, 4096), (2048, 384, 3072),
             (130, 1000, 128), (100, 1000, 4096), (512, 12288, 4096), (300, 520, 640), (8, 300, 3072),
             (512, 4096, 12288), (4096, 3072, 3072)]


def _qa_case(nv, m, n, k):
    q, ref = _rand_q(nv, n, k, seed=m * 11 + n, sigma=0.015)
    a_bits = synth.bf16_bits(np.random.default_rng(m * 5 + k).standard_normal((m, k)).astype(np.float32))
    amax = np.float32(0.8 * np.abs(oracle.bf16_bits_to_f64(a_bits)).max())  # static amax below max: clipping
    return q, ref, a_bits, amax


@pytest.mark.parametrize("mnk", QA_SHAPES)
def test_gemm_qa(nv, mnk):
    m, n, k = mnk
    _note(f"gemm qa (static amax) {mnk}")
    q, ref, a_bits, amax = _qa_case(nv, m, n, k)
    amax_d = torch.tensor([amax], dtype=torch.float32, device=DEV)
    a = to_dev_bf16(a_bits)
    c = nv.gemm_qa(a, q, amax_d).cpu().numpy()
    # the separate static-amax quantize and the W4A4 product: the same bits
    c_two = nv.gemm(_quant(nv, a, amax=amax_d), q).cpu().numpy()
    assert np.array_equal(c.view(np.uint32), c_two.view(np.uint32))
    rows = np.arange(m) if m * n * k <= 2 ** 31 else np.random.default_rng(m).choice(m, 128, replace=False)
    aref, _ = oracle.quantize(a_bits[rows] if len(rows) < m else a_bits, oracle.BF16, amax=float(amax))
    err = oracle.gemm_error(c[rows], oracle.gemm_w4a4(aref, ref))
    assert err <= GEMM_TOL, err
    if m > 1 and len(rows) == m:  # strided A and C
        out = padded(torch.empty((m, n), dtype=torch.float32, device=DEV), 4)
        nv.gemm_qa(padded(a, 8), q, amax_d, out=out)
        assert np.array_equal(out.cpu().numpy().view(np.uint32), c.view(np.uint32))


def _gemm_qa_raw(nv, a, w, amax, out, ws):
    # the C entry point with an explicit workspace (None: NULL, which leaves the staged form out)
    import ctypes
    wct = w.c()
    st = nv.lib.nvfp4_gemm_qa(a.data_ptr(), amax.data_ptr(), a.shape[0], a.stride(0), ctypes.byref(wct),
                              out.data_ptr(), out.stride(0), ws.data_ptr() if ws is not None else None,
                              ws.numel() if ws is not None else 0, nv._stream(a.device))
    assert st == 0, st
    return out


@pytest.mark.parametrize("mnk", [(200, 300, 512), (2048, 384, 3072), (300, 512, 640), (100, 500, 4096)])
def test_gemm_qa_fused_form(nv, mnk):
    # without a workspace (N <= 512, K % 64 == 0) the fused kernel quantizes A in its staging path:
    # the same operand values, another tile shape and summation order
    m, n, k = mnk
    _note(f"gemm qa fused form {mnk}")
    q, ref, a_bits, amax = _qa_case(nv, m, n, k)
    amax_d = torch.tensor([amax], dtype=torch.float32, device=DEV)
    a = to_dev_bf16(a_bits)
    c = _gemm_qa_raw(nv, a, q, amax_d, torch.empty((m, n), dtype=torch.float32, device=DEV), None)
    torch.cuda.synchronize()
    aref, _ = oracle.quantize(a_bits, oracle.BF16, amax=float(amax))
    assert oracle.gemm_error(c.cpu().numpy(), oracle.gemm_w4a4(aref, ref)) <= GEMM_TOL
    assert oracle.gemm_error(c.cpu().numpy(), nv.gemm_qa(a, q, amax_d).cpu().numpy()) <= 1e-5


def test_gemm_qa_staged_workspace_reuse_and_fallback(nv, monkeypatch):
    # one zeroed workspace for products of different group structures (row blocks, K slices, N
    # tiles): each call leaves the group counters zero.  Then with the wait bound at zero polls every
    # workgroup that finds its group incomplete quantizes its whole region itself: same bits.
    shapes = [(512, 12288, 4096), (100, 1000, 4096), (2048, 384, 3072), (512, 4096, 12288), (130, 1000, 128)]
    ws = torch.zeros(max(nv.workspace_size(nv.OP_GEMM_QA, *s) for s in shapes), dtype=torch.uint8, device=DEV)
    for spin in (None, "0"):
        if spin is not None:
            monkeypatch.setenv("NVFP4_QA_SPIN_LIMIT", spin)
        for m, n, k in shapes:
            _note(f"gemm qa staged {m}x{n}x{k}, wait bound {spin}")
            q, _, a_bits, amax = _qa_case(nv, m, n, k)
            amax_d = torch.tensor([amax], dtype=torch.float32, device=DEV)
            a = to_dev_bf16(a_bits)
            c = nv.gemm_qa(a, q, amax_d, workspace=ws)
            c_two = nv.gemm(_quant(nv, a, amax=amax_d), q)
            assert torch.equal(c.view(torch.int32), c_two.view(torch.int32)), (m, n, k, spin)
            assert not ws[:4096].any().item(), "group counters left non-zero"


def test_gemm_qa_exact_cases(nv):
    _note("gemm qa: one-hot rows, amax 0, values equal to the separate quantize")
    n, k = 192, 320
    q, ref = _rand_q(nv, n, k, seed=17)
    # one-hot rows with amax 1 (the quantized activations are 6 x 448 x g = 2688 fl(1/2688), one
    # ulp from 1): each output is one product, so it matches the float64 reference to the two fp32
    # roundings of the scale factors (K = 336: the unfused form; K = 256: fused)
    for kk in (336, 256):
        qk, refk = _rand_q(nv, n, kk, seed=18 + kk)
        eye = np.zeros((kk, kk), np.float32)
        eye[np.arange(kk), np.arange(kk)] = 1.0
        eb = synth.bf16_bits(eye)
        one = torch.tensor([1.0], dtype=torch.float32, device=DEV)
        c = nv.gemm_qa(to_dev_bf16(eb), qk, one).cpu().numpy()
        aref, _ = oracle.quantize(eb, oracle.BF16, amax=1.0)
        assert np.max(np.abs(oracle.dequantize(aref, "f64") - np.eye(kk))) <= 2.0 ** -24
        cref = oracle.gemm_w4a4(aref, refk)
        assert np.all(np.abs(c - cref) <= 2.5e-7 * np.abs(cref)), kk
    # amax 0: every code is 0, C = 0
    a_bits = synth.bf16_bits(np.random.default_rng(3).standard_normal((64, k)).astype(np.float32))
    zero = torch.zeros(1, dtype=torch.float32, device=DEV)
    assert not nv.gemm_qa(to_dev_bf16(a_bits), q, zero).cpu().numpy().any()
    # the fused form (N = 512) against the separate quantize + W4A4 product on the GPU (same operand
    # values, different summation order): within the fp32 accumulation error
    k2 = 1024
    q2, _ = _rand_q(nv, 512, k2, seed=19)
    a2 = synth.bf16_bits(np.random.default_rng(4).standard_normal((300, k2)).astype(np.float32))
    amax = torch.tensor([2.5], dtype=torch.float32, device=DEV)
    c_fused = nv.gemm_qa(to_dev_bf16(a2), q2, amax).cpu().numpy()
    aq = _quant(nv, to_dev_bf16(a2), amax=amax)
    c_two = nv.gemm(aq, q2).cpu().numpy()
    assert oracle.gemm_error(c_fused, c_two) <= 1e-5


def test_gemm_qa_attention_projection_full(nv):
    _note("gemm qa 4096x3072x3072 (full), static amax = p99.9 of |A| per channel, max over channels")
    w = synth.attn_proj_weight()
    a_bits = synth.attn_proj_activations()
    ref, _ = oracle.quantize(w)
    q = _quant(nv, to_dev_f32(w))
    _assert_q_equal(q, ref, "attn weight")
    pct, _ = nv.amax_percentile(to_dev_bf16(a_bits), 99.9, per_channel=True)
    amax = pct.max().reshape(1)
    aref, _ = oracle.quantize(a_bits, oracle.BF16, amax=float(amax.item()))
    rows = np.random.default_rng(2).choice(4096, 256, replace=False)
    c = nv.gemm_qa(to_dev_bf16(a_bits), q, amax).cpu().numpy()[rows]
    cref = oracle.gemm_f64(oracle.dequantize(aref, "f64")[rows], oracle.dequantize(ref, "f64"))
    err = oracle.gemm_error(c, cref)
    _note(f"  floored max rel err {err:.3e}")
    assert err <= GEMM_TOL


def test_gemm_lowrank_and_qa_empty(nv):
    _note("gemm lowrank / qa: M = 0 and K = 0")
    import bit_gemm_nvfp4_amd as nvm
    q, _ = _rand_q(nv, 40, 64, seed=1)
    v = torch.zeros((16, 64), dtype=torch.bfloat16, device=DEV)
    u = torch.zeros((40, 16), dtype=torch.bfloat16, device=DEV)
    a0 = torch.zeros((0, 64), dtype=torch.bfloat16, device=DEV)
    assert nv.gemm_lowrank(a0, q, v, u).shape == (0, 40)
    amax = torch.ones(1, dtype=torch.float32, device=DEV)
    assert nv.gemm_qa(a0, q, amax).shape == (0, 40)
    # K = 0: C = 0
    w0 = nvm.NVFP4Tensor(torch.zeros((5, 0), dtype=torch.uint8, device=DEV),
                         torch.zeros((5, 0), dtype=torch.uint8, device=DEV), torch.ones(1, device=DEV))
    a = torch.zeros((3, 0), dtype=torch.bfloat16, device=DEV)
    out = torch.full((3, 5), 7.0, device=DEV)
    nv.gemm_lowrank(a, w0, torch.zeros((16, 0), dtype=torch.bfloat16, device=DEV),
                    torch.zeros((5, 16), dtype=torch.bfloat16, device=DEV), out=out)
    assert not out.cpu().numpy().any()
    out.fill_(7.0)
    nv.gemm_qa(a, w0, amax, out=out)
    assert not out.cpu().numpy().any()
