"""GPU parity of nvfp4_quantize_batch: several tensors quantized in one call, each with its own
run-time amax, against the CPU oracle bit for bit (codes, scale bytes, global scale).  Covers every
source dtype, ragged and row-strided tensors, the four 3072 x 3072 FP8 weights of one block of the
layer stack, a batch too large to stay on chip together (one launch per tensor instead), workspace
reuse across batched and single calls, the non-finite flag, and HIP graph replay."""
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


def _assert_q_equal(q, ref, what=""):
    codes = q.codes.cpu().numpy()
    scales = q.scales.cpu().numpy()
    g = q.global_scale.cpu().numpy()[0]
    assert g.view(np.uint32) == np.float32(ref.g).view(np.uint32), f"{what} global scale {g} vs {ref.g}"
    assert np.array_equal(scales, ref.scales), f"{what}: {int((scales != ref.scales).sum())} scale bytes differ"
    assert np.array_equal(codes, ref.codes), f"{what}: {int((codes != ref.codes).sum())} code bytes differ"


SHAPES = [(64, 256), (1, 16), (333, 1040), (1000, 3072), (7, 48)]


def _inputs(dtype, shapes, seed):
    """(device tensors, oracle references) for one batch; tensor 2 is stored with a wider row stride."""
    xs, refs, scs = [], [], []
    for i, (r, c) in enumerate(shapes):
        x = synth.normal_f32((r, c), 0.02 * (i + 1), seed + i)
        x[r // 2, c // 3] = 0.5 * (i + 1)  # each tensor its own amax
        if dtype == "f32":
            d, ref, sc = to_dev_f32(x), oracle.quantize(x)[0], None
        elif dtype == "bf16":
            b = synth.bf16_bits(x)
            d, ref, sc = to_dev_bf16(b), oracle.quantize(b, oracle.BF16)[0], None
        elif dtype == "f16":
            h = x.astype(np.float16).view(np.uint16)
            d, ref, sc = to_dev_f16(h), oracle.quantize(h, oracle.F16)[0], None
        else:
            b, s = synth.fp8_tensorwise(x)
            if i == 1:  # one tensor without a source scale (1.0)
                d, ref, sc = to_dev_u8(b), oracle.quantize(b, oracle.E4M3, None)[0], None
            else:
                d = to_dev_u8(b)
                ref = oracle.quantize(b, oracle.E4M3, float(s))[0]
                sc = torch.tensor([s], dtype=torch.float32, device=DEV)
        if i == 2:
            d = padded(d, 32)
        xs.append(d)
        refs.append(ref)
        scs.append(sc)
    return xs, refs, scs


@pytest.mark.parametrize("dtype", ["f32", "bf16", "f16", "e4m3"])
def test_quantize_batch_dtypes_shapes(nv, dtype):
    _note(f"quantize_batch {dtype} {SHAPES}")
    xs, refs, scs = _inputs(dtype, SHAPES, 900)
    outs = nv.quantize_batch(xs, src_scales=scs if dtype == "e4m3" else None, check=True)
    for i, (q, ref) in enumerate(zip(outs, refs)):
        _assert_q_equal(q, ref, f"{dtype} tensor {i} {SHAPES[i]}")


def test_quantize_batch_single_and_eight(nv):
    _note("quantize_batch with one tensor and with eight")
    for shapes in ([(513, 272)], [(16 * (i + 1), 64 * (i + 1)) for i in range(8)]):
        xs, refs, _ = _inputs("f32", shapes, 950)
        outs = nv.quantize_batch(xs, check=True)
        for i, (q, ref) in enumerate(zip(outs, refs)):
            _assert_q_equal(q, ref, f"{len(shapes)} tensors, tensor {i}")


def test_quantize_batch_stack_block_fp8(nv):
    # the four 3072 x 3072 FP8 projection weights of one block of the layer stack, in one launch
    _note("quantize_batch: the four 3072x3072 FP8 weights of block 11")
    srcs = [synth.stack_weight_fp8(11, j) for j in range(4)]
    xs = [to_dev_u8(b) for b, _ in srcs]
    scs = [torch.tensor([s], dtype=torch.float32, device=DEV) for _, s in srcs]
    outs = nv.quantize_batch(xs, src_scales=scs, check=True)
    for j, ((b, s), q) in enumerate(zip(srcs, outs)):
        _assert_q_equal(q, oracle.quantize(b, oracle.E4M3, float(s))[0], f"block 11 weight {j}")


def test_quantize_batch_beyond_residency(nv):
    # two bf16 tensors of 4096 x 3072 hold more tiles than the batch keeps in registers: the call
    # quantizes them one launch each, with the same results
    _note("quantize_batch beyond the on-chip residency (one launch per tensor)")
    xs, refs, _ = _inputs("bf16", [(4096, 3072), (4096, 3072)], 970)
    outs = nv.quantize_batch(xs, check=True)
    for i, (q, ref) in enumerate(zip(outs, refs)):
        _assert_q_equal(q, ref, f"tensor {i}")


def test_quantize_batch_workspace_reuse_and_flags(nv):
    _note("quantize_batch: workspace shared with single calls, non-finite flag")
    ws = nv.quantize_workspace(DEV)
    for rep in range(3):
        xs, refs, _ = _inputs("f32", SHAPES, 1000 + 10 * rep)
        outs = nv.quantize_batch(xs, workspace=ws, check=True)
        for i, (q, ref) in enumerate(zip(outs, refs)):
            _assert_q_equal(q, ref, f"rep {rep} tensor {i}")
        x1 = synth.normal_f32((100, 64), 1.0, 1100 + rep)
        _assert_q_equal(nv.quantize(to_dev_f32(x1), workspace=ws, check=True), oracle.quantize(x1)[0], f"single {rep}")
    xs, _, _ = _inputs("f32", SHAPES[:3], 1200)
    xs[1][0, 3] = float("nan")
    flags = torch.zeros(1, dtype=torch.int32, device=DEV)
    nv.quantize_batch(xs, flags=flags, workspace=ws)
    assert int(flags.item()) & 1
    # the workspace is still good for the next call
    xs, refs, _ = _inputs("f32", SHAPES, 1300)
    for i, (q, ref) in enumerate(zip(nv.quantize_batch(xs, workspace=ws, check=True), refs)):
        _assert_q_equal(q, ref, f"after flags, tensor {i}")


def test_quantize_batch_replayed_from_hip_graph(nv):
    # one batched call captured in a HIP graph and replayed on new inputs (amax changing by 10x):
    # each replay's grid agreement is told apart through the workspace, as for single calls
    shapes = [(256, 1024), (64, 3072), (1000, 512)]
    _note(f"quantize_batch replayed from a HIP graph {shapes}")
    xs = [torch.zeros(s, dtype=torch.float32, device=DEV) for s in shapes]
    outs = [nv.NVFP4Tensor.empty(r, c, DEV) for r, c in shapes]
    ws = nv.quantize_workspace(DEV)
    flags = torch.zeros(1, dtype=torch.int32, device=DEV)
    nv.quantize_batch(xs, outs=outs, workspace=ws, flags=flags)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        nv.quantize_batch(xs, outs=outs, workspace=ws, flags=flags)
    for rep in range(4):
        host = []
        for i, (r, c) in enumerate(shapes):
            xi = (np.random.default_rng(1400 + 10 * rep + i).standard_normal((r, c)) * 10.0 ** (rep - i)).astype(np.float32)
            xs[i].copy_(torch.from_numpy(xi))
            host.append(xi)
        flags.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert int(flags.item()) == 0, f"replay {rep}"
        for i, xi in enumerate(host):
            _assert_q_equal(outs[i], oracle.quantize(xi)[0], f"replay {rep} tensor {i}")
