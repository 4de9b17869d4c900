"""GPU parity at the rounding edges of the format ("Qwen-Image NVFP4 on a 16 GB Ada GPU", section
"What NVFP4 is and how it differs from NF4": E2M1 magnitudes 0..6, one E4M3 scale per 16 elements,
an fp32 global scale; "Qwen3-VL-8B-Instruct-heretic-NVFP4", "Quantization Details": the e4m3fn
tensorwise quantizer).

Random data reaches the ties of the two roundings only by chance, so these inputs are built to sit
on them.  With a static amax of 2688 * 2^-j the global scale is exactly g = 2^-j; a block whose
largest magnitude is 6 * 2^-j then has t = 1, scale byte 0x38 (1.0), d = 2^-j and reciprocal 2^j,
so every element reaches the E2M1 rounding as y = |v| * 2^j with no other rounding on the way.
Likewise a block maximum of 6 m * 2^-j puts t exactly on m, so m on each E4M3 midpoint exercises the
block-scale rounding's ties; and a static FP8 amax of 448 gives the tensor scale 1, so each quotient
is the input itself.  Every result is compared bit for bit with the oracle.
"""
import sys

import numpy as np
import pytest
import torch

import oracle
from gpu_util import DEV, to_dev_f32

pytestmark = pytest.mark.gpu

E2M1_GRID = np.array([0, 0.5, 1, 1.5, 2, 3, 4, 6], dtype=np.float32)
E2M1_MID = np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0], dtype=np.float32)


@pytest.fixture(scope="module")
def nv():
    import bit_gemm_nvfp4_amd as m
    return m


def _note(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def _neighbours(points: np.ndarray, k: int) -> np.ndarray:
    """Each fp32 point and its k nearest representable neighbours on either side (non-negative)."""
    u = np.ascontiguousarray(points, dtype=np.float32).view(np.int32).astype(np.int64)
    offs = np.arange(-k, k + 1, dtype=np.int64)
    v = (u[:, None] + offs[None, :]).ravel()
    v = v[v >= 0]
    return np.unique(v.astype(np.uint32)).view(np.float32)


def _blocks_with_max(vals: np.ndarray, head: float, sign_seed: int) -> np.ndarray:
    """Rows of 16: element 0 is `head` (fixing the block maximum), elements 1..15 carry `vals`
    (padded with zeros) with pseudo-random signs."""
    n = -(-vals.size // 15)
    body = np.zeros(n * 15, dtype=np.float32)
    body[:vals.size] = vals
    sign = (np.random.default_rng(sign_seed).integers(0, 2, body.size, dtype=np.uint32) << 31)
    body = (body.view(np.uint32) | sign).view(np.float32).reshape(n, 15)
    return np.concatenate([np.full((n, 1), head, dtype=np.float32), body], axis=1)


def _unpack(codes: np.ndarray) -> np.ndarray:
    c = codes.reshape(codes.shape[0], -1)
    out = np.empty((c.shape[0], c.shape[1] * 2), dtype=np.uint8)
    out[:, 0::2] = c & 0xF
    out[:, 1::2] = c >> 4
    return out


def _quant_static(nv, x: np.ndarray, amax: float):
    flags = torch.zeros(1, dtype=torch.int32, device=DEV)
    q = nv.quantize(to_dev_f32(x), amax=torch.tensor([amax], dtype=torch.float32, device=DEV), flags=flags)
    torch.cuda.synchronize()
    assert int(flags.item()) == 0
    return q


def _assert_same_as_oracle(nv, x, amax, what):
    q = _quant_static(nv, x, amax)
    ref, _ = oracle.quantize(x, amax=amax)
    assert q.global_scale.item() == float(ref.g), what
    s = q.scales.cpu().numpy()
    assert np.array_equal(s, ref.scales), f"{what}: {(s != ref.scales).sum()} scale bytes differ"
    c = q.codes.cpu().numpy()
    bad = np.nonzero(c != ref.codes)
    assert bad[0].size == 0, (f"{what}: {bad[0].size} code bytes differ; first at {bad[0][0]},{bad[1][0]}: "
                              f"{c[bad[0][0], bad[1][0]]:#04x} vs {ref.codes[bad[0][0], bad[1][0]]:#04x}")
    return q


E2M1_SWEEP_END = 0x40C00000 + 1  # every fp32 pattern from +0 to 6.0 inclusive
E2M1_SWEEP_CHUNK = 15 << 22       # 4M blocks of 16 per launch
E2M1_SWEEP_PARTS = 3


@pytest.mark.parametrize("part", range(E2M1_SWEEP_PARTS))
def test_e2m1_every_fp32_value_in_0_to_6(nv, part):
    """Exhaustive over the parts together: every fp32 bit pattern from 0 to 6.0 inclusive
    (1 086 324 737 values) through the element encode at g = 1, s = 1 (so y = |v|), against the
    oracle's nearest-E2M1 rounding (ties to the even code), with the sign bit of v."""
    n_total = E2M1_SWEEP_END
    starts = list(range(0, n_total, E2M1_SWEEP_CHUNK))
    per_part = -(-len(starts) // E2M1_SWEEP_PARTS)
    per_chunk = E2M1_SWEEP_CHUNK
    for c0 in starts[part * per_part:(part + 1) * per_part]:
        c1 = min(n_total, c0 + per_chunk)
        _note(f"e2m1 sweep {c0:#010x}..{c1:#010x}")
        vals = np.arange(c0, c1, dtype=np.uint32).view(np.float32)
        x = _blocks_with_max(vals, 6.0, c0).reshape(-1, 4096 if (vals.size // 15) % 256 == 0 else 16)
        q = _quant_static(nv, x, 2688.0)
        assert q.global_scale.item() == 1.0
        assert np.all(q.scales.cpu().numpy() == 0x38)
        got = _unpack(q.codes.cpu().numpy()).reshape(-1, 16)
        xb = x.reshape(-1, 16)
        want = oracle.e2m1_index_array(np.abs(xb)) | (np.signbit(xb).astype(np.uint8) << 3)
        bad = np.nonzero(got != want)
        assert bad[0].size == 0, (f"{bad[0].size} codes differ; first y = {abs(xb[bad][0])!r} "
                                  f"({np.float32(abs(xb[bad][0])).view(np.uint32):#010x}): "
                                  f"{got[bad][0]} vs {want[bad][0]}")
    if part == 0:
        # the full oracle agrees with the rounding table used above on a slice of the same inputs
        vals = np.arange(0x3E000000, 0x3E000000 + 15 * 4096, dtype=np.uint32).view(np.float32)
        _assert_same_as_oracle(nv, _blocks_with_max(vals, 6.0, 1).reshape(-1, 256), 2688.0, "oracle slice")


def test_e2m1_saturation_above_six(nv):
    """Blocks whose maximum lies in (6, 6.375]: t = bamax / 6 <= 1.0625 rounds to the scale 1.0
    (1.0625 is the tie between 1 and 1.125, and goes to the even mantissa), so y = |v| exceeds 6
    and must saturate to 6.  Every fp32 value of the range, in blocks of 16."""
    lo, hi = np.float32(6.0).view(np.uint32) + 1, np.float32(6.375).view(np.uint32)
    v = np.arange(lo, hi + 1, dtype=np.uint32).view(np.float32)
    v = v[: v.size // 16 * 16].reshape(-1, 16)
    x = v * np.where(np.random.default_rng(3).integers(0, 2, v.shape) == 1, -1, 1).astype(np.float32)
    q = _assert_same_as_oracle(nv, x.reshape(-1, 256), 2688.0, "above 6")
    assert np.all(q.scales.cpu().numpy() == 0x38)
    assert np.all((_unpack(q.codes.cpu().numpy()) & 7) == 7)


@pytest.mark.parametrize("j", [0, 7, -7, 40, -40, 100])
def test_e2m1_midpoints_at_power_of_two_scales(nv, j):
    """Every E2M1 midpoint and grid point with 64 neighbours either side, plus zeros, -0, fp32
    subnormals and a strided sweep of [0, 6], at g = 2^-j (static amax 2688 * 2^-j)."""
    pts = _neighbours(np.concatenate([E2M1_MID, E2M1_GRID[1:]]), 64)
    sweep = np.arange(0, 0x40C00000, 4093, dtype=np.uint32).view(np.float32)
    vals = np.concatenate([pts, sweep, np.array([0.0, 1e-45, 1e-40, 1.1754942e-38], dtype=np.float32)])
    scale = np.float32(2.0 ** -j)
    x = _blocks_with_max(vals, 6.0, 211 + j) * scale
    x[0, 5], x[1, 7] = -0.0, np.float32(-1e-45)
    _note(f"e2m1 midpoints, g = 2^{-j}, {x.size} elements")
    x = np.concatenate([x, np.zeros((-x.shape[0] % 16, 16), np.float32)]).reshape(-1, 256)
    q = _assert_same_as_oracle(nv, x, float(np.float32(2688.0) * scale), f"j={j}")
    assert q.global_scale.item() == float(scale)


def _e4m3_midpoints() -> np.ndarray:
    vals = np.array([oracle.e4m3_value(b) for b in range(0x7F)], dtype=np.float64)
    mids = (vals[:-1] + vals[1:]) / 2  # exact: neighbours share or border an exponent
    return np.concatenate([mids, [464.0]]).astype(np.float32)  # 464: between 448 and the next (480)


@pytest.mark.parametrize("j", [0, 20, -20])
def test_e4m3_block_scale_ties(nv, j):
    """Block maxima 6 m 2^-j with m on every E4M3 midpoint (subnormal and normal steps, and the
    saturation boundary 464) and 3 fp32 neighbours either side, at g = 2^-j: t = fl(bamax / 6g) lands
    on m exactly (6 m has at most 7 significant bits), so the block-scale rounding meets its ties;
    the other 15 elements of each block are spread below the maximum."""
    scale = np.float32(2.0 ** -j)
    t = _neighbours(_e4m3_midpoints(), 3)
    t = t[t > 0]
    heads = (np.float32(6.0) * t).astype(np.float32) * scale
    rng = np.random.default_rng(40 + j)
    frac = rng.uniform(0, 1, (heads.size, 15)).astype(np.float32)
    body = (heads[:, None] * frac).astype(np.float32)
    sign = np.where(rng.integers(0, 2, body.shape) == 1, -1, 1).astype(np.float32)
    x = np.concatenate([heads[:, None], body * sign], axis=1)
    x = np.concatenate([x, np.zeros((-x.shape[0] % 16, 16), np.float32)]).reshape(-1, 256)
    _note(f"e4m3 block-scale ties, g = 2^{-j}, {heads.size} blocks")
    q = _assert_same_as_oracle(nv, x, float(np.float32(2688.0) * scale), f"j={j}")
    # the ties themselves went to the even mantissa (checked independently of the oracle)
    s = q.scales.cpu().numpy().reshape(-1)[: heads.size]
    on_mid = np.isin(t, _e4m3_midpoints())
    assert np.all(s[on_mid & (t < 448)] % 2 == 0)
    assert np.all(s[t >= 448] == 0x7E)


@pytest.mark.parametrize("j", [0, 9, -9])
def test_fp8_quantizer_ties(nv, j):
    """FP8 tensorwise quantizer with static amax 448 * 2^-j, so the tensor scale is 2^-j and each
    quotient is v * 2^j exactly: every E4M3 midpoint and grid value with 8 neighbours either side,
    values past 448 (saturation), zeros, -0 and fp32 subnormals, both signs, against the oracle."""
    grid = np.array([oracle.e4m3_value(b) for b in range(1, 0x7F)], dtype=np.float32)
    pts = _neighbours(np.concatenate([_e4m3_midpoints(), grid]), 8)
    extra = np.array([0.0, 1e-45, 1e-40, 470.0, 480.0, 1e4, 1e30], dtype=np.float32)
    v = np.concatenate([pts, extra])
    v = np.concatenate([v, -v, np.array([-0.0], np.float32)])
    v = np.concatenate([v, np.zeros(-v.size % 256, np.float32)]).reshape(-1, 256)
    scale = np.float32(2.0 ** -j)
    x = (v * scale).astype(np.float32)
    amax = float(np.float32(448.0) * scale)
    _note(f"fp8 ties, scale 2^{-j}, {x.size} values")
    flags = torch.zeros(1, dtype=torch.int32, device=DEV)
    got = nv.quantize_fp8(to_dev_f32(x), amax=torch.tensor([amax], dtype=torch.float32, device=DEV), flags=flags)
    torch.cuda.synchronize()
    assert int(flags.item()) == 0
    rb, rs, _ = oracle.quantize_fp8(x, amax=amax)
    assert got.scale.item() == float(rs) == float(scale)
    b = got.data.cpu().numpy()
    bad = np.nonzero(b != rb)
    assert bad[0].size == 0, f"{bad[0].size} bytes differ; first v = {x[bad][0]!r}: {b[bad][0]:#04x} vs {rb[bad][0]:#04x}"
    # independent of the oracle: ties of the magnitude go to the even mantissa
    mags = np.abs(v.reshape(-1))
    on_mid = np.isin(mags, _e4m3_midpoints()) & (mags < 448)
    assert np.all((b.reshape(-1)[on_mid] & 1) == 0)
