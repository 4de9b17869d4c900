"""Pins of the CPU oracle to facts the pages and the mathematics fix, independent of the oracle.

Every check here compares the oracle with something other than itself: values the pages print,
closed forms, library routines (numpy rounding, torch's float8 / bfloat16 / float16 casts, scipy's
Student-t quantile), invariants, and brute force on tiny inputs.
"""
import math

import numpy as np
import pytest
import torch

import oracle
import synth
from conftest import read_golden

pytestmark = pytest.mark.filterwarnings("ignore::RuntimeWarning")


def _block_from_golden():
    gd = read_golden("worked_block.txt")
    raw = np.array([int(b, 16) for b in gd["bytes"]], dtype=np.uint8)
    return gd, raw


# ------------------------------------------------------------------------------------------------
# the printed block ("What NVFP4 is and how it differs from NF4", stored-block figure)
# ------------------------------------------------------------------------------------------------
def test_worked_block_decodes_to_printed_values():
    gd, raw = _block_from_golden()
    want = np.array([float(v) for v in gd["values"]])
    q = oracle.QTensor(raw.reshape(1, 8), np.array([[0x38]], dtype=np.uint8), np.float32(1.0))  # s = 1, g = 1
    got = oracle.dequantize(q, "f64").ravel()
    assert np.array_equal(got, want)
    # the printed 4-bit codes, low nibble first
    codes = [int(c, 2) for c in gd["codes"]]
    assert [int(raw[j // 2] >> (4 * (j % 2))) & 15 for j in range(16)] == codes
    assert [oracle.e2m1_value(c) for c in codes] == list(want)


def test_worked_block_named_bytes():
    # the three bytes the benchmark statement names explicitly
    pairs = {0xDC: (-2.0, -3.0), 0x5F: (-6.0, 3.0), 0x01: (0.5, 0.0)}
    for byte, (lo, hi) in pairs.items():
        q = oracle.QTensor(np.array([[byte] * 8], dtype=np.uint8), np.array([[0x38]], dtype=np.uint8), 1.0)
        got = oracle.dequantize(q, "f64").ravel()
        assert (got[0], got[1]) == (lo, hi)


def test_nibble_order_control():
    # Swapping the nibbles of the printed block changes 14 of its 16 values (only 0x?? with equal
    # nibbles would survive; none here).  On a whole matrix the swap raises the relative error to
    # about sqrt(2), as the page's nibble-order control reports (9.47 % -> 141 %).
    gd, raw = _block_from_golden()
    swapped = ((raw << 4) | (raw >> 4)).astype(np.uint8)
    s = np.array([[0x38]], dtype=np.uint8)
    a = oracle.dequantize(oracle.QTensor(raw.reshape(1, 8), s, 1.0), "f64").ravel()
    b = oracle.dequantize(oracle.QTensor(swapped.reshape(1, 8), s, 1.0), "f64").ravel()
    assert np.sum(a != b) == 16
    w = np.random.default_rng(7).standard_normal((256, 512)).astype(np.float32) * 0.02
    q, _ = oracle.quantize(w)
    ok = oracle.dequantize(q, "f64")
    qs = oracle.QTensor(((q.codes << 4) | (q.codes >> 4)).astype(np.uint8), q.scales, q.g)
    bad = oracle.dequantize(qs, "f64")
    e_ok = np.linalg.norm(w - ok) / np.linalg.norm(w)
    e_bad = np.linalg.norm(w - bad) / np.linalg.norm(w)
    assert 0.05 < e_ok < 0.15
    assert abs(e_bad - math.sqrt(2)) < 0.05


def test_worked_weight_value():
    # weight = E2M1 x block scale x global scale: -2.0 x 4.5 x 0.0017439 = -0.01570
    gd, _ = _block_from_golden()
    assert oracle.e4m3_value(0x49) == float(gd["block_scale"][0])
    g = np.float32(float(gd["global_scale"][0]))
    q = oracle.QTensor(np.array([[0x0C] + [0] * 7], dtype=np.uint8), np.array([[0x49]], dtype=np.uint8), g)
    w = oracle.dequantize(q, "f32")[0, 0]
    assert w == np.float32(np.float32(-2.0 * 4.5) * g)
    assert abs(float(w) - float(gd["first_weight"][0])) <= 5e-6


def test_worked_base_encodes_to_printed_code():
    # The base weight -0.01941 under block scale 4.5 and global 0.0017439 lands on code 1100 (-2.0).
    gd, _ = _block_from_golden()
    code = oracle.element_code(float(gd["first_weight_base"][0]), 4.5, float(np.float32(0.0017439)))
    assert code == int(gd["codes"][0], 2)


# ------------------------------------------------------------------------------------------------
# storage cost and range
# ------------------------------------------------------------------------------------------------
@pytest.mark.parametrize("shape", [(1, 16), (64, 256), (3, 4096), (17, 48)])
def test_storage_is_4_5_bits(shape):
    q, _ = oracle.quantize(np.random.default_rng(1).standard_normal(shape).astype(np.float32))
    bits = (q.codes.nbytes + q.scales.nbytes) * 8
    assert bits == 4.5 * shape[0] * shape[1]


def test_range_and_amax_element():
    rng = np.random.default_rng(3)
    for trial in range(20):
        w = (rng.standard_t(3, size=(32, 64)) * 10 ** rng.uniform(-6, 3)).astype(np.float32)
        q, _ = oracle.quantize(w)
        vals = np.array([oracle.e2m1_value(c) for c in range(16)])
        lo, hi = q.codes & 15, q.codes >> 4
        assert np.abs(vals[lo]).max() <= 6 and np.abs(vals[hi]).max() <= 6
        r, c = np.unravel_index(np.argmax(np.abs(w)), w.shape)
        assert q.scales[r, c // 16] == 0x7E
        code = (q.codes[r, c // 2] >> (4 * (c % 2))) & 15
        assert code & 7 == 7 and (code >> 3) == (w[r, c] < 0)
        assert q.g == np.float32(np.abs(w).max() / np.float32(2688.0))


# ------------------------------------------------------------------------------------------------
# the two grids against library rounding
# ------------------------------------------------------------------------------------------------
def _e2m1_numpy(y):
    """Round-half-to-even onto {0,.5,1,1.5,2,3,4,6} with numpy's rint, saturating at 6."""
    y = np.asarray(y, dtype=np.float64)
    out = np.where(y < 2, np.rint(y * 2) / 2, np.where(y < 4, np.rint(y), 2 * np.rint(y / 2)))
    return np.minimum(out, 6.0)


def test_e2m1_rounding_against_numpy_rint():
    mags = np.array([0, 0.5, 1, 1.5, 2, 3, 4, 6])
    mids = (mags[1:] + mags[:-1]) / 2
    probes = [0.0, 6.0, 7.0, 1e30, np.float32(np.inf)]
    for m in np.concatenate([mags, mids]):
        m32 = np.float32(m)
        probes += [m32, np.nextafter(m32, np.float32(0)), np.nextafter(m32, np.float32(10))]
    rnd = np.random.default_rng(11)
    probes = np.concatenate([np.array(probes, dtype=np.float32),
                             rnd.uniform(0, 8, 200000).astype(np.float32),
                             (10.0 ** rnd.uniform(-45, 1, 50000)).astype(np.float32)])
    idx = oracle.e2m1_index_array(probes)
    want = _e2m1_numpy(np.where(np.isinf(probes), 1e300, probes))
    assert np.array_equal(mags[idx], want)


def test_e4m3_table_against_torch():
    b = torch.arange(256, dtype=torch.int32).to(torch.uint8)
    ref = b.view(torch.float8_e4m3fn).to(torch.float64).numpy()
    got = np.array([oracle.e4m3_value(i) for i in range(256)])
    assert np.array_equal(np.isnan(got), np.isnan(ref))
    m = ~np.isnan(ref)
    assert np.array_equal(got[m], ref[m])
    assert oracle.e4m3_value(0x7E) == 448.0 and math.isnan(oracle.e4m3_value(0x7F))
    assert oracle.e4m3_value(0x01) == 2.0 ** -9


def test_e4m3_rounding_against_torch_cast():
    vals = np.array([oracle.e4m3_value(i) for i in range(0x7F)], dtype=np.float64)
    mids = (vals[1:] + vals[:-1]) / 2
    probes = []
    for m in np.concatenate([vals, mids]):
        m32 = np.float32(m)
        probes += [m32, np.nextafter(m32, np.float32(0)), np.nextafter(m32, np.float32(1e4))]
    rnd = np.random.default_rng(12)
    probes = np.concatenate([np.array(probes, dtype=np.float32),
                             (2.0 ** rnd.uniform(-12, 8.8, 200000)).astype(np.float32)])
    probes = probes[probes < 464]  # torch's cast has no saturation above the last midpoint
    got = oracle.e4m3_encode_array(probes)
    ref = torch.from_numpy(probes).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(got, ref)
    # saturation: everything from the 448/480 midpoint up, including +inf, gives 0x7E
    big = np.array([464, 465, 1000, 3e38, np.inf], dtype=np.float32)
    assert np.all(oracle.e4m3_encode_array(big) == 0x7E)


def test_f32_to_bf16_against_torch():
    rnd = np.random.default_rng(13)
    x = np.concatenate([rnd.standard_normal(100000).astype(np.float32),
                        (rnd.integers(0, 2 ** 16, 50000) << 16 | 0x8000).astype(np.uint32).view(np.float32),
                        np.array([0.0, -0.0, 1e-40, -1e-40, 3.4e38], dtype=np.float32)])
    x = x[np.isfinite(x)]
    want = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(oracle.f32_to_bf16_bits(x), want)


def test_widen_bf16_against_torch():
    # every bf16 bit pattern widens to the fp32 value torch gives it (NaN patterns stay NaN)
    h = np.arange(65536, dtype=np.uint32).astype(np.uint16).reshape(4096, 16)
    got = oracle.widen(h, oracle.BF16)
    want = torch.from_numpy(h.view(np.int16)).view(torch.bfloat16).to(torch.float32).numpy()
    assert np.array_equal(np.isnan(got), np.isnan(want))
    m = ~np.isnan(want)
    assert np.array_equal(got[m].view(np.uint32), want[m].view(np.uint32))
    # and the bf16 -> f64 helper the GEMM references use agrees with it
    assert np.array_equal(oracle.bf16_bits_to_f64(h)[m], want[m].astype(np.float64))


def test_widen_f16_against_numpy():
    h = np.arange(65536, dtype=np.uint32).astype(np.uint16).reshape(4096, 16)
    got = oracle.widen(h, oracle.F16)
    want = h.view(np.float16).astype(np.float32)
    assert np.array_equal(np.isnan(got), np.isnan(want))
    m = ~np.isnan(want)
    assert np.array_equal(got[m].view(np.uint32), want[m].view(np.uint32))


def test_widen_e4m3_with_scale_against_torch():
    b = np.arange(256, dtype=np.uint32).astype(np.uint8).reshape(16, 16)
    sc = np.float32(0.0123)
    got = oracle.widen(b, oracle.E4M3, float(sc))
    want = (torch.from_numpy(b).view(torch.float8_e4m3fn).to(torch.float32) * torch.tensor(sc)).numpy()
    m = ~np.isnan(want)
    assert np.array_equal(np.isnan(got), ~m)
    assert np.array_equal(got[m], want[m])
    # a missing weight_scale means 1.0
    assert np.array_equal(oracle.widen(b, oracle.E4M3)[m],
                          torch.from_numpy(b).view(torch.float8_e4m3fn).to(torch.float32).numpy()[m])


# ------------------------------------------------------------------------------------------------
# brute force on tiny inputs and invariants of the quantizer
# ------------------------------------------------------------------------------------------------
def test_block_scale_is_nearest_e4m3_of_ratio():
    rnd = np.random.default_rng(21)
    for _ in range(2000):
        g = np.float32(10.0 ** rnd.uniform(-8, 2))
        bamax = np.float32(float(g) * 6 * 10.0 ** rnd.uniform(-4, 2.8))
        t = np.float32(bamax / np.float32(np.float32(6.0) * g))
        want = 0x7E if t >= 464 else int(torch.tensor([t]).to(torch.float8_e4m3fn).view(torch.uint8)[0])
        assert oracle.block_scale_byte(float(bamax), float(g)) == want


def test_codes_are_nearest_grid_values_brute_force():
    # For every element, the chosen E2M1 magnitude is the nearest grid point to |v| / (s g) computed
    # exactly, unless |v| / (s g) sits within 1e-6 (relative) of a midpoint, where the fp32
    # reciprocal-multiply may land on either side.
    rnd = np.random.default_rng(22)
    mags = np.array([0, 0.5, 1, 1.5, 2, 3, 4, 6])
    mids = (mags[1:] + mags[:-1]) / 2
    for trial in range(300):
        rows, nblk = 2, 3
        w = (rnd.standard_normal((rows, 16 * nblk)) * 10.0 ** rnd.uniform(-5, 2)).astype(np.float32)
        w[rnd.random(w.shape) < 0.1] = 0.0
        q, _ = oracle.quantize(w)
        for r in range(rows):
            for c in range(16 * nblk):
                s = oracle.e4m3_value(int(q.scales[r, c // 16]))
                code = (int(q.codes[r, c // 2]) >> (4 * (c % 2))) & 15
                assert (code >> 3) == int(np.signbit(w[r, c]))
                if s == 0:
                    assert code & 7 == 0
                    continue
                x = abs(float(w[r, c])) / (s * float(q.g))
                if np.any(np.abs(x - mids) <= 1e-6 * max(x, 1e-30)):
                    continue
                nearest = np.argmin(np.abs(mags - min(x, 6.0)))
                assert code & 7 == nearest, (x, code)


def test_round_trip_is_identity():
    # Codes and scales that dequantize to a tensor whose amax is 6 * 448 * g, with g a power of two:
    # quantizing the expanded tensor (with amax fixed to 2688 g) returns the same bits.
    rnd = np.random.default_rng(23)
    for trial in range(20):
        rows, cols = 8, 128
        g = np.float32(2.0 ** rnd.integers(-30, 0))
        codes = rnd.integers(0, 256, (rows, cols // 2), dtype=np.uint8)
        scales = rnd.integers(1, 0x7F, (rows, cols // 16), dtype=np.uint8)
        scales[0, 0] = 0x7E
        # every block carries a +-6 in its first element
        codes[:, ::8] = (codes[:, ::8] & 0xF0) | (0x7 | (rnd.integers(0, 2, (rows, cols // 16)) << 3)).astype(np.uint8)
        q = oracle.QTensor(codes, scales, g)
        w = oracle.dequantize(q, "f32")
        q2, flags = oracle.quantize(w, amax=float(np.float32(2688.0) * g))
        assert flags == 0 and q2.g == g
        assert np.array_equal(q2.scales, scales)
        assert np.array_equal(q2.codes, codes)


def test_global_amax_is_numpy_max_and_zero_tensor():
    rnd = np.random.default_rng(24)
    w = rnd.standard_t(2, size=(50, 160)).astype(np.float32)
    q, _ = oracle.quantize(w)
    assert q.g == np.float32(np.float32(np.abs(w).max()) / np.float32(2688))
    z, flags = oracle.quantize(np.zeros((4, 32), dtype=np.float32))
    assert z.g == 0 and not z.scales.any() and not z.codes.any() and flags == 0
    nz = -np.zeros((4, 32), dtype=np.float32)
    z2, _ = oracle.quantize(nz)
    assert np.all(z2.codes == 0x88)  # sign of -0 kept


def test_nonfinite_input_flagged():
    w = np.ones((2, 32), dtype=np.float32)
    w[1, 5] = np.nan
    assert oracle.quantize(w)[1] & 1
    w[1, 5] = -np.inf
    assert oracle.quantize(w)[1] & 1
    b = np.zeros((1, 16), dtype=np.uint8)
    b[0, 3] = 0x7F
    assert oracle.quantize(b, oracle.E4M3, 1.0)[1] & 1


def test_static_amax_clips():
    # With a calibrated amax below the data's, large elements saturate at +-6 x 448 x g.
    w = np.linspace(-10, 10, 64, dtype=np.float32).reshape(2, 32)
    q, _ = oracle.quantize(w, amax=1.0)
    d = oracle.dequantize(q, "f64")
    assert np.max(np.abs(d)) == pytest.approx(6 * 448 * float(q.g))
    assert q.g == np.float32(np.float32(1.0) / np.float32(2688))


def test_expansion_is_single_rounding_of_exact_product():
    rnd = np.random.default_rng(25)
    codes = rnd.integers(0, 256, (16, 64), dtype=np.uint8)
    scales = rnd.integers(0, 0x7F, (16, 8), dtype=np.uint8)
    for g in [np.float32(0.0017439), np.float32(3.1e-39), np.float32(1.7e35)]:
        q = oracle.QTensor(codes, scales, g)
        f32 = oracle.dequantize(q, "f32")
        c = np.where(np.arange(128) % 2 == 0, codes.repeat(2, 1) & 15, codes.repeat(2, 1) >> 4)
        cs = np.array([oracle.e2m1_value(i) for i in range(16)], dtype=np.float32)[c] * \
            np.array([oracle.e4m3_value(i) for i in range(128)], dtype=np.float32)[scales.repeat(16, 1)]
        want = (cs * g).astype(np.float32)  # e2m1*s is exact in fp32; one fp32 multiply by g
        assert np.array_equal(f32.view(np.uint32), want.view(np.uint32))
        bf = oracle.dequantize(q, "bf16")
        assert np.array_equal(bf, torch.from_numpy(want).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16))


# ------------------------------------------------------------------------------------------------
# GEMM reference
# ------------------------------------------------------------------------------------------------
def test_gemm_one_hot_rows_reproduce_expansion():
    rnd = np.random.default_rng(31)
    w = rnd.standard_normal((48, 96)).astype(np.float32)
    q, _ = oracle.quantize(w)
    a = np.zeros((96, 96), dtype=np.float32)
    a[np.arange(96), np.arange(96)] = 1.0
    a_bits = oracle.f32_to_bf16_bits(a)
    c = oracle.gemm_w4a16(a_bits, q)
    assert np.array_equal(c.astype(np.float32), oracle.dequantize(q, "f32").T)


def test_gemm_definition_brute_force_and_zero_weight():
    rnd = np.random.default_rng(32)
    a_bits = oracle.f32_to_bf16_bits(rnd.standard_normal((3, 32)).astype(np.float32))
    q, _ = oracle.quantize(rnd.standard_normal((5, 32)).astype(np.float32))
    c = oracle.gemm_w4a16(a_bits, q)
    a = oracle.widen(a_bits, oracle.BF16).astype(np.float64)
    w = oracle.dequantize(q, "f64")
    for m in range(3):
        for n in range(5):
            assert c[m, n] == pytest.approx(sum(a[m, k] * w[n, k] for k in range(32)), rel=1e-14, abs=1e-300)
    qz, _ = oracle.quantize(np.zeros((5, 32), dtype=np.float32))
    assert not oracle.gemm_w4a16(a_bits, qz).any()


def _lowrank_case(m, n, k, r, seed):
    rnd = np.random.default_rng(seed)
    a_bits = oracle.f32_to_bf16_bits(rnd.standard_normal((m, k)).astype(np.float32))
    q, _ = oracle.quantize((rnd.standard_normal((n, k)) * 0.02).astype(np.float32))
    v_bits = oracle.f32_to_bf16_bits((rnd.standard_normal((r, k)) * 0.05).astype(np.float32))
    u_bits = oracle.f32_to_bf16_bits((rnd.standard_normal((n, r)) * 0.05).astype(np.float32))
    return a_bits, q, v_bits, u_bits


def test_gemm_lowrank_brute_force_and_zero_branch():
    a_bits, q, v_bits, u_bits = _lowrank_case(3, 5, 32, 4, 41)
    c = oracle.gemm_lowrank(a_bits, q, v_bits, u_bits)
    a = oracle.widen(a_bits, oracle.BF16).astype(np.float64)
    w = oracle.dequantize(q, "f64")
    v = oracle.widen(v_bits, oracle.BF16).astype(np.float64)
    u = oracle.widen(u_bits, oracle.BF16).astype(np.float64)
    for i in range(3):
        for j in range(5):
            main = math.fsum(a[i, kk] * w[j, kk] for kk in range(32))
            branch = math.fsum(math.fsum(a[i, kk] * v[t, kk] for kk in range(32)) * u[j, t] for t in range(4))
            assert c[i, j] == pytest.approx(main + branch, rel=1e-13, abs=1e-15)
    # a zero branch leaves the plain W4A16 product, bit for bit
    zv = np.zeros_like(v_bits)
    assert np.array_equal(oracle.gemm_lowrank(a_bits, q, zv, u_bits), oracle.gemm_w4a16(a_bits, q))


def test_gemm_lowrank_equals_product_with_the_rank_r_matrix():
    # (A . V^T) . U^T = A . (U . V)^T: the branch as one product with the dense rank-r matrix U . V
    a_bits, q, v_bits, u_bits = _lowrank_case(17, 40, 96, 16, 42)
    a = oracle.widen(a_bits, oracle.BF16).astype(np.float64)
    lr = oracle.widen(u_bits, oracle.BF16).astype(np.float64) @ oracle.widen(v_bits, oracle.BF16).astype(np.float64)
    want = oracle.gemm_w4a16(a_bits, q) + np.einsum("mk,nk->mn", a, lr)
    got = oracle.gemm_lowrank(a_bits, q, v_bits, u_bits)
    assert np.max(np.abs(got - want)) <= 1e-12 * np.max(np.abs(want))
    # one-hot: A = e_0, V = e_3 (row 0), U = e_7 (column 0) adds exactly 1 to C[0, 7]
    a1 = np.zeros((1, 96), dtype=np.uint16)
    a1[0, 3] = 0x3F80  # bf16 1.0
    v1 = np.zeros((16, 96), dtype=np.uint16)
    v1[0, 3] = 0x3F80
    u1 = np.zeros((40, 16), dtype=np.uint16)
    u1[7, 0] = 0x3F80
    d = oracle.gemm_lowrank(a1, q, v1, u1) - oracle.gemm_w4a16(a1, q)
    assert d[0, 7] == 1.0 and np.count_nonzero(d) == 1


def test_gemm_lowrank_w4a4_main_product_uses_quantized_activations():
    a_bits, q, v_bits, u_bits = _lowrank_case(6, 24, 64, 16, 43)
    qa, _ = oracle.quantize(a_bits, oracle.BF16)
    got = oracle.gemm_lowrank(a_bits, q, v_bits, u_bits, a_q=qa)
    branch = oracle.gemm_lowrank(a_bits, q, v_bits, u_bits) - oracle.gemm_w4a16(a_bits, q)
    want = oracle.gemm_w4a4(qa, q) + branch
    assert np.max(np.abs(got - want)) <= 1e-13 * np.max(np.abs(want))


def test_gemm_error_metric_floor():
    cref = np.array([[1.0, -1.0, 1e-9]])
    c = cref + np.array([[1e-4, 0, 5e-6]])
    # the near-zero output is judged against 1e-2 of its row's largest magnitude
    assert oracle.gemm_error(c, cref) == pytest.approx(5e-4)


# ------------------------------------------------------------------------------------------------
# percentile calibration
# ------------------------------------------------------------------------------------------------
def test_rank_nearest_rank_definition():
    assert oracle.rank(99.9, 217088) == 216871
    assert oracle.rank(100.0, 10) == 10
    assert oracle.rank(50.0, 4) == 2
    assert oracle.rank(1e-9, 1000) == 1
    for n in [1, 7, 1000, 4096]:
        perm = np.random.default_rng(n).permutation(np.arange(1, n + 1)).astype(np.float32).reshape(n, 1)
        pct, mx = oracle.amax_percentile(perm, 99.9)
        assert pct[0] == math.ceil(0.999 * n) and mx[0] == n


def test_percentile_against_numpy_sort():
    rnd = np.random.default_rng(41)
    x = (rnd.standard_t(3, size=(1000, 12)) * rnd.choice([-1, 1], size=(1000, 12))).astype(np.float32)
    x[5, 3] = -0.0
    for p in [0.1, 50, 99, 99.9, 100]:
        pct, mx = oracle.amax_percentile(x, p)
        srt = np.sort(np.abs(x), axis=0)
        k = math.ceil(p * 1000 / 100)
        assert np.array_equal(pct, srt[k - 1]) and np.array_equal(mx, srt[-1])
        pt, mt = oracle.amax_percentile(x, p, per_channel=False)
        assert pt[0] == np.sort(np.abs(x).ravel())[math.ceil(p * x.size / 100) - 1] and mt[0] == np.abs(x).max()


def test_percentile_student_t_closed_form():
    # |t_3| has its 99.9 % point at the two-sided 0.1 % quantile of Student-t(3), 12.924.
    # Over 217 088 rows the per-channel estimate has a standard error of about 0.30.
    scipy_stats = pytest.importorskip("scipy.stats")
    q = scipy_stats.t.ppf(1 - 0.0005, 3)
    assert q == pytest.approx(12.924, abs=1e-3)
    x = np.random.default_rng(5000).standard_t(3, size=(53 * 4096, 32)).astype(np.float32)
    pct, mx = oracle.amax_percentile(x, 99.9)
    assert np.all(np.abs(pct - q) < 1.3)
    assert abs(pct.mean() - q) < 0.25
    assert np.all(mx >= pct)


def test_gemm_against_unquantized_tracks_weight_error():
    # With independent Gaussian weight errors, the W4A16 product's Frobenius error against the
    # unquantized product equals the weight's relative quantization error (about 9.5 % for
    # N(0, 0.02) weights, the Gaussian counterpart of the pages' per-matrix 6.3-9.6 %).  A wrong
    # scale, sign or nibble order anywhere in quantize, expand or GEMM breaks the equality.
    w = synth.normal_f32((256, 1024), 0.02, 11)
    a = synth.bf16_bits(np.random.default_rng(12).standard_normal((128, 1024)).astype(np.float32))
    q, _ = oracle.quantize(w)
    werr = np.linalg.norm(oracle.dequantize(q, "f64") - w) / np.linalg.norm(w)
    cq = oracle.gemm_w4a16(a, q)
    cu = oracle.gemm_f64(oracle.bf16_bits_to_f64(a), w.astype(np.float64))
    cerr = np.linalg.norm(cq - cu) / np.linalg.norm(cu)
    assert 0.07 < werr < 0.12
    assert 0.85 * werr < cerr < 1.15 * werr


# ------------------------------------------------------------------------------------------------
# FP8 tensorwise ("Qwen3-VL-8B-Instruct-heretic-NVFP4", "Quantization Details": float8_e4m3fn,
# tensorwise, round to nearest; "Runtime / hardware": FP4 weight x dynamically quantized FP8
# activation)
# ------------------------------------------------------------------------------------------------
def test_fp8_bytes_against_torch_division_and_cast():
    # torch's float32 division and its float8_e4m3fn cast are an independent implementation of
    # byte = nearest-even E4M3 of fl(v / scale); probes sit on grid points, midpoints and their
    # neighbours after scaling, for several scales, both signs
    vals = np.array([oracle.e4m3_value(i) for i in range(0x7F)], dtype=np.float64)
    mids = (vals[1:] + vals[:-1]) / 2
    rnd = np.random.default_rng(41)
    for scale in [np.float32(1.0), np.float32(0.02 * 4.5 / 448), np.float32(3.7e-3), np.float32(1.2345e2)]:
        q = []
        for m in np.concatenate([vals, mids]):
            m32 = np.float32(m * float(scale))
            q += [m32, np.nextafter(m32, np.float32(0)), np.nextafter(m32, np.float32(1e30))]
        q = np.array(q, dtype=np.float32)
        q = np.concatenate([q, (float(scale) * 2.0 ** rnd.uniform(-12, 8.8, 50000)).astype(np.float32)])
        q = np.concatenate([q, -q, np.array([0.0, -0.0], dtype=np.float32)])
        tq = torch.from_numpy(q) / torch.tensor(scale, dtype=torch.float32)
        keep = (tq.abs() < 464).numpy()
        ref = tq[torch.from_numpy(keep)].to(torch.float8_e4m3fn).view(torch.uint8).numpy()
        got = np.array([oracle.fp8_byte(float(v), float(scale)) for v in q[keep]], dtype=np.uint8)
        assert np.array_equal(got, ref), f"scale {scale}"


def test_fp8_scale_and_largest_element():
    rnd = np.random.default_rng(42)
    for shape in [(7, 48), (64, 256)]:
        x = (rnd.standard_t(4, size=shape) * 0.02).astype(np.float32)
        b, sc, flags = oracle.quantize_fp8(x)
        amax = np.float32(np.abs(x).max())
        assert flags == 0 and sc == np.float32(amax / np.float32(448))
        i = np.unravel_index(np.argmax(np.abs(x)), shape)
        assert b[i] & 0x7F == 0x7E  # |amax| / fl(amax / 448) rounds to 448
        assert (b[i] & 0x80 != 0) == bool(x[i] < 0)
        assert np.all((b & 0x7F) != 0x7F)  # no NaN byte is produced


def test_fp8_round_trip_and_error_bound():
    rnd = np.random.default_rng(43)
    x = (rnd.standard_normal((32, 512)) * 0.05).astype(np.float32)
    b, sc, _ = oracle.quantize_fp8(x)
    v = oracle.fp8_values(b, sc)
    # requantizing the dequantized values with the same scale reproduces the bytes
    b2 = np.array([[oracle.fp8_byte(float(np.float32(t)), float(sc)) for t in row] for row in v], dtype=np.uint8)
    assert np.array_equal(b2, b)
    # nearest rounding: within half a grid step (relative 2^-4) in the normal range, 2^-10 * scale below it
    err = np.abs(v - x.astype(np.float64))
    bound = np.maximum(np.abs(x) * 2.0 ** -4, 2.0 ** -10 * float(sc)) * (1 + 1e-6)
    assert np.all(err <= bound)


def test_fp8_zero_tensor_static_amax_and_flags():
    b, sc, flags = oracle.quantize_fp8(np.zeros((2, 32), dtype=np.float32))
    assert sc == 1.0 and not b.any() and flags == 0
    x = np.array([[0.5, -4.0, 2.0, -0.0] * 8], dtype=np.float32)
    b, sc, _ = oracle.quantize_fp8(x, amax=1.0)
    assert sc == np.float32(1.0 / 448)
    assert b[0, 1] == 0xFE and b[0, 2] == 0x7E and b[0, 3] == 0x80  # beyond the static amax: saturate
    x[0, 5] = np.nan
    assert oracle.quantize_fp8(x)[2] & 1


def test_gemm_w4a8_one_hot_and_definition():
    rnd = np.random.default_rng(44)
    q, _ = oracle.quantize(rnd.standard_normal((24, 64)).astype(np.float32))
    eye = np.zeros((64, 64), dtype=np.float32)
    eye[np.arange(64), np.arange(64)] = 1.0
    b, sc, _ = oracle.quantize_fp8(eye)
    c = oracle.gemm_w4a8(b, sc, q)
    assert np.array_equal(c, oracle.dequantize(q, "f64").T * (448.0 * float(sc)))
    xa = rnd.standard_normal((3, 64)).astype(np.float32)
    ba, sa, _ = oracle.quantize_fp8(xa)
    c = oracle.gemm_w4a8(ba, sa, q)
    a = oracle.fp8_values(ba, sa)
    w = oracle.dequantize(q, "f64")
    for m in range(3):
        for n in range(0, 24, 5):
            assert c[m, n] == pytest.approx(sum(a[m, k] * w[n, k] for k in range(64)), rel=1e-14, abs=1e-300)


# ------------------------------------------------------------------------------------------------
# matrix statistics ("Qwen-Image NVFP4 on a 16 GB Ada GPU", section "Quality: the error of each
# matrix": relative error of each matrix, kurtosis, max / std in blocks of 64)
# ------------------------------------------------------------------------------------------------
def test_stats_kurtosis_and_moments_against_scipy():
    import scipy.stats
    rnd = np.random.default_rng(51)
    for x in [rnd.standard_normal((64, 512)), rnd.standard_t(3, (128, 256)) * 0.02, rnd.uniform(-1, 1, (32, 1024))]:
        x = x.astype(np.float32)
        st = oracle.matrix_stats(x)
        xd = x.ravel().astype(np.float64)
        assert st["kurtosis"] == pytest.approx(scipy.stats.kurtosis(xd, fisher=True, bias=True), rel=1e-10, abs=1e-12)
        assert st["mean"] == pytest.approx(xd.mean(), rel=1e-12, abs=1e-15)
        assert st["std"] == pytest.approx(xd.std(), rel=1e-12)
        assert st["max_abs"] == np.abs(xd).max()
    # uniform on [-1, 1]: excess kurtosis -6/5
    big = rnd.uniform(-1, 1, (1024, 1024)).astype(np.float32)
    assert oracle.matrix_stats(big)["kurtosis"] == pytest.approx(-1.2, abs=0.01)


def test_stats_relative_error_against_numpy_norm():
    rnd = np.random.default_rng(52)
    w = (rnd.standard_normal((96, 768)) * 0.02).astype(np.float32)
    q, _ = oracle.quantize(w)
    wh = oracle.dequantize(q, "f64")
    ref = np.linalg.norm(w.astype(np.float64) - wh) / np.linalg.norm(w.astype(np.float64))
    assert oracle.matrix_stats(w, q)["rel_error"] == pytest.approx(ref, rel=1e-12)
    assert np.isnan(oracle.matrix_stats(w)["rel_error"])
    # Gaussian weights sit in the page's band for NVFP4 (median 9.47 %, all matrices 6.3 .. 9.6 %)
    assert 0.08 < oracle.matrix_stats(w, q)["rel_error"] < 0.11


def test_stats_block_ratio_closed_forms():
    # one spike per block of 64: mean x/64, std x sqrt(63)/64, so max/std = 64/sqrt(63)
    x = np.zeros((4, 128), dtype=np.float32)
    x[:, 5] = 3.0
    x[:, 64 + 17] = -0.25
    st = oracle.matrix_stats(x)
    assert st["blocks"] == 8 and st["block_max_over_std"] == pytest.approx(64 / math.sqrt(63), rel=1e-14)
    # alternating +-a: std a, max a
    y = np.tile(np.array([0.5, -0.5], dtype=np.float32), (8, 96))
    assert oracle.matrix_stats(y)["block_max_over_std"] == pytest.approx(1.0, rel=1e-15)
    # constant blocks have std 0 and are left out; a shorter last block counts with its own length
    z = np.full((3, 48), 2.0, dtype=np.float32)  # 144 elements: blocks of 64, 64, 16
    z[2, 32] = 0.0                                # inside the last block (elements 128..143)
    st = oracle.matrix_stats(z)
    assert st["blocks"] == 1
    assert st["block_max_over_std"] == pytest.approx(2.0 / (math.sqrt(15) / 16 * 2.0), rel=1e-14)
    # Gaussian blocks of 64: the page reports 2.61 for its non-modulation matrices
    g = np.random.default_rng(53).standard_normal((256, 1024)).astype(np.float32)
    assert 2.5 < oracle.matrix_stats(g)["block_max_over_std"] < 2.8
