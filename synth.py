"""Seeded synthetic inputs shared by the tests, the smoke check and the benchmark.

This module draws random tensors and converts them to storage formats with library casts
(numpy, and torch's CPU casts to bfloat16 / float8_e4m3fn).  It holds none of the NVFP4 method's
arithmetic: no block scales, no E2M1 rounding, no global scale.

Shapes and distributions follow the pages' workloads:
- Qwen-Image attention projection: 3072 x 3072 weights, 4096 tokens (64 x 64 latent patches at
  1024^2) x 3072 activations with a few outlier channels;
- the modulation matrices of "Qwen-Image NVFP4 on a 16 GB Ada GPU" (18432 x 3072, section
  "Quality: the error of each matrix"), stored as FP8 E4M3 with a per-tensor fp32 weight_scale as in
  "Qwen-Rapid-AIO-NVFP4", section "Why This Exists";
- a Qwen3-VL-8B text MLP (gate/up 12288 x 4096, down 4096 x 12288) with 512 tokens
  ("Qwen3-VL-8B-Instruct-heretic-NVFP4", "Quantization Details");
- heavy-tailed activations (Student-t, 3 degrees of freedom) for p99.9 calibration over
  53 samples x 4096 tokens x 3072 channels ("Qwen-Rapid-AIO-NVFP4", "Recommended Model").
No dataset or checkpoint is read: everything here is drawn from numpy's default_rng.

Seeds: config 1 uses one generator seeded 0 (weights first, then activations); config c in 2..5
seeds tensor i with c * 1000 + i.
"""
from __future__ import annotations

import numpy as np
import torch


def rng(seed: int) -> np.random.Generator:
    return np.random.default_rng(seed)


def normal_f32(shape, sigma: float, seed: int | np.random.Generator) -> np.ndarray:
    g = seed if isinstance(seed, np.random.Generator) else rng(seed)
    return (g.standard_normal(shape) * sigma).astype(np.float32)


def bf16_bits(x: np.ndarray) -> np.ndarray:
    """fp32 -> bf16 (torch's round-to-nearest-even cast), returned as uint16 bit patterns."""
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16)


def fp8_tensorwise(w: np.ndarray) -> tuple[np.ndarray, np.float32]:
    """A per-tensor FP8 E4M3 checkpoint tensor: scale = amax / 448, bytes = cast(w / scale).
    Returns (uint8 bytes, fp32 weight_scale)."""
    w = np.ascontiguousarray(w, dtype=np.float32)
    amax = np.float32(np.abs(w).max())
    scale = np.float32(amax / np.float32(448.0)) if amax > 0 else np.float32(1.0)
    t = (torch.from_numpy(w) / torch.tensor(scale, dtype=torch.float32)).to(torch.float8_e4m3fn)
    return t.view(torch.uint8).numpy().copy(), scale


# ------------------------------------------------------------------------------------------------
# the five workloads
# ------------------------------------------------------------------------------------------------
def tiny():
    """64 x 256 fp32 weight ~ N(0, 0.02^2), then 16 x 256 bf16 activations ~ N(0, 1), one rng."""
    g = rng(0)
    w = normal_f32((64, 256), 0.02, g)
    a = bf16_bits(g.standard_normal((16, 256)).astype(np.float32))
    return {"w": w, "a": a}


def attn_proj_weight(rows: int = 3072, cols: int = 3072) -> np.ndarray:
    return normal_f32((rows, cols), 0.02, 2000)


def attn_proj_activations(tokens: int = 4096, channels: int = 3072) -> np.ndarray:
    """N(0, 1) with 0.1 % of channels (3 of 3072) scaled x20 as outliers; bf16 bits."""
    g = rng(2001)
    a = g.standard_normal((tokens, channels))
    n_out = max(1, int(round(channels * 0.001)))
    cols = g.choice(channels, size=n_out, replace=False)
    a[:, cols] *= 20.0
    return bf16_bits(a.astype(np.float32))


def modulation_weight(rows: int = 18432, cols: int = 3072) -> np.ndarray:
    return normal_f32((rows, cols), 0.01, 3000)


def modulation_activations(m: int = 2, cols: int = 3072) -> np.ndarray:
    return bf16_bits(rng(3001).standard_normal((m, cols)).astype(np.float32))


def modulation_fp8(i: int, rows: int = 18432, cols: int = 3072):
    """Weight i (0..59) of the requantization batch as an FP8 checkpoint tensor."""
    return fp8_tensorwise(normal_f32((rows, cols), 0.01, 3100 + i))


def mlp_weights(hidden: int = 4096, inter: int = 12288):
    wg = normal_f32((inter, hidden), 0.015, 4000)
    wu = normal_f32((inter, hidden), 0.015, 4001)
    wd = normal_f32((hidden, inter), 0.015, 4002)
    return wg, wu, wd


def mlp_activations(tokens: int = 512, hidden: int = 4096) -> np.ndarray:
    return bf16_bits(rng(4003).standard_normal((tokens, hidden)).astype(np.float32))


def calib_activations(rows: int = 53 * 4096, cols: int = 3072, seed: int = 5000) -> np.ndarray:
    """Student-t (nu = 3) activations, bf16 bits [rows x cols]."""
    return bf16_bits(rng(seed).standard_t(3, size=(rows, cols)).astype(np.float32))


def stack_weight_fp8(block: int, j: int):
    """Weight j of block `block` in the 60-block stack: j 0..3 are 3072 x 3072, j 4 is
    12288 x 3072, j 5 is 3072 x 12288; each 0.02 * N(0, 1) stored as FP8 tensorwise."""
    shape = [(3072, 3072)] * 4 + [(12288, 3072), (3072, 12288)]
    return fp8_tensorwise(normal_f32(shape[j], 0.02, 5100 + 6 * block + j))
