"""Helpers for the GPU parity tests: move numpy arrays (fp32, bf16/fp16 bit patterns, E4M3 bytes)
to the device as torch tensors and back.  No NVFP4 arithmetic lives here."""
import numpy as np
import torch

DEV = torch.device("cuda:0")


def to_dev_f32(x: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(DEV)


def to_dev_bf16(bits: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(bits, dtype=np.uint16).view(np.int16)).to(DEV).view(torch.bfloat16)


def to_dev_f16(bits: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(bits, dtype=np.uint16).view(np.int16)).to(DEV).view(torch.float16)


def to_dev_u8(b: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(b, dtype=np.uint8)).to(DEV)


def bits16(t: torch.Tensor) -> np.ndarray:
    return t.view(torch.int16).cpu().numpy().view(np.uint16)


def padded(t: torch.Tensor, extra_cols: int) -> torch.Tensor:
    """The same matrix stored with a larger row stride (a view into a wider buffer)."""
    rows, cols = t.shape
    buf = torch.empty((rows, cols + extra_cols), dtype=t.dtype, device=t.device)
    buf[:, :cols] = t
    return buf[:, :cols]
