"""Shared test helpers: moving bit patterns between numpy and torch, tolerances."""
import numpy as np
import torch

# Tolerances on max_n |y_gpu - y_exact| / max(|y_exact|, 1e-3 * rms(y_exact))
TOL_BF16 = 1e-2
TOL_F32 = 2e-3


def dev():
    return torch.device("cuda:0")


def to_gpu_f32(a: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(dev())


def to_gpu_bf16_bits(bits: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(bits, dtype=np.uint16).view(np.int16)).to(dev()).view(torch.bfloat16)


def to_gpu_packed(p: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(p, dtype=np.uint32).view(np.int32)).to(dev())


def packed_np(t: torch.Tensor) -> np.ndarray:
    return t.cpu().numpy().view(np.uint32)


def bf16_bits_np(t: torch.Tensor) -> np.ndarray:
    return t.view(torch.int16).cpu().numpy().view(np.uint16)


def out_np(t: torch.Tensor) -> np.ndarray:
    """Output tensor values as float64 (bf16 widened exactly)."""
    return t.float().cpu().numpy().astype(np.float64)


def upload_quantized(packed: np.ndarray, scales: np.ndarray, biases: np.ndarray):
    return to_gpu_packed(packed), to_gpu_bf16_bits(scales), to_gpu_bf16_bits(biases)
