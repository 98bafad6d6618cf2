"""Helpers for GPU parity tests: moving seeded inputs to the device and the
error metric max|x - ref| / max|ref| used throughout."""
import numpy as np
import torch

from workloads import bf16_bits_to_f32


def to_dev(a: np.ndarray, dev="cuda"):
    """uint16 (bf16 bits) -> bf16 tensor; float32 -> float32 tensor."""
    if a.dtype == np.uint16:
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(dev).view(torch.bfloat16)
    return torch.from_numpy(np.ascontiguousarray(a)).to(dev)


def to_host(t: torch.Tensor) -> np.ndarray:
    """bf16 tensor -> uint16 bits; float32 -> float32."""
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).cpu().numpy().view(np.uint16)
    return t.cpu().numpy()


def as_f64(a: np.ndarray) -> np.ndarray:
    if a.dtype == np.uint16:
        return bf16_bits_to_f32(a).astype(np.float64)
    return a.astype(np.float64)


def eps(x, ref) -> float:
    x = as_f64(np.asarray(x)) if np.asarray(x).dtype == np.uint16 else np.asarray(x, np.float64)
    ref = np.asarray(ref, np.float64)
    den = float(np.max(np.abs(ref)))
    num = float(np.max(np.abs(x - ref)))
    if not np.isfinite(num):
        return float("inf")
    return num / den if den > 0 else num


def stats_eps(stats: np.ndarray) -> float:
    """Global eps from per-head (max |diff|, max |ref|) oracle statistics."""
    return float(np.max(stats[:, 0]) / np.max(stats[:, 1]))
