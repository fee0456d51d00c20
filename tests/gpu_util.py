"""Helpers of the GPU parity tests (test code only)."""
from __future__ import annotations

import numpy as np
import torch

# Tolerance on the BF16 output, GPU vs oracle: max |d| <= 2e-2 and mean |d| <= 2e-3.
MAX_ABS = 2e-2
MEAN_ABS = 2e-3


def to_device(inp: dict, device="cuda") -> dict:
    out = {}
    for k, v in inp.items():
        out[k] = v.to(device) if isinstance(v, torch.Tensor) else v
    return out


def to_host(inp: dict) -> dict:
    out = {}
    for k, v in inp.items():
        out[k] = v.cpu() if isinstance(v, torch.Tensor) else v
    return out


def bf16_bits_to_float(bits: np.ndarray) -> np.ndarray:
    return (bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def gpu_out_float(out: torch.Tensor) -> np.ndarray:
    return out.float().cpu().double().numpy()


def compare(gpu: np.ndarray, ref_bf16_bits: np.ndarray, what: str = ""):
    ref = bf16_bits_to_float(ref_bf16_bits).reshape(gpu.shape)
    assert np.isfinite(gpu).all(), f"{what}: non-finite GPU output"
    d = np.abs(gpu - ref)
    mx, mean = float(d.max()) if d.size else 0.0, float(d.mean()) if d.size else 0.0
    assert mx <= MAX_ABS and mean <= MEAN_ABS, f"{what}: max|d|={mx:.3g} mean|d|={mean:.3g}"
    return mx, mean
