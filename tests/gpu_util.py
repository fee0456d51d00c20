"""Helpers of the GPU parity tests (test code only)."""
from __future__ import annotations

import numpy as np
import torch

# Tolerance on the BF16 output, GPU vs the oracle's BF16 output:
#   every element |d| <= 2e-2 + one bf16 ulp of the reference value, and
#   mean |d| <= 2e-3.
# Both sides end with one round-to-nearest cast to bf16; when their unrounded
# values straddle a rounding boundary the results differ by one ulp however
# close they were, and for |out| >= 4 one ulp (>= 2^-5) already exceeds 2e-2.
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


def bf16_ulp(x: np.ndarray) -> np.ndarray:
    """Spacing of bf16 values at |x| (normal range)."""
    a = np.maximum(np.abs(x), 2.0 ** -126)
    return 2.0 ** (np.floor(np.log2(a)) - 7)


def compare(gpu: np.ndarray, ref_bf16_bits: np.ndarray, what: str = ""):
    ref = bf16_bits_to_float(ref_bf16_bits).reshape(gpu.shape)
    assert np.isfinite(gpu).all(), f"{what}: non-finite GPU output"
    d = np.abs(gpu - ref)
    if d.size == 0:
        return 0.0, 0.0
    mx, mean = float(d.max()), float(d.mean())
    i = np.unravel_index(np.argmax(d), d.shape)
    ulps = d / bf16_ulp(ref)
    msg = (f"{what}: max|d|={mx:.3g} at {tuple(int(v) for v in i)} gpu={gpu[i]:.6g} ref={ref[i]:.6g} "
           f"({float(ulps[i]):.2f} bf16 ulp); max ulps={float(ulps.max()):.2f} mean|d|={mean:.3g}")
    print(msg, flush=True)
    over = d - (MAX_ABS + bf16_ulp(ref))
    assert float(over.max()) <= 0.0 and mean <= MEAN_ABS, msg
    return mx, mean
