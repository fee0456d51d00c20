"""Helpers of the GPU parity tests (test code only)."""
from __future__ import annotations

import numpy as np
import torch

# Tolerance on the BF16 output, GPU vs the oracle's unrounded FP64 output:
#   every element |gpu - ref| <= 2e-2 + half a bf16 ulp of the GPU value, and
#   mean |gpu - ref| <= 2e-3 over the compared output.
# The GPU value is bf16(x) for its own FP32 result x; the half ulp is that
# final rounding (ulp(bf16(x)) >= ulp(x), so half of it bounds the rounding
# error), and 2e-2 bounds |x - ref|.
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
    """Spacing of bf16 values at |x| (normal range; the subnormal spacing below it)."""
    a = np.maximum(np.abs(x), 2.0 ** -126)
    return 2.0 ** (np.floor(np.log2(a)) - 7)


ULP_FLOOR = 2.0 ** -4


def parity_stats(gpu: np.ndarray, ref: dict) -> dict:
    """Error statistics of a GPU bf16 output against the oracle result ``ref``
    (a dict with the FP64 ``out`` and its bf16 rounding ``out_bf16``):
    max/mean |gpu - out|, the largest excess over the per-element bound, and
    how many bf16 ulps the GPU value lies from the oracle's own bf16 value --
    ulps of max(|ref|, 1/16), so that values near zero (whose ulp is tiny
    while their error is the absolute error of the sum) are measured on the
    scale of the output rather than their own."""
    exact = np.asarray(ref["out"], dtype=np.float64).reshape(gpu.shape)
    ref_bf = bf16_bits_to_float(np.asarray(ref["out_bf16"])).reshape(gpu.shape)
    d = np.abs(gpu - exact)
    bound = MAX_ABS + 0.5 * bf16_ulp(gpu)
    ulps = np.abs(gpu - ref_bf) / bf16_ulp(np.maximum(np.abs(ref_bf), ULP_FLOOR))
    i = np.unravel_index(int(np.argmax(d)), d.shape) if d.size else ()
    return dict(n=int(d.size), max_abs=float(d.max()) if d.size else 0.0, mean_abs=float(d.mean()) if d.size else 0.0,
                excess=float((d - bound).max()) if d.size else -1.0, max_ulps=float(ulps.max()) if d.size else 0.0,
                frac_bit_equal=float((ulps == 0).mean()) if d.size else 1.0,
                frac_within_1ulp=float((ulps <= 1).mean()) if d.size else 1.0,
                at=tuple(int(v) for v in i), gpu_at=float(gpu[i]) if d.size else 0.0,
                ref_at=float(exact[i]) if d.size else 0.0)


def compare(gpu: np.ndarray, ref: dict, what: str = "", max_ulps: float = None):
    """Assert the parity bar of a GPU bf16 output against the oracle (see the
    constants above); ``max_ulps`` adds a regression gate on the distance in
    bf16 ulps from the oracle's own bf16 output.  Returns the statistics."""
    assert np.isfinite(gpu).all(), f"{what}: non-finite GPU output"
    st = parity_stats(gpu, ref)
    msg = (f"[parity] {what}: n={st['n']} max|d|={st['max_abs']:.4g} at {st['at']} gpu={st['gpu_at']:.6g} "
           f"ref={st['ref_at']:.6g} mean|d|={st['mean_abs']:.4g} max_ulps={st['max_ulps']:.0f} "
           f"bit_equal={st['frac_bit_equal']:.4f} within_1ulp={st['frac_within_1ulp']:.5f}")
    print(msg, flush=True)
    assert st["excess"] <= 0.0, msg
    assert st["mean_abs"] <= MEAN_ABS, msg
    if max_ulps is not None:
        assert st["max_ulps"] <= max_ulps, f"{msg} (gate {max_ulps} ulps)"
    return st
