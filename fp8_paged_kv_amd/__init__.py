"""FP8 paged-attention decode for MI355X (gfx950).

The decode runs in hand-written HIP kernels behind a C ABI
(include/pa_fp8.h, built into libpa_fp8.so); ``binding`` marshals torch
tensors into it and ``synth`` draws seeded synthetic inputs.
"""
from . import synth  # noqa: F401

__all__ = ["synth", "binding", "build"]
