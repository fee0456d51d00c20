"""Host-side checks of two arithmetic shortcuts the decode kernels rely on,
emulated in IEEE float32 with numpy (CPU only).

* small integer quotients: floor(x / d) == trunc((x + 0.5) * RN(1 / d)) for
  0 <= x < 4096 and 1 <= d <= 1024 (the kernels' ranges: rows and groups <= 32,
  batch x group indices < 1024);
* step 1's query codes: RN(q / s) == q0 + RN(q - s q0) * y, y = RN(1 / s),
  q0 = RN(q y), for every bf16 value q and scales s in [2^-60, 2^60]
  (Markstein's correction), whenever the quotient's magnitude is below 2048
  and the residual is a normal number (|q| >= 2^-100); for smaller |q| both
  quotients are far below E4M3's smallest code, so the codes agree (zero).
  numpy has no fused multiply-add, so the residual q - s q0 is formed exactly
  in float64 (a product of two floats is exact there) and rounded once.
"""
from __future__ import annotations

import numpy as np


def test_small_int_division_by_reciprocal():
    x = np.arange(4096, dtype=np.int64)
    for d in range(1, 1025):
        inv = np.float32(1.0) / np.float32(d)
        got = ((x.astype(np.float32) + np.float32(0.5)) * inv).astype(np.int64)
        assert np.array_equal(got, x // d), d


def _bf16_values():
    bits = np.arange(1 << 16, dtype=np.uint32) << 16
    v = bits.view(np.float32)
    return v[np.isfinite(v)]


def test_corrected_reciprocal_quotient_is_correctly_rounded():
    np.seterr(over="ignore", invalid="ignore", under="ignore")
    q = _bf16_values()
    rng = np.random.default_rng(5)
    mant = np.float32(1.0) + rng.random(600).astype(np.float32)
    expo = rng.integers(-60, 61, 600)
    scales = np.ldexp(mant, expo).astype(np.float32)
    scales[::5] = np.ldexp(np.float32(1.0), expo[::5]).astype(np.float32)
    for s in scales:
        y = np.float32(1.0) / s
        q0 = q * y                                             # RN(q y) in float32
        resid = (q.astype(np.float64) - np.float64(s) * q0.astype(np.float64)).astype(np.float32)
        fast = (q0.astype(np.float64) + resid.astype(np.float64) * np.float64(y)).astype(np.float32)
        ref = q / s                                            # IEEE float32 division
        corr = (q0 != 0) & (np.abs(q0) < 2048)
        use = corr & (np.abs(q) >= np.float32(2.0 ** -100))
        assert np.array_equal(fast[use].view(np.uint32), ref[use].view(np.uint32)), s
        tiny = corr & ~use
        assert np.all(np.abs(fast[tiny]) < 2.0 ** -40) and np.all(np.abs(ref[tiny]) < 2.0 ** -40), s
