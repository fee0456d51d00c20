"""Pins of the oracle's KvCompressEpilog (quant modes 0 and 1), CPU only.

Against: the page's two worked cache-row sizes (tests/golden/page_constants.json,
"kv_compress_cache_col"); torch's own bf16 and float8_e4m3fn casts on the
page's formula; the defining properties of the scales (the e8m0 power of two
is the smallest one >= amax / 448 with roundScale, the largest one <= it
without); exact round trips for values that are E4M3 values times a power of
two; the dequantisation error bound; the row layout and the skip rule.
"""
from __future__ import annotations

import json
import os

import numpy as np
import pytest
import torch

from fp8_paged_kv_amd import synth

GOLDEN = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "page_constants.json")))


def _cfg(**kw):
    base = dict(name="ep", num_tokens=40, d=256, block_num=4, block_size=16, head_dim=384, quant_mode=1,
                round_scale=True, skip=3, seed=1)
    base.update(kw)
    return synth.EpilogConfig(**base)


def _run(oracle_mod, inp):
    c = inp["cfg"]
    r = oracle_mod.kv_compress_epilog(inp["cache"], inp["x"], inp["slot_mapping"], c.quant_mode, c.round_scale,
                                      block_stride=(c.block_num, c.block_size, c.head_dim, inp["block_stride"]))
    return r


def _rows(inp, cache):
    """slot -> the cache row bytes (head_dim of them), from the flat buffer."""
    c = inp["cfg"]
    out = {}
    for t, s in enumerate(inp["slot_mapping"].tolist()):
        if s < 0:
            continue
        base = (s // c.block_size) * inp["block_stride"] + (s % c.block_size) * c.head_dim
        out[t] = cache[base:base + c.head_dim]
    return out


def test_cache_col_page_values(oracle_mod):
    for d, mode, col in GOLDEN["kv_compress_cache_col"]["cases"]:
        assert oracle_mod.kv_compress_cache_col(d, mode) == col
    ex = GOLDEN["kv_compress_cache_col"]["example_call"]
    assert oracle_mod.kv_compress_cache_col(ex["x_shape"][1], ex["quant_mode"]) <= ex["cache_shape"][3]


def _decode_row(row, d, mode):
    nope, groups = d - 64, (d - 64) // 64
    rope = row[:128].view(np.uint16)
    codes = row[128:128 + nope]
    sc = row[128 + nope:128 + nope + groups * (2 if mode == 0 else 1)]
    if mode == 0:
        scales = torch.from_numpy(sc.view(np.int16).copy()).view(torch.bfloat16).double().numpy()
    else:
        scales = np.array([2.0 ** (int(b) - 127) for b in sc])
    vals = torch.from_numpy(codes.copy()).view(torch.float8_e4m3fn).double().numpy()
    return rope, codes, vals, scales


@pytest.mark.parametrize("mode,round_scale", [(0, True), (1, True), (1, False)])
def test_matches_torch_casts(oracle_mod, mode, round_scale):
    """amax, scale = amax/448 in fp32, the stored scale (torch's bf16 cast, or
    a power of two), the fp32 quotient and torch's saturated e4m3 cast."""
    inp = synth.make_epilog_inputs(_cfg(quant_mode=mode, round_scale=round_scale, d=320, head_dim=448,
                                        seed=2 + mode))
    r = _run(oracle_mod, inp)
    rows = _rows(inp, r["cache"])
    x = inp["x"].float().reshape(inp["x"].shape[0], -1, 64)[:, :-1]           # nope groups (last 64 = rope)
    amax = x.abs().amax(dim=-1)
    scale = amax / 448.0
    if mode == 0:
        used = scale.to(torch.bfloat16).float()
    else:
        used = torch.zeros_like(scale)
        for idx in np.ndindex(*scale.shape):
            s = float(scale[idx])
            if s > 0:
                k = int(np.ceil(np.log2(s))) if round_scale else int(np.floor(np.log2(s)))
                used[idx] = 2.0 ** max(-127, min(127, k))
    q = torch.where(used[..., None] > 0, x / torch.where(used > 0, used, 1.0)[..., None], torch.zeros_like(x))
    codes = q.clamp(-448, 448).to(torch.float8_e4m3fn).view(torch.uint8).reshape(x.shape[0], -1).numpy()
    for t, row in rows.items():
        assert np.array_equal(row[128:128 + 256], codes[t]), t
        if mode == 0:
            sb = used[t].to(torch.bfloat16).view(torch.int16).numpy().view(np.uint8)
            assert np.array_equal(row[384:384 + 8], sb)


@pytest.mark.parametrize("round_scale", [True, False])
def test_e8m0_scale_is_the_bracketing_power_of_two(oracle_mod, round_scale):
    inp = synth.make_epilog_inputs(_cfg(quant_mode=1, round_scale=round_scale, seed=7))
    r = _run(oracle_mod, inp)
    x = inp["x"].double().numpy()
    for t, row in _rows(inp, r["cache"]).items():
        _, _, vals, scales = _decode_row(row, 256, 1)
        for g in range(3):
            s = np.float32(np.abs(x[t, 64 * g:64 * g + 64]).max() / np.float32(448.0))
            if s == 0:
                assert row[128 + 192 + g] == 0
                continue
            if round_scale:
                assert scales[g] >= s and scales[g] / 2 < s
            else:
                assert scales[g] <= s and scales[g] * 2 > s


def test_exact_round_trip_for_representable_values(oracle_mod):
    """x = e4m3 value * 2^k with a group maximum of 448 * 2^k: the mode-1 scale is
    exactly 2^k and the codes give x back exactly."""
    rng = np.random.default_rng(4)
    T, d = 6, 192
    all_vals = torch.arange(256, dtype=torch.uint8).view(torch.float8_e4m3fn).double().numpy()
    finite = all_vals[np.isfinite(all_vals)]
    x = np.zeros((T, d))
    ks = rng.integers(-30, 30, size=(T, 2))
    for t in range(T):
        for g in range(2):
            v = rng.choice(finite, 64)
            v[rng.integers(64)] = 448.0 * rng.choice([-1, 1])
            x[t, 64 * g:64 * g + 64] = v * 2.0 ** ks[t, g]
        x[t, 128:] = rng.standard_normal(64)
    xb = torch.from_numpy(x).to(torch.bfloat16)
    assert torch.equal(xb.double(), torch.from_numpy(x)[:, :].to(torch.bfloat16).double())
    cache = np.zeros((1, 8, 1, 264), np.uint8)
    r = oracle_mod.kv_compress_epilog(cache, xb, np.arange(T, dtype=np.int32), 1, True)
    for t in range(T):
        row = r["cache"][0, t, 0]
        _, _, vals, scales = _decode_row(row, d, 1)
        assert np.array_equal(scales, 2.0 ** ks[t].astype(float))
        rec = vals.reshape(2, 64) * scales[:, None]
        assert np.array_equal(rec.reshape(-1), xb[t, :128].double().numpy())


@pytest.mark.parametrize("mode", [0, 1])
def test_dequantisation_error_bound(oracle_mod, mode):
    """|code * stored_scale - x| <= half an E4M3 quantum at the value (relative
    2^-4 for normal codes, absolute 2^-10 * scale in the subnormal range), and
    the group maximum lands in the top binade (mode 1: in [224, 448])."""
    inp = synth.make_epilog_inputs(_cfg(quant_mode=mode, seed=11))
    r = _run(oracle_mod, inp)
    x = inp["x"].double().numpy()
    for t, row in _rows(inp, r["cache"]).items():
        _, codes, vals, scales = _decode_row(row, 256, mode)
        for g in range(3):
            xg = x[t, 64 * g:64 * g + 64]
            if not np.abs(xg).max():
                assert not codes[64 * g:64 * g + 64].any()
                continue
            rec = vals[64 * g:64 * g + 64] * scales[g]
            q = np.abs(xg) / scales[g]
            quantum = np.where(q < 2.0 ** -6, 2.0 ** -9, 2.0 ** (np.floor(np.log2(np.maximum(q, 2.0 ** -6))) - 3))
            assert np.all(np.abs(rec - xg) <= 0.5 * quantum * scales[g] * (1 + 1e-6) + 1e-300)
            top = np.abs(vals[64 * g:64 * g + 64]).max()
            assert (top == 448.0) if mode == 0 else (224.0 <= top <= 448.0)


def test_rope_layout_padding_and_skips(oracle_mod):
    inp = synth.make_epilog_inputs(_cfg(quant_mode=0, skip=5, block_pad=48, seed=5))
    c = inp["cfg"]
    before = inp["cache"].numpy()
    r = _run(oracle_mod, inp)
    after = r["cache"]
    row_bytes = oracle_mod.kv_compress_row_bytes(c.d, 0)
    touched = np.zeros_like(before, dtype=bool)
    for t, s in enumerate(inp["slot_mapping"].tolist()):
        if s < 0:
            continue
        base = (s // c.block_size) * inp["block_stride"] + (s % c.block_size) * c.head_dim
        touched[base:base + row_bytes] = True
        rope = inp["x"][t, c.d - 64:].view(torch.int16).numpy().view(np.uint8)
        assert np.array_equal(after[base:base + 128], rope)
    assert r["written"] == c.num_tokens - 5
    assert np.array_equal(after[~touched], before[~touched])        # padding, skipped and unused rows
