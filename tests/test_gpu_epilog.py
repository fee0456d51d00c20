"""GPU parity of KvCompressEpilog modes 0/1 (pa_fp8_kv_compress_epilog) against
the oracle: bit-exact cache bytes.  Every test prints its case first."""
from __future__ import annotations

import json
import os

import numpy as np
import pytest
import torch

from fp8_paged_kv_amd import synth

pytestmark = pytest.mark.gpu

GOLDEN = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "page_constants.json")))


@pytest.fixture(scope="module")
def B():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from fp8_paged_kv_amd import binding
    binding.lib()
    return binding


def _check(B, oracle_mod, inp, tag):
    c = inp["cfg"]
    print(f"[gpu] epilog {tag}: T={c.num_tokens} d={c.d} mode={c.quant_mode} round={c.round_scale} "
          f"blocks={c.block_num}x{c.block_size} head_dim={c.head_dim} pad={c.block_pad} int{c.slot_bits} "
          f"skip={c.skip}", flush=True)
    ref = oracle_mod.kv_compress_epilog(inp["cache"], inp["x"], inp["slot_mapping"], c.quant_mode, c.round_scale,
                                        block_stride=(c.block_num, c.block_size, c.head_dim, inp["block_stride"]))
    d = {k: (v.cuda() if isinstance(v, torch.Tensor) else v) for k, v in inp.items()}
    B.epilog_inputs(d)
    torch.cuda.synchronize()
    got = d["cache"].cpu().numpy()
    if not np.array_equal(got, ref["cache"]):
        bad = np.flatnonzero(got != ref["cache"])
        raise AssertionError(f"{tag}: {bad.size} bytes differ, first at {bad[:8].tolist()}")


@pytest.mark.parametrize("mode,round_scale", [(0, True), (1, True), (1, False)])
@pytest.mark.parametrize("bits", [32, 64])
@pytest.mark.parametrize("shape", [
    (37, 256, 5, 16, None, 0, 4),      # head_dim = the page's 323 in mode 1: rows at odd addresses
    (64, 512, 4, 32, None, 40, 0),     # 583 in mode 1; blocks with padding between them
    (9, 128, 2, 8, 416, 0, 2),         # smallest d (one nope group)
    (6, 8192, 2, 4, 8576, 0, 1),       # largest d: 127 groups, 16 chunks of 512 columns
    (300, 576, 8, 64, 704, 0, 20),     # the MLA latent width (512 nope + 64 rope)
    (37, 256, 5, 16, 357, 0, 4),       # odd head_dim in both modes: every row alignment mod 8
    (50, 128, 4, 16, 227, 3, 5),       # odd head_dim and an odd gap between blocks; one scale piece
])
def test_epilog_parity(B, oracle_mod, mode, round_scale, bits, shape):
    T, d, nb, bs, hd, pad, skip = shape
    if hd is None:
        hd = oracle_mod.kv_compress_cache_col(d, mode)
    cfg = synth.EpilogConfig("ep", num_tokens=T, d=d, block_num=nb, block_size=bs, head_dim=hd, quant_mode=mode,
                             round_scale=round_scale, slot_bits=bits, skip=skip, block_pad=pad, seed=T + d + mode)
    _check(B, oracle_mod, synth.make_epilog_inputs(cfg), f"parity {shape}")


def test_epilog_page_example_shapes(B, oracle_mod):
    ex = GOLDEN["kv_compress_cache_col"]["example_call"]
    nb, bs, _, hd = ex["cache_shape"]
    T, d = ex["x_shape"]
    cfg = synth.EpilogConfig("page-example", num_tokens=T, d=d, block_num=nb, block_size=bs, head_dim=hd,
                             quant_mode=ex["quant_mode"], round_scale=ex["round_scale"], seed=3)
    _check(B, oracle_mod, synth.make_epilog_inputs(cfg), "page example")


def test_epilog_full_size(B, oracle_mod):
    """The benchmark's workload: 131072 MLA-latent rows (d = 576), mode 1."""
    cfg = synth.EpilogConfig("epilog-bench", num_tokens=131072, d=576, block_num=1024, block_size=128,
                             head_dim=649, quant_mode=1, round_scale=True, seed=9)
    _check(B, oracle_mod, synth.make_epilog_inputs(cfg), "full size")


@pytest.mark.parametrize("mode,round_scale", [(0, True), (1, True), (1, False)])
def test_epilog_extreme_group_magnitudes(B, oracle_mod, mode, round_scale):
    """Groups whose maxima sit at the ends of the bf16 range: at 2^-120 the fp32
    scale is subnormal, the e8m0 exponent reaches its clamp at -127 and many
    inputs are bf16 subnormals; at 2^126 the exponent reaches 119-120."""
    d = 320
    cfg = synth.EpilogConfig("extreme", num_tokens=16, d=d, block_num=2, block_size=16,
                             head_dim=oracle_mod.kv_compress_cache_col(d, mode), quant_mode=mode,
                             round_scale=round_scale, seed=5)
    inp = synth.make_epilog_inputs(cfg)
    x = inp["x"].double()
    gains = [2.0 ** -120, 2.0 ** -100, 2.0 ** 100, 2.0 ** 126, 1.0]
    for t in range(cfg.num_tokens):
        for g in range(4):
            grp = x[t, 64 * g:64 * g + 64]
            amax = float(grp.abs().max())
            if amax > 0:
                x[t, 64 * g:64 * g + 64] = grp / amax * gains[(t + g) % len(gains)]
    inp["x"] = x.to(torch.bfloat16)
    _check(B, oracle_mod, inp, f"extreme magnitudes mode={mode} round={round_scale}")
