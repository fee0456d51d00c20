"""pa_fp8_decode_noalloc (the library's static scratch instead of a caller's
workspace) against pa_fp8_decode on the same inputs, through the C ABI: two
calls in a row, the second on a smaller input, on the whole-row path and on
the per-head path with split sequences (whose arrival counters live in the
scratch).  Results must be bit-identical to the workspace entry point and
within the parity bar of the oracle."""
from __future__ import annotations

from dataclasses import replace

import numpy as np
import pytest
import torch

from fp8_paged_kv_amd import synth
from tests.gpu_util import compare, gpu_out_float, to_device

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def B():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from fp8_paged_kv_amd import binding
    binding.lib()
    return binding


@pytest.mark.parametrize("num_splits", [0, 3])
def test_noalloc_matches_decode_two_calls(B, oracle_mod, num_splits):
    full = synth.CONFIGS[1]
    big_cfg = replace(full, name="noalloc-big", B=12, num_blocks=12 * full.max_blocks_per_seq, seed=61)
    big = synth.make_gqa_inputs(big_cfg)
    small = synth.make_gqa_inputs(synth.CONFIGS[0])
    refs = {"big": oracle_mod.gqa_decode(big), "small": oracle_mod.gqa_decode(small)}
    dev = {"big": to_device(big), "small": to_device(small)}
    with_ws = {}
    for name in ("big", "small"):
        print(f"[gpu] decode with workspace, {name}, splits={num_splits}", flush=True)
        with_ws[name] = gpu_out_float(B.decode_inputs(dev[name], num_splits=num_splits))
    outs = {name: torch.empty_like(dev[name]["q"]) for name in ("big", "small")}
    for name in ("big", "small"):             # back to back: the second call reuses the scratch
        print(f"[gpu] decode_noalloc, {name}, splits={num_splits}", flush=True)
        B.decode_noalloc_inputs(dev[name], num_splits=num_splits, out=outs[name])
    torch.cuda.synchronize()
    for name in ("big", "small"):
        got = gpu_out_float(outs[name])
        assert np.array_equal(got, with_ws[name]), f"{name}: noalloc differs from the workspace entry point"
        compare(got, refs[name], f"noalloc {name} splits={num_splits}")
