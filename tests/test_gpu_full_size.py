"""Full-size parity: every output element of the five workloads, in the launch
configuration the benchmark times, against the CPU oracle (through the C ABI).

Also the six shapes of the GLM-4.5 page's own test list (section
测试用例与精度校验: (b, s1, s2, nq, nkv) = (1, 2, 2048, 48, 8),
(16, 1, 8195, 12, 2), (16, 1, 8192, 12, 1), (16, 1, 8192, 12, 2),
(2, 1, 1024, 12, 1), (16, 1, 256, 16, 4), every sequence s2 tokens long,
b * ceil(s2 / 128) blocks in a randomly permuted pool), and the in-kernel
gather / query-code dumps at full size.

Every test prints the case it runs before touching the GPU.
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

from fp8_paged_kv_amd import synth
from tests.gpu_util import compare, gpu_out_float, to_device, to_host

pytestmark = pytest.mark.gpu

_cache = {}


@pytest.fixture(scope="module")
def B():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from fp8_paged_kv_amd import binding
    binding.lib()
    return binding


def _inputs(cfg_id, causal=False):
    """Device inputs of a full-size workload, their host copy and the oracle's
    result over every output row (computed once per module)."""
    key = (cfg_id, causal)
    if key not in _cache:
        from oracle import oracle
        cfg = synth.CONFIGS[cfg_id]
        print(f"[gpu] full-size config {cfg_id} causal={causal}: generating on the GPU", flush=True)
        dev = synth.make_gqa_inputs(cfg, device="cuda")
        if causal:
            dev["causal"] = True
        host = to_host(dev)
        print(f"[cpu] oracle over all {cfg.B * cfg.s1 * cfg.nq} rows", flush=True)
        if cfg.B >= 16:
            ref = oracle.gqa_decode(host)
        else:       # few long sequences: spread the rows over the threads instead of the batches
            ref = oracle.gqa_decode_rows(host, np.arange(cfg.B * cfg.s1 * cfg.nq))
        _cache[key] = (dev, host, ref)
    return _cache[key]


def _decode(B, dev, tag, num_splits=0):
    print(f"[gpu] {tag} splits={num_splits}", flush=True)
    out = B.decode_inputs(dev, num_splits=num_splits)
    torch.cuda.synchronize()
    return gpu_out_float(out)


# Regression gates on the largest distance, in bf16 ulps, from the oracle's own bf16
# output (ulps of max(|ref|, 1/16)); about twice the level measured when they were set
# (config 1: 19, where a few outputs near zero sum outliers x20; config 2: 1; config 3
# and its causal variant: 4; the page shapes: 0; MLA: 1).
MAX_ULPS = {1: 40, 2: 4, 3: 8}


@pytest.mark.parametrize("cfg_id", [1, 2, 3])
def test_full_size_every_element(B, cfg_id):
    dev, _, ref = _inputs(cfg_id)
    cfg = synth.CONFIGS[cfg_id]
    got = _decode(B, dev, f"config{cfg_id} full").reshape(cfg.B * cfg.s1 * cfg.nq, cfg.D)
    compare(got, {"out": ref["out"].reshape(got.shape), "out_bf16": ref["out_bf16"].reshape(got.shape)},
            f"config{cfg_id} full, whole-row path", max_ulps=MAX_ULPS[cfg_id])


def test_full_size_config3_causal_every_element(B):
    dev, _, ref = _inputs(3, causal=True)
    got = _decode(B, dev, "config3 causal full")
    compare(got, ref, "config3 causal full", max_ulps=MAX_ULPS[3])


def test_full_size_config1_dumps_bit_exact(B):
    """Whole-row path at full size: the physical row gathered for every
    logical token and the FP8 query codes equal the oracle's."""
    dev, _, ref = _inputs(1)
    cfg = synth.CONFIGS[1]
    print("[gpu] config1 full debug dumps, whole-row path", flush=True)
    out, rows, q8 = B.decode_debug(dev["q"], dev["q_scale"], dev["k_cache"], dev["k_scale"], dev["v_cache"],
                                   dev["v_scale"], dev["block_table"], dev["kv_act_seqs"], dev["softmax_scale"],
                                   cfg.s2_tile)
    torch.cuda.synchronize()
    assert np.array_equal(rows.cpu().numpy(), ref["rows"])
    assert np.array_equal(q8.cpu().numpy(), ref["q8"])
    compare(gpu_out_float(out), ref, "config1 full debug", max_ulps=MAX_ULPS[1])


@pytest.mark.parametrize("num_splits", [1, 4])
def test_full_size_config1_per_head_path(B, num_splits):
    """The per-head path (explicit split count) on the full config-1 workload:
    every output element, and the gather and query-code dumps bit-exact."""
    dev, _, ref = _inputs(1)
    cfg = synth.CONFIGS[1]
    got = _decode(B, dev, "config1 full per-head", num_splits)
    compare(got, ref, f"config1 full per-head splits={num_splits}", max_ulps=MAX_ULPS[1])
    print(f"[gpu] config1 full debug dumps, per-head path, splits={num_splits}", flush=True)
    _, rows, q8 = B.decode_debug(dev["q"], dev["q_scale"], dev["k_cache"], dev["k_scale"], dev["v_cache"],
                                 dev["v_scale"], dev["block_table"], dev["kv_act_seqs"], dev["softmax_scale"],
                                 cfg.s2_tile, num_splits=num_splits)
    torch.cuda.synchronize()
    assert np.array_equal(rows.cpu().numpy(), ref["rows"])
    assert np.array_equal(q8.cpu().numpy(), ref["q8"])


# The page's six test shapes; its s2_tile rule ("1024 for long s2, else 128")
# lost its comparator in the text, so both tiles run on every shape.
PAGE_SHAPES = [(1, 2, 2048, 48, 8), (16, 1, 8195, 12, 2), (16, 1, 8192, 12, 1), (16, 1, 8192, 12, 2),
               (2, 1, 1024, 12, 1), (16, 1, 256, 16, 4)]


@pytest.mark.parametrize("shape", PAGE_SHAPES, ids=lambda s: "b{}_s1_{}_s2_{}_nq{}_nkv{}".format(*s))
@pytest.mark.parametrize("s2_tile", [128, 1024])
def test_page_test_shapes(B, oracle_mod, shape, s2_tile):
    b, s1, s2, nq, nkv = shape
    mb = (s2 + 127) // 128
    cfg = synth.GqaConfig(f"page-b{b}-s1{s1}-s2{s2}-nq{nq}-nkv{nkv}", B=b, s1=s1, nq=nq, nkv=nkv,
                          seq_lens=(s2,) * b, s2_tile=s2_tile, num_blocks=b * mb, max_blocks_per_seq=mb,
                          seed=PAGE_SHAPES.index(shape) + 50)
    inp = synth.make_gqa_inputs(cfg)
    ref = oracle_mod.gqa_decode(inp)
    d = to_device(inp)
    for ns in (0, 1):
        print(f"[gpu] page shape {shape} s2_tile={s2_tile} splits={ns}", flush=True)
        out = B.decode_inputs(d, num_splits=ns)
        torch.cuda.synchronize()
        compare(gpu_out_float(out), ref, f"page shape {shape} s2_tile={s2_tile} splits={ns}", max_ulps=2)


@pytest.fixture(scope="module")
def mla_full():
    from oracle import oracle
    cfg = synth.CONFIGS[4]
    inp = synth.make_mla_inputs(cfg)
    print("[cpu] MLA oracle over all 16 batches", flush=True)
    return inp, oracle.mla_decode(inp)


def test_full_size_mla_every_element(B, mla_full):
    inp, ref = mla_full
    print("[gpu] mla config4 full, packed rows", flush=True)
    out = B.mla_decode_inputs(to_device(inp))
    torch.cuda.synchronize()
    compare(gpu_out_float(out), ref, "mla config4 full, packed rows", max_ulps=4)


def test_full_size_mla_kv_split_every_element(B, mla_full):
    inp, ref = mla_full
    print("[gpu] mla config4 full, kv_split", flush=True)
    out = B.mla_decode_kv_split_inputs(to_device(synth.mla_kv_split(inp)))
    torch.cuda.synchronize()
    compare(gpu_out_float(out), ref, "mla config4 full, kv_split", max_ulps=4)
