"""Pins of the oracle's FP8 KV-cache writer (CPU only).

The writer of the ops-transformer scatter_pa_kv_cache_with_k_scale page is
pinned against: the page's own worked example (tests/golden/page_constants.json,
"scatter_example"), an independent numpy formulation (assignment through a
reshaped slot-major view), the page's skip rule for out-of-range slots, and a
round trip through the decode oracle (a cache rebuilt by the writer decodes
bit-identically to the generated one).
"""
from __future__ import annotations

import json
import os
from dataclasses import replace

import numpy as np
import pytest
import torch

from fp8_paged_kv_amd import synth

GOLDEN = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "page_constants.json")))


def _codes(rng, shape):
    return rng.integers(1, 127, size=shape, dtype=np.uint8)      # never 0: untouched bytes stay 0


def test_page_worked_example(oracle_mod):
    ex = GOLDEN["scatter_example"]
    T, H, dk, dv = ex["num_tokens"], ex["num_head"], ex["k_head_size"], ex["v_head_size"]
    nb, bs = ex["num_blocks"], ex["block_size"]
    rng = np.random.default_rng(0)
    key, value = _codes(rng, (T, H, dk)), _codes(rng, (T, H, dv))
    ks = (np.arange(T * H, dtype=np.float32).reshape(T, H) + 1.0) / 64.0
    kc = np.zeros((nb, H, bs, dk), np.uint8)
    vc = np.zeros((nb, H, bs, dv), np.uint8)
    ksc = np.zeros((nb, H, bs, 1), np.float32)
    r = oracle_mod.scatter_kv_cache(key, value, kc, vc, np.array(ex["slot_mapping"], np.int32), ks, ksc,
                                    ex["cache_layout"])
    assert r["written"] == T
    seen = np.zeros((nb, bs), bool)
    for i, (blk, off) in enumerate(ex["block_offset"]):
        seen[blk, off] = True
        for j in range(H):
            assert np.array_equal(r["key_cache"][blk, j, off], key[i, j])
            assert np.array_equal(r["value_cache"][blk, j, off], value[i, j])
            assert r["key_scale_cache"].reshape(nb, H, bs)[blk, j, off] == ks[i, j]
    # nothing else was touched
    untouched = ~seen
    assert not r["key_cache"].transpose(0, 2, 1, 3)[untouched].any()
    assert not r["value_cache"].transpose(0, 2, 1, 3)[untouched].any()
    assert not r["key_scale_cache"].reshape(nb, H, bs).transpose(0, 2, 1)[untouched].any()


def _numpy_scatter(key, value, ks, kc, vc, ksc, slots, layout):
    """Independent form: bring the caches to slot-major order, assign rows by
    fancy indexing, and bring them back."""
    if layout == "BNBD":
        kc, vc, ksc = kc.transpose(0, 2, 1, 3), vc.transpose(0, 2, 1, 3), ksc.transpose(0, 2, 1)
    nb, bs, H, dk = kc.shape
    kf = np.ascontiguousarray(kc).reshape(nb * bs, H, dk).copy()
    vf = np.ascontiguousarray(vc).reshape(nb * bs, H, -1).copy()
    sf = np.ascontiguousarray(ksc).reshape(nb * bs, H).copy()
    ok = (slots >= 0) & (slots < nb * bs)
    kf[slots[ok]] = key[ok]
    vf[slots[ok]] = value[ok]
    sf[slots[ok]] = ks[ok]
    kf, vf, sf = kf.reshape(nb, bs, H, dk), vf.reshape(nb, bs, H, -1), sf.reshape(nb, bs, H)
    if layout == "BNBD":
        kf, vf, sf = kf.transpose(0, 2, 1, 3), vf.transpose(0, 2, 1, 3), sf.transpose(0, 2, 1)
    return np.ascontiguousarray(kf), np.ascontiguousarray(vf), np.ascontiguousarray(sf), int(ok.sum())


@pytest.mark.parametrize("layout", ["BSND", "BNBD"])
@pytest.mark.parametrize("shape", [(37, 3, 128, 128, 2, 128, 32), (200, 8, 64, 192, 3, 128, 64),
                                   (5, 1, 16, 16, 1, 16, 64)])
def test_matches_slot_major_assignment(oracle_mod, layout, shape):
    T, H, dk, dv, nb, bs, bits = shape
    cfg = synth.ScatterConfig("pin", num_tokens=T, num_head=H, k_head_size=dk, v_head_size=dv,
                              num_blocks=nb, block_size=bs, layout=layout, slot_bits=bits,
                              skip=min(4, T // 2), seed=3)
    inp = synth.make_scatter_inputs(cfg)
    n = lambda t: t.numpy()
    r = oracle_mod.scatter_kv_cache(inp["key"], inp["value"], inp["key_cache"], inp["value_cache"],
                                    inp["slot_mapping"], inp["key_scale"], inp["key_scale_cache"], layout)
    ek, ev, es, cnt = _numpy_scatter(n(inp["key"]), n(inp["value"]), n(inp["key_scale"]), n(inp["key_cache"]),
                                     n(inp["value_cache"]), n(inp["key_scale_cache"]),
                                     n(inp["slot_mapping"]).astype(np.int64), layout)
    assert r["written"] == cnt == T - min(4, T // 2)
    assert np.array_equal(r["key_cache"], ek)
    assert np.array_equal(r["value_cache"], ev)
    assert np.array_equal(r["key_scale_cache"].view(np.uint32), es.view(np.uint32))


def test_out_of_range_slots_are_skipped(oracle_mod):
    nb, bs, H = 2, 16, 2
    rng = np.random.default_rng(1)
    slots = np.array([-1, 0, nb * bs - 1, nb * bs, nb * bs + 100, -(2 ** 40), 2 ** 40], np.int64)
    T = len(slots)
    key, value = _codes(rng, (T, H, 16)), _codes(rng, (T, H, 16))
    ks = rng.random((T, H), dtype=np.float32)
    kc = np.zeros((nb, bs, H, 16), np.uint8)
    r = oracle_mod.scatter_kv_cache(key, value, kc, kc.copy(), slots, ks, np.zeros((nb, bs, H), np.float32))
    assert r["written"] == 2
    flat = r["key_cache"].reshape(nb * bs, H, 16)
    assert np.array_equal(flat[0], key[1]) and np.array_equal(flat[nb * bs - 1], key[2])
    assert not flat[1:nb * bs - 1].any()


def test_writer_rebuilds_the_decode_cache(oracle_mod):
    """Per-token rows written at the prefill slots of a workload reproduce the
    pool positions its decode reads: the decode oracle on the rebuilt cache is
    bit-identical to the decode on the generated one."""
    cfg = replace(synth.CONFIGS[0], seed=5)
    inp = synth.make_gqa_inputs(cfg)
    pre = synth.prefill_slots(cfg)
    assert torch.equal(pre["block_table"], inp["block_table"])
    slots = pre["slots"].to(torch.int64)
    nkv, D = cfg.nkv, cfg.D
    kflat = inp["k_cache"].reshape(-1, nkv, D)
    vflat = inp["v_cache"].reshape(-1, nkv, D)
    sflat = inp["k_scale"].reshape(-1, nkv)
    key, value, ks = kflat[slots], vflat[slots], sflat[slots]      # the rows as a producer would emit them
    # start from garbage everywhere; only the written positions are ever read
    g = torch.Generator().manual_seed(9)
    kc0 = torch.randint(0, 256, inp["k_cache"].shape, generator=g, dtype=torch.int32).to(torch.uint8)
    vc0 = torch.randint(0, 256, inp["v_cache"].shape, generator=g, dtype=torch.int32).to(torch.uint8)
    sc0 = torch.full(inp["k_scale"].shape, float("nan"))
    r = oracle_mod.scatter_kv_cache(key, value, kc0, vc0, pre["slots"], ks, sc0, "BSND")
    assert r["written"] == len(slots)
    rebuilt = dict(inp, k_cache=torch.from_numpy(r["key_cache"]), v_cache=torch.from_numpy(r["value_cache"]),
                   k_scale=torch.from_numpy(r["key_scale_cache"]))
    a = oracle_mod.gqa_decode(inp)["out_bf16"]
    b = oracle_mod.gqa_decode(rebuilt)["out_bf16"]
    assert np.array_equal(a, b)
