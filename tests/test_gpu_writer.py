"""GPU parity of the FP8 KV-cache writer (pa_fp8_scatter_kv_cache) against the
oracle's writer: bit-exact caches.  Every test prints its case first."""
from __future__ import annotations

import json
import os
from dataclasses import replace

import numpy as np
import pytest
import torch

from fp8_paged_kv_amd import synth
from tests.gpu_util import compare, gpu_out_float, to_device

pytestmark = pytest.mark.gpu

GOLDEN = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "page_constants.json")))


@pytest.fixture(scope="module")
def B():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from fp8_paged_kv_amd import binding
    binding.lib()
    return binding


def _check_against_oracle(B, oracle_mod, inp, tag):
    cfg = inp["cfg"]
    print(f"[gpu] writer {tag}: T={cfg.num_tokens} H={cfg.num_head} dk={cfg.k_head_size} dv={cfg.v_head_size} "
          f"nb={cfg.num_blocks} bs={cfg.block_size} {cfg.layout} int{cfg.slot_bits} skip={cfg.skip}", flush=True)
    ref = oracle_mod.scatter_kv_cache(inp["key"], inp["value"], inp["key_cache"], inp["value_cache"],
                                      inp["slot_mapping"], inp["key_scale"], inp["key_scale_cache"], cfg.layout)
    d = to_device(inp)
    B.scatter_inputs(d)
    torch.cuda.synchronize()
    assert np.array_equal(d["key_cache"].cpu().numpy(), ref["key_cache"]), tag
    assert np.array_equal(d["value_cache"].cpu().numpy(), ref["value_cache"]), tag
    assert np.array_equal(d["key_scale_cache"].cpu().numpy().view(np.uint32),
                          ref["key_scale_cache"].view(np.uint32)), tag


@pytest.mark.parametrize("layout", ["BSND", "BNBD"])
@pytest.mark.parametrize("bits", [32, 64])
@pytest.mark.parametrize("shape", [
    (1, 8, 128, 128, 1, 128, 0),        # one token (a decode step of one sequence)
    (33, 8, 128, 128, 2, 128, 5),       # odd token count, skipped slots
    (257, 3, 64, 192, 5, 128, 9),       # odd heads, different key / value sizes
    (96, 1, 576, 512, 2, 64, 0),        # rows over 1 KB: several pieces per lane
    (500, 16, 128, 128, 4, 128, 17),    # 4 KB rows
])
def test_writer_parity(B, oracle_mod, layout, bits, shape):
    T, H, dk, dv, nb, bs, skip = shape
    cfg = synth.ScatterConfig("w", num_tokens=T, num_head=H, k_head_size=dk, v_head_size=dv, num_blocks=nb,
                              block_size=bs, layout=layout, slot_bits=bits, skip=skip, seed=T + H)
    _check_against_oracle(B, oracle_mod, synth.make_scatter_inputs(cfg), f"parity {shape}")


def test_writer_page_example(B, oracle_mod):
    ex = GOLDEN["scatter_example"]
    cfg = synth.ScatterConfig("page-example", num_tokens=ex["num_tokens"], num_head=ex["num_head"],
                              k_head_size=ex["k_head_size"], v_head_size=ex["v_head_size"],
                              num_blocks=ex["num_blocks"], block_size=ex["block_size"], layout=ex["cache_layout"])
    inp = synth.make_scatter_inputs(cfg)
    inp["slot_mapping"] = torch.tensor(ex["slot_mapping"], dtype=torch.int32)
    _check_against_oracle(B, oracle_mod, inp, "page example")


def test_writer_strided_inputs(B, oracle_mod):
    """Key / value rows taken from a wider per-token buffer and a transposed
    key-scale view: the strides are passed through, nothing is copied."""
    T, H, d = 70, 4, 128
    cfg = synth.ScatterConfig("strided", num_tokens=T, num_head=H, num_blocks=3, layout="BSND", skip=3, seed=5)
    inp = synth.make_scatter_inputs(cfg)
    print("[gpu] writer strided inputs", flush=True)
    ref = oracle_mod.scatter_kv_cache(inp["key"], inp["value"], inp["key_cache"], inp["value_cache"],
                                      inp["slot_mapping"], inp["key_scale"], inp["key_scale_cache"], "BSND")
    wide = torch.zeros((T, 3 * H * d), dtype=torch.uint8)
    wide[:, H * d:2 * H * d] = inp["key"].reshape(T, -1)
    wide[:, 2 * H * d:] = inp["value"].reshape(T, -1)
    wide = wide.cuda()
    key = wide[:, H * d:2 * H * d].view(T, H, d)
    value = wide[:, 2 * H * d:].view(T, H, d)
    ks = inp["key_scale"].t().contiguous().cuda().t()               # strides (1, T)
    kc, vc, ksc = inp["key_cache"].cuda(), inp["value_cache"].cuda(), inp["key_scale_cache"].cuda()
    B.scatter_kv_cache(key, value, kc, vc, inp["slot_mapping"].cuda(), ks, ksc, "BSND")
    torch.cuda.synchronize()
    assert np.array_equal(kc.cpu().numpy(), ref["key_cache"])
    assert np.array_equal(vc.cpu().numpy(), ref["value_cache"])
    assert np.array_equal(ksc.cpu().numpy().view(np.uint32), ref["key_scale_cache"].view(np.uint32))


def _gather_token_rows(inp, slots):
    nkv, D = inp["cfg"].nkv, inp["cfg"].D
    s = slots.to(torch.int64)
    return (inp["k_cache"].reshape(-1, nkv, D)[s], inp["v_cache"].reshape(-1, nkv, D)[s],
            inp["k_scale"].reshape(-1, nkv)[s])


def test_writer_then_decode(B, oracle_mod):
    """The GPU writer rebuilds a decode workload's pool from per-token rows; the
    GPU decode of that pool matches the oracle decode of the generated one and
    is bit-identical to the GPU decode of the generated pool."""
    cfg = replace(synth.CONFIGS[0], seed=6)
    inp = synth.make_gqa_inputs(cfg)
    pre = synth.prefill_slots(cfg)
    key, value, ks = _gather_token_rows(inp, pre["slots"])
    print(f"[gpu] writer then decode: {len(pre['slots'])} tokens", flush=True)
    d = to_device(inp)
    g = torch.Generator().manual_seed(3)
    kc = torch.randint(0, 256, inp["k_cache"].shape, generator=g, dtype=torch.int32).to(torch.uint8).cuda()
    vc = torch.randint(0, 256, inp["v_cache"].shape, generator=g, dtype=torch.int32).to(torch.uint8).cuda()
    sc = torch.full(inp["k_scale"].shape, float("nan"), device="cuda")
    B.scatter_kv_cache(key.cuda(), value.cuda(), kc, vc, pre["slots"].cuda(), ks.cuda(), sc, "BSND")
    rebuilt = dict(d, k_cache=kc, v_cache=vc, k_scale=sc)
    out_rebuilt = gpu_out_float(B.decode_inputs(rebuilt))
    out_direct = gpu_out_float(B.decode_inputs(d))
    torch.cuda.synchronize()
    assert np.array_equal(out_rebuilt, out_direct)
    compare(out_rebuilt, oracle_mod.gqa_decode(inp), "writer then decode")


def test_writer_full_size_prefill(B, oracle_mod):
    """The benchmark's workload: every token of the GLM-4.5-shaped decode
    workload (B=32, lengths 1k-8k, 8 KV heads) written into its 2048-block pool."""
    cfg = synth.CONFIGS[1]
    pre = synth.prefill_slots(cfg)
    T = len(pre["slots"])
    print(f"[gpu] writer full-size prefill: {T} tokens", flush=True)
    g = torch.Generator().manual_seed(11)
    key = torch.randint(0, 256, (T, cfg.nkv, cfg.D), generator=g, dtype=torch.int32).to(torch.uint8)
    value = torch.randint(0, 256, (T, cfg.nkv, cfg.D), generator=g, dtype=torch.int32).to(torch.uint8)
    ks = torch.rand((T, cfg.nkv), generator=g)
    shape = (cfg.num_blocks, cfg.block_size, cfg.nkv, cfg.D)
    kc0 = torch.zeros(shape, dtype=torch.uint8)
    ksc0 = torch.zeros(shape[:3])
    ref = oracle_mod.scatter_kv_cache(key, value, kc0, kc0, pre["slots"], ks, ksc0, "BSND")
    kc, vc, ksc = kc0.cuda(), kc0.clone().cuda(), ksc0.cuda()
    B.scatter_kv_cache(key.cuda(), value.cuda(), kc, vc, pre["slots"].cuda(), ks.cuda(), ksc, "BSND")
    torch.cuda.synchronize()
    assert ref["written"] == T
    assert np.array_equal(kc.cpu().numpy(), ref["key_cache"])
    assert np.array_equal(vc.cpu().numpy(), ref["value_cache"])
    assert np.array_equal(ksc.cpu().numpy().view(np.uint32), ref["key_scale_cache"].view(np.uint32))
