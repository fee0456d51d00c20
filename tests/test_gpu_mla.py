"""GPU parity of the HIP MLA sparse decode against the CPU oracle (through the C ABI).

Every test prints the case it runs before touching the GPU.
"""
from __future__ import annotations

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


def _cfg(name, **kw):
    base = dict(name=name, B=2, s1=1, nq=32, topk=1024, seq_range=None, num_blocks=40,
                max_blocks_per_seq=16, s2_tile=512, seed=11, seq_lens=(700, 1500))
    base.update(kw)
    return synth.MlaConfig(**base)


def _run(B, inp_h, tag):
    cfg = inp_h["cfg"]
    print(f"[gpu] mla {tag} B={cfg.B} s1={cfg.s1} nq={cfg.nq} topk={cfg.topk} s2_tile={inp_h.get('s2_tile', cfg.s2_tile)} "
          f"seqs={inp_h['kv_act_seqs'].tolist()}", flush=True)
    out = B.mla_decode_inputs(to_device(inp_h))
    torch.cuda.synchronize()
    return out


@pytest.mark.parametrize("s2_tile", [128, 256, 512])
def test_mla_small_parity(B, oracle_mod, s2_tile):
    inp = synth.make_mla_inputs(_cfg(f"mla-t{s2_tile}", s2_tile=s2_tile, seq_lens=(100, 700, 1500), B=3,
                                     num_blocks=40))
    ref = oracle_mod.mla_decode(inp)
    compare(gpu_out_float(_run(B, inp, f"tile{s2_tile}")), ref["out_bf16"], f"mla s2_tile={s2_tile}")


def test_mla_two_query_positions(B, oracle_mod):
    # s1 = 2: the valid count n = clamp(seq - s1 + 1 + s, 0, topk) differs between the positions
    inp = synth.make_mla_inputs(_cfg("mla-s1-2", s1=2, topk=512, seq_lens=(300, 513), s2_tile=256))
    ref = oracle_mod.mla_decode(inp)
    compare(gpu_out_float(_run(B, inp, "s1=2")), ref["out_bf16"], "mla s1=2")


def test_mla_empty_sequence_gives_zeros(B, oracle_mod):
    inp = synth.make_mla_inputs(_cfg("mla-empty", seq_lens=(0, 600)))
    ref = oracle_mod.mla_decode(inp)
    got = gpu_out_float(_run(B, inp, "empty"))
    compare(got, ref["out_bf16"], "mla empty")
    assert np.all(got.reshape(2, 32, 512)[0] == 0.0)


def test_mla_deterministic_and_relabelling(B):
    inp = synth.make_mla_inputs(_cfg("mla-relabel"))
    a = _run(B, inp, "repeat-1")
    b = _run(B, inp, "repeat-2")
    assert torch.equal(a, b)
    # permute the physical pool and rewrite the table: the output must not change
    cfg = inp["cfg"]
    nb = cfg.num_blocks
    perm = torch.randperm(nb, generator=torch.Generator().manual_seed(5))
    inv = torch.empty_like(perm)
    inv[perm] = torch.arange(nb)
    cache = inp["cache"].view(nb, cfg.block_size, -1)[inv].reshape(inp["cache"].shape).contiguous()
    t = inp["block_table"].clone()
    t[t >= 0] = perm[t[t >= 0].long()].to(torch.int32)
    inp2 = dict(inp, cache=cache, block_table=t)
    c = _run(B, inp2, "relabelled")
    assert torch.equal(a, c)


def test_mla_full_size_sampled_batches(B, oracle_mod):
    # the full MLA workload (B=16, nq=128, topk 2048, seq 4k-32k); oracle on two batches
    cfg = synth.CONFIGS[4]
    inp = synth.make_mla_inputs(cfg)
    got = gpu_out_float(_run(B, inp, "config4")).reshape(cfg.B * cfg.s1, cfg.nq, 512)
    ref = oracle_mod.mla_decode(inp, b_range=(0, 2))["out_bf16"].reshape(cfg.B * cfg.s1, cfg.nq, 512)
    compare(got[:2 * cfg.s1], ref[:2 * cfg.s1], "mla config4 batches 0-1")


def _run_split(B, inp_h, tag):
    print(f"[gpu] mla kv_split {tag} seqs={inp_h['kv_act_seqs'].tolist()[:8]}", flush=True)
    out = B.mla_decode_kv_split_inputs(to_device(synth.mla_kv_split(inp_h)))
    torch.cuda.synchronize()
    return out


@pytest.mark.parametrize("s2_tile", [128, 512])
def test_mla_kv_split_matches_packed_and_oracle(B, oracle_mod, s2_tile):
    """The kv_split layout (three tensors) gives the packed layout's output bit for
    bit on the same values, and matches the oracle."""
    inp = synth.make_mla_inputs(_cfg(f"mla-split-t{s2_tile}", s2_tile=s2_tile, seq_lens=(100, 700, 1500), B=3,
                                     num_blocks=40, seed=13))
    packed = _run(B, inp, f"packed tile{s2_tile}")
    split = _run_split(B, inp, f"tile{s2_tile}")
    assert torch.equal(packed, split)
    compare(gpu_out_float(split), oracle_mod.mla_decode(inp)["out_bf16"], f"mla kv_split s2_tile={s2_tile}")


def test_mla_kv_split_full_size(B, oracle_mod):
    cfg = synth.CONFIGS[4]
    inp = synth.make_mla_inputs(cfg)
    got = gpu_out_float(_run_split(B, inp, "config4")).reshape(cfg.B * cfg.s1, cfg.nq, 512)
    ref = oracle_mod.mla_decode(inp, b_range=(2, 4))["out_bf16"].reshape(cfg.B * cfg.s1, cfg.nq, 512)
    compare(got[2 * cfg.s1:4 * cfg.s1], ref[2 * cfg.s1:4 * cfg.s1], "mla kv_split config4 batches 2-3")
