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
    compare(gpu_out_float(_run(B, inp, f"tile{s2_tile}")), ref, f"mla s2_tile={s2_tile}")


def test_mla_two_query_positions(B, oracle_mod):
    # s1 = 2: the valid count n = clamp(seq - s1 + 1 + s, 0, topk) differs between the positions
    inp = synth.make_mla_inputs(_cfg("mla-s1-2", s1=2, topk=512, seq_lens=(300, 513), s2_tile=256))
    ref = oracle_mod.mla_decode(inp)
    compare(gpu_out_float(_run(B, inp, "s1=2")), ref, "mla s1=2")


def test_mla_empty_sequence_gives_zeros(B, oracle_mod):
    inp = synth.make_mla_inputs(_cfg("mla-empty", seq_lens=(0, 600)))
    ref = oracle_mod.mla_decode(inp)
    got = gpu_out_float(_run(B, inp, "empty"))
    compare(got, ref, "mla empty")
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
    compare(gpu_out_float(split), oracle_mod.mla_decode(inp), f"mla kv_split s2_tile={s2_tile}")


def _selected_rows(inp):
    """Cache rows the decode may read: the first n entries of every top-k slice
    (positions clamped to [0, seq)) mapped through the table."""
    cfg = inp["cfg"]
    topk = inp["topk"].cpu().numpy()
    table = inp["block_table"].cpu().numpy()
    seqs = inp["kv_act_seqs"].cpu().numpy()
    K = cfg.topk
    rows = set()
    for b in range(cfg.B):
        seq = min(max(int(seqs[b]), 0), table.shape[1] * cfg.block_size)
        for s in range(cfg.s1):
            n = min(max(seq - cfg.s1 + 1 + s, 0), K)
            for h in range(cfg.nkv):
                for p in topk[b * cfg.s1 + s, h * K:h * K + n]:
                    p = min(max(int(p), 0), seq - 1)
                    bid = int(table[b, p // cfg.block_size])
                    bid = 0 if bid < 0 or bid >= cfg.num_blocks else bid
                    rows.add(bid * cfg.block_size + p % cfg.block_size)
    return rows


def _poison_mla(inp):
    """NaN codes, NaN rope values and NaN / Inf group scales in every cache row
    the decode must not use, garbage in the top-k entries past n and random ids
    in the table entries past each sequence."""
    cfg = inp["cfg"]
    sel = _selected_rows(inp)
    cache = inp["cache"].clone()
    bad = torch.ones(cache.shape[0], dtype=torch.bool)
    bad[list(sel)] = False
    nbad = int(bad.sum())
    cache[bad, :512] = 0x7F
    cache[bad, 512:640] = 0xFF
    scl = torch.tensor([float("nan"), float("inf"), -float("inf"), float("nan")], dtype=torch.float32)
    cache[bad, 640:656] = scl.view(torch.uint8).repeat(nbad, 1)
    topk = inp["topk"].clone()
    seqs = inp["kv_act_seqs"].tolist()
    g = torch.Generator().manual_seed(99)
    K = cfg.topk
    for b in range(cfg.B):
        for s in range(cfg.s1):
            n = min(max(seqs[b] - cfg.s1 + 1 + s, 0), K)
            for h in range(cfg.nkv):
                junk = torch.randint(-2 ** 30, 2 ** 30, (K - n,), generator=g, dtype=torch.int64).to(torch.int32)
                topk[b * cfg.s1 + s, h * K + n:(h + 1) * K] = junk
    table = inp["block_table"].clone()
    for b in range(cfg.B):
        used = (seqs[b] + cfg.block_size - 1) // cfg.block_size
        table[b, used:] = torch.randint(0, cfg.num_blocks, (table.shape[1] - used,), generator=g, dtype=torch.int32)
    return dict(inp, cache=cache, topk=topk, block_table=table), bad


@pytest.mark.parametrize("s2_tile", [128, 512])
def test_mla_poison_outside_selection_bit_identical(B, oracle_mod, s2_tile):
    """Rows the top-k entries do not select -- row 0 among them -- hold NaN
    codes, NaN rope values and NaN / Inf scales; entries past n are garbage.
    With seq < topk and s1 = 2 the tiles end part-way, so positions past n
    read row 0: the output must equal the clean run bit for bit."""
    inp = synth.make_mla_inputs(_cfg("mla-poison", s1=2, topk=1024, seq_lens=(300, 1500, 700), B=3, num_blocks=60,
                                     s2_tile=s2_tile, seed=17))
    dirty, bad = _poison_mla(inp)
    assert bool(bad[0]), "row 0 must be one of the poisoned rows"
    clean = _run(B, inp, f"poison clean tile{s2_tile}")
    got = _run(B, dirty, f"poison dirty tile{s2_tile}")
    assert torch.equal(clean, got)
    compare(gpu_out_float(got), oracle_mod.mla_decode(inp), f"mla poison s2_tile={s2_tile}")
    split = B.mla_decode_kv_split_inputs(to_device(synth.mla_kv_split(dirty)))
    torch.cuda.synchronize()
    assert torch.equal(clean, split)


def test_mla_out_of_range_indices_clamped(B, oracle_mod):
    """Top-k entries below 0 or at / past seq inside the first n are clamped
    to [0, seq) (the table's own rule for ids, applied to positions)."""
    inp = synth.make_mla_inputs(_cfg("mla-clamp", topk=512, seq_lens=(700, 1500), seed=23))
    topk = inp["topk"].clone()
    topk[0, 3] = -5
    topk[0, 10] = 700
    topk[1, 0] = 10 ** 9
    topk[1, 511] = -(2 ** 31)
    inp = dict(inp, topk=topk)
    compare(gpu_out_float(_run(B, inp, "clamp")), oracle_mod.mla_decode(inp), "mla clamped indices")


@pytest.mark.parametrize("nkv", [2, 4])
def test_mla_several_kv_heads(B, oracle_mod, nkv):
    """nkv KV heads, each with its own top-k slice over the shared latent rows
    (topk_indices (t, n_kv*topk)); 32 query heads per KV head."""
    inp = synth.make_mla_inputs(_cfg(f"mla-nkv{nkv}", nq=32 * nkv, nkv=nkv, s1=2, topk=512,
                                     seq_lens=(300, 1100), s2_tile=256, seed=30 + nkv))
    got = gpu_out_float(_run(B, inp, f"nkv={nkv}"))
    compare(got, oracle_mod.mla_decode(inp), f"mla nkv={nkv}")
    # each head group reads its own slice: swapping the first two slices together
    # with the query heads of the first two groups swaps those groups' outputs
    K, nq = inp["cfg"].topk, 32 * nkv
    t = inp["topk"]
    swapped = torch.cat([t[:, K:2 * K], t[:, :K], t[:, 2 * K:]], dim=1).contiguous()

    def swap_heads(q):
        q3 = q.view(-1, nq, q.shape[-1])
        return torch.cat([q3[:, 32:64], q3[:, :32], q3[:, 64:]], dim=1).reshape(q.shape).contiguous()

    inp2 = dict(inp, topk=swapped, q_nope=swap_heads(inp["q_nope"]), q_rope=swap_heads(inp["q_rope"]))
    got2 = gpu_out_float(_run(B, inp2, f"nkv={nkv} swapped")).reshape(-1, nq, 512)
    g1 = got.reshape(-1, nq, 512)
    assert np.array_equal(got2[:, :32], g1[:, 32:64]) and np.array_equal(got2[:, 32:64], g1[:, :32])
    assert np.array_equal(got2[:, 64:], g1[:, 64:])


@pytest.mark.parametrize("nq,nkv", [(64, 1), (128, 2), (192, 1)])
def test_mla_wide_query_groups_parity(B, oracle_mod, nq, nkv):
    """Query groups of 64, 64 and 192 heads (several 32-head workgroups per tile) at
    s2_tile 512, s1 = 2 and lengths 0, 100, 300, 700 and 1500 under topk 1024: empty
    rows, a tile whose second half holds no valid row, tiles ending part-way and two
    tiles."""
    inp = synth.make_mla_inputs(_cfg(f"mla-groups-{nq}-{nkv}", nq=nq, nkv=nkv, s1=2, topk=1024, B=5,
                                     seq_lens=(0, 100, 300, 700, 1500), num_blocks=80, seed=41 + nq))
    compare(gpu_out_float(_run(B, inp, f"groups nq={nq} nkv={nkv}")), oracle_mod.mla_decode(inp),
            f"mla groups nq={nq} nkv={nkv}")


def test_mla_wide_group_poison_and_kv_split(B, oracle_mod):
    """A 64-head query group under the poisoned cache (NaN / Inf in every unselected
    row, row 0 among them) gives the clean output bit for bit, in both layouts."""
    inp = synth.make_mla_inputs(_cfg("mla-groups-poison", nq=64, s1=2, topk=1024, seq_lens=(300, 1500, 700), B=3,
                                     num_blocks=60, s2_tile=512, seed=17))
    dirty, bad = _poison_mla(inp)
    assert bool(bad[0]), "row 0 must be one of the poisoned rows"
    clean = _run(B, inp, "groups poison clean")
    got = _run(B, dirty, "groups poison dirty")
    assert torch.equal(clean, got)
    compare(gpu_out_float(got), oracle_mod.mla_decode(inp), "mla groups poison")
    split = _run_split(B, dirty, "groups poison")
    assert torch.equal(clean, split)
