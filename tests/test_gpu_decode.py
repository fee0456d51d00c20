"""GPU parity of the HIP decode against the CPU oracle (through the C ABI).

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


def _case(name, **kw):
    base = dict(name=name, B=2, s1=1, nq=8, nkv=2, D=128, seq_lens=(200, 513), s2_tile=256,
                num_blocks=10, max_blocks_per_seq=6, seed=7)
    base.update(kw)
    return synth.GqaConfig(**base)


def _run(B, inp_h, num_splits=0, tag=""):
    print(f"[gpu] {tag} cfg={inp_h['cfg'].name} splits={num_splits} "
          f"seqs={inp_h['kv_act_seqs'].tolist()[:8]}", flush=True)
    d = to_device(inp_h)
    out = B.decode_inputs(d, num_splits=num_splits)
    torch.cuda.synchronize()
    return gpu_out_float(out)


def test_config0_parity(B, oracle_mod):
    inp = synth.make_gqa_inputs(synth.CONFIGS[0])
    ref = oracle_mod.gqa_decode(inp)
    for ns in (0, 1, 2, 3):
        got = _run(B, inp, ns, "config0")
        compare(got, ref, f"config0 splits={ns}")


def test_config0_gather_and_q_codes_bit_exact(B, oracle_mod):
    inp = synth.make_gqa_inputs(synth.CONFIGS[0])
    ref = oracle_mod.gqa_decode(inp)
    print("[gpu] config0 debug dump", flush=True)
    d = to_device(inp)
    out, rows, q8 = B.decode_debug(d["q"], d["q_scale"], d["k_cache"], d["k_scale"], d["v_cache"],
                                   d["v_scale"], d["block_table"], d["kv_act_seqs"], d["softmax_scale"],
                                   inp["cfg"].s2_tile)
    torch.cuda.synchronize()
    assert np.array_equal(rows.cpu().numpy(), ref["rows"])
    assert np.array_equal(q8.cpu().numpy(), ref["q8"])
    compare(gpu_out_float(out), ref, "config0 debug")


@pytest.mark.parametrize("num_splits", [0, 1])
def test_q_codes_wide_scales_bit_exact(B, oracle_mod, num_splits):
    """Step 1's FP8 query codes on both paths (0: whole-row, 1: per-head) for
    q_scale drawn over 2^-70 .. 2^70 (across the range where the kernels divide
    through one reciprocal per row and the range where they divide per value),
    powers of two, zeros and negative scales, and query values of every
    binade: the codes equal the oracle's FP32 division, byte for byte."""
    cfg = _case("qcodes", B=3, s1=2, nq=16, nkv=2, seq_lens=(5, 130, 300), num_blocks=10, max_blocks_per_seq=4,
                seed=21)
    inp = synth.make_gqa_inputs(cfg)
    g = torch.Generator().manual_seed(22)
    n = inp["q_scale"].numel()
    mant = 1.0 + torch.rand(n, generator=g, dtype=torch.float64)
    expo = torch.randint(-70, 71, (n,), generator=g).double()
    qs = (mant * torch.pow(2.0, expo)).float()
    qs[::7] = torch.pow(2.0, expo[::7]).float()                     # powers of two
    qs[3::11] = 0.0
    qs[5::13] = -qs[5::13]
    inp["q_scale"] = qs.reshape(inp["q_scale"].shape).contiguous()
    bits = torch.randint(0, 1 << 16, inp["q"].shape, generator=g, dtype=torch.int32)
    bits = torch.where((bits & 0x7F80) == 0x7F80, bits & ~0x4000, bits)     # no inf / NaN queries
    inp["q"] = bits.to(torch.int16).view(torch.bfloat16).contiguous()
    ref = oracle_mod.gqa_decode(inp)
    print(f"[gpu] q codes, wide scales, splits={num_splits}", flush=True)
    d = to_device(inp)
    _, _, q8 = B.decode_debug(d["q"], d["q_scale"], d["k_cache"], d["k_scale"], d["v_cache"], d["v_scale"],
                              d["block_table"], d["kv_act_seqs"], d["softmax_scale"], cfg.s2_tile,
                              num_splits=num_splits)
    torch.cuda.synchronize()
    got = q8.cpu().numpy()
    if not np.array_equal(got, ref["q8"]):
        bad = np.argwhere(got != ref["q8"])
        raise AssertionError(f"{len(bad)} codes differ, first {bad[:4].tolist()}")


@pytest.mark.parametrize("B_,nq,nkv", [(1024, 4, 1), (256, 32, 8)])
def test_whole_row_most_pairs(B, oracle_mod, B_, nq, nkv):
    """The largest (batch, head group) count the whole-row path takes (1024):
    one head per workgroup (nkv odd) and two; mostly short sequences with a
    long one every 64 batches, so ranges hold many whole sequences and some
    sequences are split.  Every output row against the oracle."""
    lens = [(37 * b) % 250 + 1 if b % 64 else 1500 + b for b in range(B_)]
    mb = (max(lens) + 127) // 128
    nblk = sum((x + 127) // 128 for x in lens) + 4
    cfg = _case(f"pairs-{B_}x{nkv}", B=B_, nq=nq, nkv=nkv, seq_lens=tuple(lens), num_blocks=nblk,
                max_blocks_per_seq=mb, s2_tile=256, seed=B_ + nkv)
    inp = synth.make_gqa_inputs(cfg)
    ref = oracle_mod.gqa_decode(inp)
    compare(_run(B, inp, 0, "most pairs"), ref, f"B={B_} nkv={nkv}")


@pytest.mark.parametrize("s2_tile", [128, 256, 512, 1024, 2048])
def test_tile_sizes(B, oracle_mod, s2_tile):
    cfg = _case(f"tile{s2_tile}", seq_lens=(1, 127, 129, 1500, 2048, 2100), B=6, nq=8, nkv=2,
                num_blocks=64, max_blocks_per_seq=17, s2_tile=s2_tile, seed=s2_tile)
    inp = synth.make_gqa_inputs(cfg)
    ref = oracle_mod.gqa_decode(inp)
    for ns in (1, 0, 5):
        compare(_run(B, inp, ns, f"tile{s2_tile}"), ref, f"s2_tile={s2_tile} splits={ns}")


@pytest.mark.parametrize("s1,nq,nkv", [(1, 12, 1), (1, 96, 8), (2, 48, 8), (4, 32, 4), (3, 48, 3),
                                        (4, 64, 4), (1, 16, 16), (1, 64, 1)])
def test_row_shapes(B, oracle_mod, s1, nq, nkv):
    # rows per KV head = s1 * nq / nkv: 12, 12, 12, 32, 48, 64, 1, 64
    cfg = _case(f"rows-s1{s1}-nq{nq}-nkv{nkv}", B=3, s1=s1, nq=nq, nkv=nkv, seq_lens=(77, 600, 1100),
                num_blocks=20, max_blocks_per_seq=9, s2_tile=256, seed=nq + s1)
    inp = synth.make_gqa_inputs(cfg)
    ref = oracle_mod.gqa_decode(inp)
    for ns in (0, 1, 4):
        compare(_run(B, inp, ns, "rows"), ref, f"s1={s1} nq={nq} nkv={nkv} splits={ns}")


def test_edge_lengths(B, oracle_mod):
    # empty sequence, length 1, exact tile / block multiples, ragged tails, a full row
    cfg = _case("edges", B=8, seq_lens=(0, 1, 128, 256, 257, 511, 512, 768), num_blocks=40,
                max_blocks_per_seq=6, s2_tile=256, seed=3)
    inp = synth.make_gqa_inputs(cfg)
    ref = oracle_mod.gqa_decode(inp)
    for ns in (1, 2, 3, 0):
        got = _run(B, inp, ns, "edges")
        compare(got, ref, f"edges splits={ns}")
        assert np.all(got.reshape(8, 8, 128)[0] == 0.0)


def test_clamped_length_and_bad_ids(B, oracle_mod):
    cfg = _case("clamp", B=2, seq_lens=(300, 700), num_blocks=12, max_blocks_per_seq=6, seed=4)
    inp = synth.make_gqa_inputs(cfg)
    inp["kv_act_seqs"] = torch.tensor([300, 10 ** 6], dtype=torch.int32)     # clamped to 768
    t = inp["block_table"].clone()
    t[1, 5] = -1                                # inside the clamped length: reads block 0
    t[0, 1] = 10 ** 7                           # out of range: reads block 0
    inp["block_table"] = t
    ref = oracle_mod.gqa_decode(inp)
    for ns in (1, 0):
        compare(_run(B, inp, ns, "clamp"), ref, f"clamp splits={ns}")


@pytest.mark.parametrize("num_splits", [0, 1, 3])
def test_poison_beyond_sequence_bit_identical(B, num_splits):
    """NaN codes and NaN scales in every token slot past the sequences and
    random ids in unused table entries change no output bit, on the whole-row
    path (0) and on the per-head path without and with splits."""
    cfg = _case("poison", B=4, seq_lens=(1, 200, 513, 1000), num_blocks=20, max_blocks_per_seq=8, seed=9)
    clean = _run(B, synth.make_gqa_inputs(cfg), num_splits, "poison-clean")
    dirty_inp = synth.make_gqa_inputs(cfg, poison=True)
    assert torch.isnan(dirty_inp["k_scale"]).any()
    dirty = _run(B, dirty_inp, num_splits, "poison-dirty")
    assert np.array_equal(clean, dirty)


def test_block_relabelling_bit_identical(B):
    cfg = _case("relabel", B=3, seq_lens=(100, 700, 1300), num_blocks=24, max_blocks_per_seq=11, seed=10)
    inp = synth.make_gqa_inputs(cfg)
    base = _run(B, inp, 0, "relabel-base")
    perm = torch.randperm(cfg.num_blocks, generator=torch.Generator().manual_seed(1))
    inv = torch.empty_like(perm)
    inv[perm] = torch.arange(cfg.num_blocks)
    t = inp["block_table"].clone()
    t[t >= 0] = inv[t[t >= 0].long()].to(torch.int32)
    moved = dict(inp, k_cache=inp["k_cache"][perm].contiguous(), v_cache=inp["v_cache"][perm].contiguous(),
                 k_scale=inp["k_scale"][perm].contiguous(), block_table=t)
    assert np.array_equal(base, _run(B, moved, 0, "relabel-moved"))


def test_deterministic_repeat(B):
    cfg = _case("repeat", B=4, seq_lens=(900, 20, 3000, 1), num_blocks=40, max_blocks_per_seq=24, seed=12)
    inp = synth.make_gqa_inputs(cfg)
    a = _run(B, inp, 0, "repeat-1")
    b = _run(B, inp, 0, "repeat-2")
    assert np.array_equal(a, b)


@pytest.mark.parametrize("cfg_id", [1, 3])
def test_scaled_down_configs_full_parity(B, oracle_mod, cfg_id):
    # the full-size shapes with fewer sequences, every output row checked
    from dataclasses import replace
    full = synth.CONFIGS[cfg_id]
    cfg = replace(full, B=4 if cfg_id == 1 else 16, num_blocks=full.max_blocks_per_seq * (4 if cfg_id == 1 else 16))
    inp = synth.make_gqa_inputs(cfg)
    ref = oracle_mod.gqa_decode(inp)
    for ns in (0, 1):
        compare(_run(B, inp, ns, f"config{cfg_id}-small"), ref, f"config{cfg_id} small splits={ns}")


def _run_dev(B, inp_d, tag, num_splits=0):
    print(f"[gpu] {tag} splits={num_splits}", flush=True)
    out = B.decode_inputs(inp_d, num_splits=num_splits)
    torch.cuda.synchronize()
    return gpu_out_float(out)


def test_shared_workspace_between_paths(B, oracle_mod):
    """One zero-filled workspace serving whole-row calls and split calls in turn:
    the whole-row path must leave the split path's arrival counters at zero."""
    cfg = _case("shared-ws", B=3, seq_lens=(1500, 700, 2100), num_blocks=60, max_blocks_per_seq=20, seed=21)
    inp = synth.make_gqa_inputs(cfg)
    ref = oracle_mod.gqa_decode(inp)
    d = to_device(inp)
    c = inp["cfg"]
    need = max(B.workspace_size(c.B, c.s1, c.nq, c.nkv, c.D, 128, c.max_blocks_per_seq, c.s2_tile, ns)[0]
               for ns in (0, 3))
    ws = torch.zeros(need, dtype=torch.uint8, device="cuda")
    for i, ns in enumerate((0, 3, 0, 3)):
        print(f"[gpu] shared workspace call {i} splits={ns}", flush=True)
        out = B.decode_inputs(d, num_splits=ns, workspace=ws)
        torch.cuda.synchronize()
        compare(gpu_out_float(out), ref, f"shared workspace call {i} splits={ns}")


@pytest.mark.parametrize("s1,nq,nkv,s2_tile,seqs", [
    (4, 32, 4, 256, (1, 3, 4, 5, 257, 258, 515, 1024)),     # seq < s1, last tiles with fewer tokens than s1
    (2, 48, 8, 512, (700, 1, 513, 2049)),
    (3, 30, 3, 128, (130, 129, 3, 384)),                     # odd KV heads (one head per workgroup)
    (1, 96, 8, 512, (900, 4000)),                            # s1 = 1: the plain decode
])
def test_causal_parity(B, oracle_mod, s1, nq, nkv, s2_tile, seqs):
    mb = (max(seqs) + 127) // 128 + 1
    cfg = _case(f"causal-s1{s1}", B=len(seqs), s1=s1, nq=nq, nkv=nkv, s2_tile=s2_tile, seq_lens=seqs,
                num_blocks=mb * len(seqs), max_blocks_per_seq=mb, seed=40 + s1)
    inp = dict(synth.make_gqa_inputs(cfg), causal=True)
    ref = oracle_mod.gqa_decode(inp)
    for ns in (0, 1, 3):                     # whole-row path, per-head path without and with splits
        got = _run(B, inp, ns, "causal")
        compare(got, ref, f"causal s1={s1} nq={nq} nkv={nkv} tile={s2_tile} splits={ns}")
        if s1 == 1:
            assert np.array_equal(got, _run(B, dict(inp, causal=False), ns, "plain"))


def _rows_ref(oracle_mod, inp):
    """The oracle over every output row, rows spread over the threads (few long batches)."""
    c = inp["cfg"]
    return oracle_mod.gqa_decode_rows(inp, np.arange(c.B * c.s1 * c.nq))


@pytest.mark.parametrize("s1,nq,nkv,s2_tile,seqs", [
    (128, 12, 1, 256, (700, 2000, 128, 100)),     # G = 12: 1536 query rows per KV head; seq < s1 in the last
    (128, 96, 8, 512, (1100, 2600)),              # the GLM-4.5 head layout
    (512, 12, 1, 512, (600, 1500, 300)),          # 6144 rows; seq 300 < s1: the first 211 positions see nothing
    (512, 12, 1, 128, (1024, 513)),
])
def test_prefill_causal_parity(B, oracle_mod, s1, nq, nkv, s2_tile, seqs):
    """Causal decode with prefill-length s1 (the page pair's Decode / Prefill
    entries share one signature): the per-head path in blocks of 32 query rows,
    position s seeing the first seq - s1 + 1 + s tokens; without and with
    splits."""
    mb = (max(seqs) + 127) // 128 + 1
    cfg = _case(f"prefill-s1{s1}-nq{nq}", B=len(seqs), s1=s1, nq=nq, nkv=nkv, s2_tile=s2_tile, seq_lens=seqs,
                num_blocks=mb * len(seqs), max_blocks_per_seq=mb, seed=70 + s1 + nq)
    inp = dict(synth.make_gqa_inputs(cfg), causal=True)
    ref = _rows_ref(oracle_mod, inp)
    for ns in (0, 2):
        got = _run(B, inp, ns, f"prefill s1={s1}")
        # measured: at most 7 ulps (s1 = 128, one KV head)
        compare(got.reshape(-1, 128), ref, f"prefill causal s1={s1} nq={nq} nkv={nkv} tile={s2_tile} splits={ns}",
                max_ulps=16)
        rows = got.reshape(len(seqs), s1, nq, 128)
        for bi, sq in enumerate(seqs):          # positions that see no token are zero rows
            nz = max(0, s1 - sq)
            assert np.all(rows[bi, :nz] == 0.0)


def test_long_s1_non_causal_parity(B, oracle_mod):
    """More than 64 query rows per KV head without the causal limit (every
    position attends to the whole sequence): row blocks of 32."""
    cfg = _case("long-s1", B=3, s1=16, nq=48, nkv=4, s2_tile=256, seq_lens=(900, 77, 1400), num_blocks=40,
                max_blocks_per_seq=12, seed=81)
    inp = synth.make_gqa_inputs(cfg)
    ref = oracle_mod.gqa_decode(inp)
    for ns in (0, 1, 4):
        compare(_run(B, inp, ns, "long s1"), ref, f"long s1 non-causal splits={ns}")


def test_row_blocks_dumps_bit_exact(B, oracle_mod):
    """The whole-row path with a KV head's rows in blocks of 32 (s1 = 6, G = 11:
    66 rows, the last block of 2): the gathered rows and the query codes dumped
    from inside the kernel equal the oracle's, and so does the output."""
    cfg = _case("row-blocks", B=5, s1=6, nq=22, nkv=2, s2_tile=512, seq_lens=(1300, 1, 640, 0, 2049),
                num_blocks=60, max_blocks_per_seq=17, seed=83)
    inp = synth.make_gqa_inputs(cfg)
    ref = oracle_mod.gqa_decode(inp)
    d = to_device(inp)
    print("[gpu] row-block dumps", flush=True)
    out, rows, q8 = B.decode_debug(d["q"], d["q_scale"], d["k_cache"], d["k_scale"], d["v_cache"], d["v_scale"],
                                   d["block_table"], d["kv_act_seqs"], d["softmax_scale"], cfg.s2_tile, s1=cfg.s1)
    torch.cuda.synchronize()
    assert np.array_equal(rows.cpu().numpy(), ref["rows"])
    assert np.array_equal(q8.cpu().numpy(), ref["q8"])
    compare(gpu_out_float(out), ref, "row-block debug")
    for ns in (0, 3):
        compare(_run(B, inp, ns, "row blocks"), ref, f"row blocks splits={ns}")


@pytest.mark.parametrize("num_splits", [0, 2])
def test_prefill_causal_poison_bit_identical(B, num_splits):
    """NaN codes and scales past every sequence change no output bit of the
    causal prefill either."""
    cfg = _case("prefill-poison", B=3, s1=64, nq=12, nkv=1, s2_tile=256, seq_lens=(40, 700, 1300), num_blocks=30,
                max_blocks_per_seq=11, seed=91)
    clean = _run(B, dict(synth.make_gqa_inputs(cfg), causal=True), num_splits, "prefill poison clean")
    dirty = _run(B, dict(synth.make_gqa_inputs(cfg, poison=True), causal=True), num_splits, "prefill poison dirty")
    assert np.array_equal(clean, dirty)


@pytest.mark.parametrize("s1,nq,nkv,s2_tile,seqs,causal", [
    (128, 32, 4, 128, (100, 700, 1500), True),          # 8 row tiles of 128; seq < s1 in the first
    (100, 24, 4, 256, (0, 333, 1024, 1900), True),      # 600 rows: a last row tile of 88; an empty sequence
    (16, 64, 4, 512, (5, 900, 77, 1400, 513, 2048, 0, 1025), False),   # 256 rows, no causal limit
])
def test_prefill_kernel_parity(B, oracle_mod, s1, nq, nkv, s2_tile, seqs, causal):
    """128 or more query rows per KV head and at least 64 (batch, KV head, 128-row)
    workgroups: the prefill kernel (each K / V block staged and converted once per
    128 rows).  Against the oracle; positions that see no token give zero rows."""
    mb = (max(seqs) + 127) // 128 + 1
    cfg = _case(f"prefill-kernel-s1{s1}-nq{nq}", B=len(seqs), s1=s1, nq=nq, nkv=nkv, s2_tile=s2_tile,
                seq_lens=seqs, num_blocks=mb * len(seqs), max_blocks_per_seq=mb, seed=110 + s1 + nq)
    inp = dict(synth.make_gqa_inputs(cfg), causal=causal)
    ref = oracle_mod.gqa_decode(inp)
    got = _run(B, inp, 0, f"prefill kernel s1={s1} nq={nq} nkv={nkv} tile={s2_tile} causal={causal}")
    compare(got, ref, f"prefill kernel s1={s1} nq={nq} nkv={nkv} tile={s2_tile} causal={causal}", max_ulps=16)
    rows = got.reshape(len(seqs), s1, nq, 128)
    for bi, sq in enumerate(seqs):
        nz = max(0, s1 - sq) if causal else (s1 if sq == 0 else 0)
        assert np.all(rows[bi, :nz] == 0.0)


def test_prefill_kernel_many_batches(B, oracle_mod):
    """More batches than the prefill kernel orders by length (300 > 256): workgroups take
    the batches in index order.  s1=16, G=8 (128 query rows per KV head), lengths from 0
    to 899 (some shorter than s1), causal; against the oracle."""
    seqs = tuple((37 * i + (i * i) % 11) % 900 for i in range(300))
    mb = (max(seqs) + 127) // 128 + 1
    cfg = _case("prefill-kernel-b300", B=len(seqs), s1=16, nq=8, nkv=1, s2_tile=256, seq_lens=seqs,
                num_blocks=mb * len(seqs), max_blocks_per_seq=mb, seed=131)
    inp = dict(synth.make_gqa_inputs(cfg), causal=True)
    ref = oracle_mod.gqa_decode(inp)
    got = _run(B, inp, 0, "prefill kernel B=300 s1=16 nq=8 nkv=1 tile=256 causal")
    compare(got, ref, "prefill kernel B=300", max_ulps=16)


def test_prefill_kernel_poison_bit_identical(B):
    """The prefill kernel: NaN codes and scales past every sequence change no output bit."""
    cfg = _case("prefill-kernel-poison", B=3, s1=64, nq=64, nkv=8, s2_tile=256, seq_lens=(40, 700, 1300),
                num_blocks=30, max_blocks_per_seq=11, seed=93)
    clean = _run(B, dict(synth.make_gqa_inputs(cfg), causal=True), 0, "prefill kernel poison clean")
    dirty = _run(B, dict(synth.make_gqa_inputs(cfg, poison=True), causal=True), 0, "prefill kernel poison dirty")
    assert np.array_equal(clean, dirty)
