"""Pins of the CPU oracle against what the pages and the mathematics fix.

Every test here is CPU-only.  None retypes the oracle: codecs are checked
against torch's own casts and against their defining property, the decode
against closed forms (tests/closed_forms.py), invariances, special cases with
known answers and the page-stated constants (tests/golden/page_constants.json).
"""
import json
import math
import os
from dataclasses import replace

import numpy as np
import pytest
import torch

from fp8_paged_kv_amd import synth
from tests import closed_forms as cf

GOLDEN = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "page_constants.json")))


def small_cfg(**kw):
    base = dict(name="pin", B=2, s1=1, nq=8, nkv=2, D=128, seq_lens=(200, 513), s2_tile=256,
                num_blocks=10, max_blocks_per_seq=6, seed=11)
    base.update(kw)
    return synth.GqaConfig(**base)


# ------------------------------------------------------------------ codecs

def test_e4m3_decode_matches_torch_all_codes(oracle_mod):
    codes = np.arange(256, dtype=np.uint8)
    ours = oracle_mod.e4m3_decode(codes)
    ref = cf.e4m3_value(codes)
    nan = np.isnan(ref)
    assert list(np.nonzero(nan)[0]) == [0x7F, 0xFF]
    assert np.array_equal(np.isnan(ours), nan)
    assert np.array_equal(ours[~nan], ref[~nan])


def test_e4m3_max_is_page_value(oracle_mod):
    assert oracle_mod.e4m3_decode(np.array([0x7E]))[0] == GOLDEN["e4m3_max"]["value"]
    assert oracle_mod.e4m3_decode(np.array([0xFE]))[0] == -GOLDEN["e4m3_max"]["value"]
    finite = oracle_mod.e4m3_decode(np.arange(256, dtype=np.uint8))
    assert np.nanmax(np.abs(finite)) == 448.0


def _sweep_points():
    vals = cf.e4m3_value(np.arange(0, 0x7F, dtype=np.uint8))   # 0 .. 448 ascending
    pts = []
    for lo, hi in zip(vals[:-1], vals[1:]):
        mid = 0.5 * (lo + hi)
        pts += [lo, hi, mid, lo + 0.25 * (hi - lo), lo + 0.75 * (hi - lo)]
        m32 = np.float32(mid)
        pts += [float(np.nextafter(m32, np.float32(0))), float(np.nextafter(m32, np.float32(1e9)))]
    pts = np.array(pts, dtype=np.float32).astype(np.float64)
    return np.concatenate([pts, -pts])


def test_e4m3_encode_rne_matches_torch_in_range(oracle_mod):
    x = _sweep_points()
    ours = oracle_mod.e4m3_encode(x)
    ref = torch.as_tensor(x.astype(np.float32)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    bad = np.nonzero(ours != ref)[0]
    assert bad.size == 0, [(x[i], ours[i], ref[i]) for i in bad[:10]]


def test_e4m3_encode_is_nearest_ties_even(oracle_mod):
    # Defining property, checked by brute force over all finite codes.
    rng = np.random.default_rng(5)
    x = np.concatenate([rng.uniform(-448, 448, 3000), rng.uniform(-0.02, 0.02, 2000)]).astype(np.float32).astype(np.float64)
    vals = cf.e4m3_value(np.arange(256, dtype=np.uint8))
    finite = ~np.isnan(vals)
    codes = np.arange(256)[finite]
    v = vals[finite]
    ours = oracle_mod.e4m3_encode(x)
    for xi, ci in zip(x, ours):
        d = np.abs(v - xi)
        best = codes[d == d.min()]
        dec = cf.e4m3_value(np.array([ci]))[0]
        assert abs(dec - xi) == d.min()
        if best.size > 1 and not np.all(v[d == d.min()] == 0):
            assert ci % 2 == 0                       # tie -> even mantissa


def test_e4m3_encode_saturates_and_keeps_sign_of_zero(oracle_mod):
    big = np.array([448.0, 448.5, 463.9, 464.0, 480.0, 1e6, np.inf])
    assert list(oracle_mod.e4m3_encode(big)) == [0x7E] * len(big)
    assert list(oracle_mod.e4m3_encode(-big)) == [0xFE] * len(big)
    assert oracle_mod.e4m3_encode(np.array([0.0, -0.0, -1e-9]))[0] == 0x00
    assert list(oracle_mod.e4m3_encode(np.array([-0.0, -1e-9]))) == [0x80, 0x80]
    # subnormals: smallest 2^-9, RNE between 0 and it
    assert list(oracle_mod.e4m3_encode(np.array([2.0 ** -9, 2.0 ** -10, 1.5 * 2.0 ** -9]))) == [1, 0, 2]


def test_bf16_encode_matches_torch_and_nearest(oracle_mod):
    rng = np.random.default_rng(3)
    f = rng.standard_normal(4000).astype(np.float32)
    # exact ties: low 16 bits 0x8000
    u = f.view(np.uint32)
    ties = ((u & 0xFFFF0000) | 0x8000).view(np.float32)
    x = np.concatenate([f, ties]).astype(np.float64)
    ours = oracle_mod.bf16_encode(x)
    ref = torch.as_tensor(x.astype(np.float32)).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ours, ref)
    # FP64 inputs between bf16 values: nearest of the two neighbours
    y = rng.standard_normal(2000) * 3
    enc = oracle_mod.bf16_encode(y)
    dec = oracle_mod.bf16_decode(enc)
    lo = torch.as_tensor(y.astype(np.float32)).to(torch.bfloat16).float().double().numpy()
    ulp = np.abs(np.spacing(lo.astype(np.float32)).astype(np.float64)) * 65536
    assert np.all(np.abs(dec - y) <= 0.5 * ulp + 1e-300)


# ------------------------------------------------------------ page formulas

def test_tile_count_formula_cases():
    for seq, tile, n in GOLDEN["tiles_per_sequence"]["cases"]:
        assert (seq + tile - 1) // tile == n


def test_kv_pool_formula_cases():
    for b, s2, n in GOLDEN["kv_num_blocks"]["cases"]:
        assert b * math.ceil(s2 / GOLDEN["block_size"]["value"]) == n


# --------------------------------------------------------- decode: closed forms

@pytest.fixture(scope="module")
def pin_inputs():
    return synth.make_gqa_inputs(small_cfg(), keep_float=True)


@pytest.fixture(scope="module")
def pin_result(oracle_mod, pin_inputs):
    return oracle_mod.gqa_decode(pin_inputs)


def _all_rows(cfg):
    for b in range(cfg.B):
        for s in range(cfg.s1):
            for qh in range(cfg.nq):
                yield b, s, qh


def test_closed_form_multi_tile(pin_inputs, pin_result):
    cfg = pin_inputs["cfg"]
    for b, s, qh in _all_rows(cfg):
        ref, L, M = cf.closed_form_row(pin_inputs, b, s, qh, cfg.s2_tile)
        got = pin_result["out"][b * cfg.s1 + s, qh]
        np.testing.assert_allclose(got, ref, rtol=1e-12, atol=1e-14)
        np.testing.assert_allclose(pin_result["L"][b * cfg.s1 + s, qh], L, rtol=1e-12)   # sum of softmax weights
        assert pin_result["M"][b * cfg.s1 + s, qh] == pytest.approx(M, rel=1e-14)


def test_closed_form_single_tile(oracle_mod, pin_inputs):
    # s2_tile >= seq: one tile, weights E4M3(448 e^{S-m}) / 448
    inp = dict(pin_inputs, s2_tile=1024)
    res = oracle_mod.gqa_decode(inp)
    cfg = inp["cfg"]
    for b, s, qh in _all_rows(cfg):
        ref, _, _ = cf.closed_form_row(inp, b, s, qh, 1024)
        np.testing.assert_allclose(res["out"][b * cfg.s1 + s, qh], ref, rtol=1e-12, atol=1e-14)


def test_tiling_changes_the_result(oracle_mod, pin_inputs, pin_result):
    # P quantisation is per tile, so the tile size is observable: guards
    # against an implementation that ignores s2_tile.
    res = oracle_mod.gqa_decode(dict(pin_inputs, s2_tile=1024))
    assert not np.array_equal(res["out"][1], pin_result["out"][1])      # seq 513: 3 tiles vs 1
    assert np.array_equal(res["out"][0], pin_result["out"][0])          # seq 200: one tile either way


def test_softmax_weights_sum_to_one(pin_inputs, pin_result):
    # L (online) equals the direct sum of e^{S-M}: the normalised weights sum to 1.
    cfg = pin_inputs["cfg"]
    for b, s, qh in _all_rows(cfg):
        S, _ = cf.scores(pin_inputs, b, s, qh)
        r = b * cfg.s1 + s
        w = np.exp(S - pin_result["M"][r, qh]) / pin_result["L"][r, qh]
        assert abs(w.sum() - 1.0) < 1e-12


def test_quantised_pipeline_close_to_exact_attention(pin_inputs, pin_result):
    cfg = pin_inputs["cfg"]
    num = den = 0.0
    for b, s, qh in _all_rows(cfg):
        exact = cf.exact_attention_row(pin_inputs, b, s, qh)
        got = pin_result["out"][b * cfg.s1 + s, qh]
        num += ((got - exact) ** 2).sum()
        den += (exact ** 2).sum()
    assert math.sqrt(num / den) <= 0.08


def test_q_codes(pin_inputs, pin_result):
    cfg = pin_inputs["cfg"]
    q = pin_inputs["q"].float()
    ref = (q / pin_inputs["q_scale"][..., None]).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(pin_result["q8"], ref)


def test_gather_rows(pin_inputs, pin_result):
    cfg = pin_inputs["cfg"]
    bs = cfg.block_size
    for b in range(cfg.B):
        seq = int(pin_inputs["kv_act_seqs"][b])
        table = pin_inputs["block_table"][b].numpy()
        expect = np.full(cfg.max_blocks_per_seq * bs, -1)
        for i in range((seq + bs - 1) // bs):
            expect[i * bs:(i + 1) * bs] = np.arange(table[i] * bs, (table[i] + 1) * bs)
        expect[seq:] = -1
        assert np.array_equal(pin_result["rows"][b], expect)


# --------------------------------------------------------------- invariances

def test_block_relabelling_is_bit_identical(oracle_mod, pin_inputs, pin_result):
    cfg = pin_inputs["cfg"]
    perm = torch.randperm(cfg.num_blocks, generator=torch.Generator().manual_seed(99))
    inv = torch.empty_like(perm)
    inv[perm] = torch.arange(cfg.num_blocks)
    inp = dict(pin_inputs)
    # physical block i moves to position inv[i]; the table follows it
    inp["k_cache"] = pin_inputs["k_cache"][perm]
    inp["v_cache"] = pin_inputs["v_cache"][perm]
    inp["k_scale"] = pin_inputs["k_scale"][perm]
    t = pin_inputs["block_table"].clone()
    t[t >= 0] = inv[t[t >= 0].long()].to(torch.int32)
    inp["block_table"] = t
    res = oracle_mod.gqa_decode(inp)
    assert np.array_equal(res["out"], pin_result["out"])


def test_poison_beyond_sequence_is_bit_identical(oracle_mod):
    cfg = small_cfg(seed=21)
    clean = oracle_mod.gqa_decode(synth.make_gqa_inputs(cfg))
    poisoned_inp = synth.make_gqa_inputs(cfg, poison=True)
    assert torch.isnan(poisoned_inp["k_scale"]).any()
    poisoned = oracle_mod.gqa_decode(poisoned_inp)
    assert np.array_equal(clean["out"], poisoned["out"])
    assert np.isfinite(poisoned["out"]).all()


def test_minus_one_and_out_of_range_ids_read_block_zero(oracle_mod):
    cfg = small_cfg(seed=5)
    inp = synth.make_gqa_inputs(cfg)
    ref_t = inp["block_table"].clone()
    ref_t[0, 0] = 0
    base = oracle_mod.gqa_decode(dict(inp, block_table=ref_t))
    for bad in (-1, -7, cfg.num_blocks, 10 ** 6):
        t = inp["block_table"].clone()
        t[0, 0] = bad
        res = oracle_mod.gqa_decode(dict(inp, block_table=t))
        assert np.array_equal(res["out"], base["out"])


def test_head_permutation_within_group(oracle_mod, pin_inputs, pin_result):
    cfg = pin_inputs["cfg"]
    G = cfg.nq // cfg.nkv
    perm = torch.arange(cfg.nq)
    perm[0], perm[G - 1] = G - 1, 0            # swap two heads of KV head 0's group
    inp = dict(pin_inputs, q=pin_inputs["q"][:, perm].contiguous(), q_scale=pin_inputs["q_scale"][:, perm].contiguous())
    res = oracle_mod.gqa_decode(inp)
    assert np.array_equal(res["out"], pin_result["out"][:, perm.numpy()])


# -------------------------------------------------------------- special cases

def test_seq_one_returns_the_value_row(oracle_mod):
    cfg = small_cfg(seq_lens=(1, 1), seed=8)
    inp = synth.make_gqa_inputs(cfg)
    res = oracle_mod.gqa_decode(inp)
    G = cfg.nq // cfg.nkv
    for b in range(cfg.B):
        slot = int(inp["block_table"][b, 0]) * cfg.block_size
        for qh in range(cfg.nq):
            h = qh // G
            v = cf.e4m3_value(inp["v_cache"].reshape(-1, cfg.nkv, cfg.D)[slot, h].numpy())
            expect = v * inp["v_scale"][b, h].double().numpy()
            np.testing.assert_allclose(res["out"][b, qh], expect, rtol=1e-15, atol=0)


def test_identical_keys_give_the_mean_value(oracle_mod):
    cfg = small_cfg(seed=9)
    inp = synth.make_gqa_inputs(cfg)
    k = inp["k_cache"].clone()
    k[...] = k[0, 0][None, None]
    ks = inp["k_scale"].clone()
    ks[...] = ks[0, 0][None, None]
    inp = dict(inp, k_cache=k, k_scale=ks)
    res = oracle_mod.gqa_decode(inp)
    G = cfg.nq // cfg.nkv
    for b in range(cfg.B):
        K, V, _ = cf.dense_kv(inp, b)
        for qh in range(cfg.nq):
            h = qh // G
            expect = cf.e4m3_value(V[:, h]).mean(axis=0) * inp["v_scale"][b, h].double().numpy()
            np.testing.assert_allclose(res["out"][b, qh], expect, rtol=1e-12, atol=1e-15)


def test_kv_head_mapping_contiguous_groups(oracle_mod):
    # V of KV head h is the constant (h+1) and all keys are equal (uniform
    # weights, every FP8 weight 448): query head qh must return qh // G + 1.
    cfg = small_cfg(nq=12, nkv=3, seed=12)
    inp = synth.make_gqa_inputs(cfg)
    k = inp["k_cache"].clone()
    k[...] = k[0, 0][None, None]
    ks = inp["k_scale"].clone()
    ks[...] = ks[0, 0][None, None]
    inp = dict(inp, k_cache=k, k_scale=ks)
    v = inp["v_cache"].clone()
    codes = [0x38, 0x40, 0x44]                        # 1.0, 2.0, 3.0
    for h in range(cfg.nkv):
        v[:, :, h, :] = codes[h]
    vs = torch.ones_like(inp["v_scale"])
    res = oracle_mod.gqa_decode(dict(inp, v_cache=v, v_scale=vs))
    for qh in range(cfg.nq):
        np.testing.assert_allclose(res["out"][:, qh], float(qh // 4 + 1), rtol=1e-15)


def test_empty_and_clamped_sequences(oracle_mod):
    cfg = small_cfg(seq_lens=(0, 513), seed=13)
    inp = synth.make_gqa_inputs(cfg)
    res = oracle_mod.gqa_decode(inp)
    assert np.all(res["out"][0] == 0.0)
    # a length beyond the table capacity is clamped to it
    cap = cfg.max_blocks_per_seq * cfg.block_size
    cfg2 = small_cfg(seq_lens=(200, cap), seed=13, num_blocks=12)
    inp2 = synth.make_gqa_inputs(cfg2)
    res2 = oracle_mod.gqa_decode(inp2)
    inp3 = dict(inp2, kv_act_seqs=torch.tensor([200, cap + 999], dtype=torch.int32))
    res3 = oracle_mod.gqa_decode(inp3)
    assert np.array_equal(res2["out"], res3["out"])


def test_multi_position_rows_share_the_sequence(oracle_mod):
    # s1 > 1 with no causal mask: each position is an independent query over [0, seq)
    cfg = small_cfg(s1=3, seed=14)
    inp = synth.make_gqa_inputs(cfg)
    res = oracle_mod.gqa_decode(inp)
    for b in range(cfg.B):
        for s in range(cfg.s1):
            for qh in (0, cfg.nq - 1):
                ref, _, _ = cf.closed_form_row(inp, b, s, qh, cfg.s2_tile)
                np.testing.assert_allclose(res["out"][b * cfg.s1 + s, qh], ref, rtol=1e-12, atol=1e-14)


def test_rows_entry_matches_batch_entry(oracle_mod, pin_inputs, pin_result):
    rows = [0, 5, 8, 15]
    r = oracle_mod.gqa_decode_rows(pin_inputs, rows)
    flat = pin_result["out"].reshape(-1, pin_inputs["cfg"].D)
    assert np.array_equal(r["out"], flat[rows])


@pytest.mark.parametrize("case", GOLDEN["p1_test_shapes"]["rows"][:1] + GOLDEN["p1_test_shapes"]["rows"][4:])
def test_page_test_shapes_closed_form(oracle_mod, case):
    # the page's own test shapes (sequence lengths shortened where huge), spot rows
    b, s1, s2, nq, nkv = case
    s2 = min(s2, 1024)
    nblk = (s2 + 127) // 128
    cfg = synth.GqaConfig("page-shape", B=b, s1=s1, nq=nq, nkv=nkv, seq_lens=tuple([s2] * b),
                          s2_tile=256, num_blocks=b * nblk, max_blocks_per_seq=nblk, seed=31)
    inp = synth.make_gqa_inputs(cfg)
    rows = [0, nq - 1, (b * s1 - 1) * nq]
    r = oracle_mod.gqa_decode_rows(inp, rows)
    for i, row in enumerate(rows):
        bb, s, qh = row // (s1 * nq), (row // nq) % s1, row % nq
        ref, _, _ = cf.closed_form_row(inp, bb, s, qh, 256)
        np.testing.assert_allclose(r["out"][i], ref, rtol=1e-12, atol=1e-14)


# ---------------------------------------------------------------------- MLA

def mla_small(**kw):
    base = dict(name="mla-pin", B=2, s1=1, nq=4, topk=96, seq_range=None, seq_lens=(300, 50),
                num_blocks=6, max_blocks_per_seq=3, s2_tile=32, seed=17)
    base.update(kw)
    return synth.MlaConfig(**base)


def test_mla_dequant_matches_reshape_form(oracle_mod):
    inp = synth.make_mla_inputs(mla_small())
    cache = inp["cache"].numpy()
    ref = cf.mla_dequant_rows(cache[:50])
    import ctypes
    out = np.zeros(576)
    for i in range(50):
        row = np.ascontiguousarray(cache[i])
        oracle_mod.lib().oracle_mla_dequant_row(row.ctypes.data_as(ctypes.c_void_p), out.ctypes.data_as(ctypes.c_void_p))
        assert np.array_equal(out, ref[i])


def test_mla_row_layout_constants():
    lay = GOLDEN["mla_row_layout"]
    assert lay["row_bytes"] == synth.MLA_ROW_BYTES == 512 + 64 * 2 + 4 * 4 + 16
    assert lay["nope"] == [0, synth.MLA_NOPE]
    assert lay["rope_bf16"] == [512, 512 + 2 * synth.MLA_ROPE]
    assert lay["scales_fp32"] == [640, 640 + 4 * synth.MLA_GROUPS]


@pytest.mark.parametrize("s2_tile", [32, 4096])
def test_mla_closed_form(oracle_mod, s2_tile):
    inp = synth.make_mla_inputs(mla_small(s2_tile=s2_tile))
    res = oracle_mod.mla_decode(inp)
    cfg = inp["cfg"]
    for b in range(cfg.B):
        for hq in range(cfg.nq):
            ref = cf.mla_closed_form_row(inp, b, 0, hq, s2_tile)
            np.testing.assert_allclose(res["out"][b * cfg.nq + hq], ref, rtol=1e-12, atol=1e-14)


@pytest.mark.parametrize("nkv", [2, 3])
def test_mla_kv_heads_read_their_own_slice(oracle_mod, nkv):
    """nkv KV heads: query head hq uses the top-k slice of KV head hq / (nq / nkv)
    (the page's topk_indices (t, n_kv*topk)); the closed form gathers that
    slice itself.  A dropped slice offset or a wrong head-to-slice mapping
    fails here, since the slices are drawn independently."""
    cfg = mla_small(nq=2 * nkv, nkv=nkv, s1=2, seq_lens=(200, 40), topk=64, seed=40 + nkv)
    inp = synth.make_mla_inputs(cfg)
    assert not np.array_equal(inp["topk"][:, :64].numpy(), inp["topk"][:, 64:128].numpy())
    res = oracle_mod.mla_decode(inp)
    for b in range(cfg.B):
        for s in range(cfg.s1):
            for hq in range(cfg.nq):
                ref = cf.mla_closed_form_row(inp, b, s, hq, cfg.s2_tile)
                np.testing.assert_allclose(res["out"][(b * cfg.s1 + s) * cfg.nq + hq], ref, rtol=1e-12, atol=1e-14)


def test_mla_valid_count_formula(oracle_mod):
    for seq, s1, s, topk, n in GOLDEN["mla_valid_count"]["cases"]:
        assert max(0, min(seq - s1 + 1 + s, topk)) == n
    # s1 = 2 and short sequences: position 0 sees one index fewer
    cfg = mla_small(s1=2, seq_lens=(15, 1), topk=32, seed=19)
    inp = synth.make_mla_inputs(cfg)
    res = oracle_mod.mla_decode(inp)
    for b in range(cfg.B):
        for s in range(2):
            for hq in range(cfg.nq):
                ref = cf.mla_closed_form_row(inp, b, s, hq, cfg.s2_tile)
                got = res["out"][(b * 2 + s) * cfg.nq + hq]
                np.testing.assert_allclose(got, ref, rtol=1e-12, atol=1e-14)
    assert np.all(res["out"][(1 * 2 + 0) * cfg.nq:(1 * 2 + 1) * cfg.nq] == 0)   # seq 1, s 0 -> n = 0


def test_mla_kv_split_planes_follow_the_row_layout():
    """synth.mla_kv_split cuts the three kv_split tensors at the byte ranges the
    page's 672-byte row layout names (nope, rope, scales)."""
    lay = GOLDEN["mla_row_layout"]
    cfg = synth.MlaConfig("split-pin", B=1, s1=1, nq=32, topk=64, seq_range=None, num_blocks=2,
                          max_blocks_per_seq=2, seq_lens=(100,), seed=2)
    inp = synth.make_mla_inputs(cfg)
    sp = synth.mla_kv_split(inp)
    cache = inp["cache"].numpy()
    lo, hi = lay["nope"]
    assert np.array_equal(sp["kn_quant"].numpy(), cache[:, lo:hi])
    lo, hi = lay["rope_bf16"]
    assert np.array_equal(sp["kr"].view(torch.int16).numpy().view(np.uint8).reshape(cache.shape[0], -1),
                          cache[:, lo:hi])
    lo, hi = lay["scales_fp32"]
    assert np.array_equal(sp["kn_scales"].numpy().view(np.uint8).reshape(cache.shape[0], -1), cache[:, lo:hi])


# ------------------------------------------------------- causal multi-token

def _causal_inp(seq_lens, s1, s2_tile=256, seed=31):
    cfg = small_cfg(B=len(seq_lens), s1=s1, nq=8, nkv=2, seq_lens=tuple(seq_lens), s2_tile=s2_tile,
                    num_blocks=6 * len(seq_lens) + 4, max_blocks_per_seq=6, seed=seed)
    return synth.make_gqa_inputs(cfg)


def test_causal_row_is_the_plain_decode_of_its_prefix(oracle_mod):
    """Position s of s1 is token seq - s1 + s of its sequence and sees tokens up to
    itself: its causal output equals the plain single-position decode of the
    same query over the first seq - s1 + 1 + s tokens, bit for bit."""
    s1 = 3
    inp = _causal_inp((300, 257, 2), s1)
    causal = oracle_mod.gqa_decode(dict(inp, causal=True))["out_bf16"]
    cfg = inp["cfg"]
    for b, seq in enumerate(cfg.seq_lens):
        for s in range(s1):
            n = max(0, seq - s1 + 1 + s)
            one = dict(inp, cfg=replace(cfg, B=1, s1=1, seq_lens=(n,)),
                       q=inp["q"][b * s1 + s:b * s1 + s + 1], q_scale=inp["q_scale"][b * s1 + s:b * s1 + s + 1],
                       block_table=inp["block_table"][b:b + 1], kv_act_seqs=torch.tensor([n], dtype=torch.int32),
                       v_scale=inp["v_scale"][b:b + 1])
            plain = oracle_mod.gqa_decode(one)["out_bf16"]
            assert np.array_equal(causal[b * s1 + s], plain[0]), (b, s, n)


def test_causal_with_one_position_is_the_plain_decode(oracle_mod):
    inp = _causal_inp((300, 513), 1)
    assert np.array_equal(oracle_mod.gqa_decode(dict(inp, causal=True))["out_bf16"],
                          oracle_mod.gqa_decode(inp)["out_bf16"])


def test_causal_positions_before_the_sequence_are_zero(oracle_mod):
    # seq = 2 with s1 = 4: positions 0 and 1 precede the sequence (n = -1, 0)
    inp = _causal_inp((2, 130), 4)
    out = oracle_mod.gqa_decode(dict(inp, causal=True))["out"]
    assert not out[0].any() and not out[1].any()
    assert np.abs(out[2]).sum() > 0 and np.abs(out[3]).sum() > 0
