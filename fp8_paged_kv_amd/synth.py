"""Seeded synthetic inputs for FP8 paged-attention decode.

This module is shared by the tests, the benchmark and the smoke check.  It
holds no step of the decode itself: it draws random tensors with torch's
seeded generators, rounds them with torch's own casts (``bfloat16``,
``float8_e4m3fn``) and lays them out as a paged cache.  Everything the decode
computes lives elsewhere (the HIP library) and is checked by the oracle.

Sources for the layouts and scale rules used to *prepare* inputs:
[P1] the web page "PyPTO 实现 GLM-4.5 Paged Attention FP8 量化算子分页 KV Cache
     与 E4M3 混合精度 Kernel 实战解析" (m.nxbn.cn/news/52221):
     - kernel signature section: q [B*S1, NQ, D], k/v caches
       [num_blocks, block_size, NKV, D], k_scale [num_blocks, block_size, NKV, 1],
       v_scale [B, NKV, D], block_table [B, max_blocks], kv_act_seqs [B];
     - quantisation-strategy section: K scaled per KV token, V per channel
       over the sequence, Q per token; scale = amax / 448 is stored as the
       dequantisation multiplier (the page stores 448/amax and uses its
       reciprocal to dequantise);
     - golden-reference section: the block table is a random permutation of
       the global block ids, unused entries are -1.
[P2] the web page "PyPTO-Gym 算子实战DeepSeek V32 MLA 的 Sparse Attention FP8
     反量化算子" (www.mhpn.cn/news/2272720), section "核心参数与 KV Cache 布局":
     the 672-byte cache row [0:512) e4m3 nope, [512:640) 64 bf16 rope,
     [640:656) four fp32 group scales, 16 bytes of padding.
[P3] the web page "CANN ops-transformer aclnnKvCompressEpilog 算子详解"
     (www.lmnt.cn/news/267091), section 参数说明: x [tokens, d] bf16 with
     d % 64 == 0, slotMapping [tokens] int32 / int64 (-1 = skip), cache
     [blockNum, blockSize, 1, headDim] uint8.
[P5] the web page on ops-transformer's scatter_pa_kv_cache_with_k_scale
     (www.lmnt.cn/news/278797), section 函数原型: key / value
     [num_tokens, num_head, head_size] FP8, key_scale [num_tokens, num_head]
     float, slot_mapping [num_tokens] int32 / int64 with distinct values.
"""
from __future__ import annotations

import math
import warnings
from dataclasses import dataclass, field, replace
from typing import Optional, Sequence

import torch

E4M3_MAX = 448.0            # [P1] key-features section: E4M3 range [-448, 448]
BLOCK_SIZE = 128            # [P1] semantic conventions: 128 tokens per block
MLA_ROW_BYTES = 672         # [P2] cache-layout table
MLA_NOPE = 512
MLA_ROPE = 64
MLA_GROUPS = 4


@dataclass(frozen=True)
class GqaConfig:
    """Shape and value recipe of one FP8 paged GQA decode workload."""
    name: str
    B: int
    s1: int
    nq: int
    nkv: int
    D: int = 128
    block_size: int = BLOCK_SIZE
    seq_lens: Optional[Sequence[int]] = None   # fixed lengths, or
    seq_range: Optional[tuple] = None          # inclusive uniform range
    s2_tile: int = 512
    num_blocks: int = 0                        # physical pool size
    max_blocks_per_seq: int = 0                # block_table row length
    outlier_frac: float = 0.0                  # fraction of (kv-head, channel) pairs scaled
    outlier_gain: float = 20.0
    seed: int = 0

    @property
    def group(self) -> int:
        return self.nq // self.nkv

    @property
    def softmax_scale(self) -> float:
        # [P1] configuration section: softmax_scale = qd ** -0.5
        return 1.0 / math.sqrt(self.D)


@dataclass(frozen=True)
class MlaConfig:
    """Shape recipe of the MLA-style sparse decode (one latent KV head)."""
    name: str
    B: int
    s1: int
    nq: int
    topk: int
    seq_range: tuple
    num_blocks: int
    max_blocks_per_seq: int
    block_size: int = BLOCK_SIZE
    s2_tile: int = 512
    seed: int = 4
    seq_lens: Optional[Sequence[int]] = None
    nkv: int = 1                               # KV heads, each with its own top-k slice

    @property
    def softmax_scale(self) -> float:
        return 1.0 / math.sqrt(MLA_NOPE + MLA_ROPE)


# The five workloads.  Config 0 is small enough for the oracle to finish in
# well under a second; 1-3 are the full-size GQA decode shapes; 4 is MLA.
CONFIGS = {
    0: GqaConfig("tiny-gqa-b2-nq8-nkv2", B=2, s1=1, nq=8, nkv=2, seq_lens=(200, 513),
                 s2_tile=256, num_blocks=8, max_blocks_per_seq=6, seed=0),
    1: GqaConfig("glm45-decode-b32-nq96-nkv8-seq1k-8k", B=32, s1=1, nq=96, nkv=8,
                 seq_range=(1024, 8192), s2_tile=512, num_blocks=2048, max_blocks_per_seq=64,
                 outlier_frac=0.01, seed=1),
    2: GqaConfig("long-decode-b4-nq96-nkv8-seq64k-128k", B=4, s1=1, nq=96, nkv=8,
                 seq_range=(65536, 131072), s2_tile=512, num_blocks=4096, max_blocks_per_seq=1024,
                 outlier_frac=0.01, seed=2),
    3: GqaConfig("multitoken-decode-b256-s1-4-nq32-nkv4-seq512-2k", B=256, s1=4, nq=32, nkv=4,
                 seq_range=(512, 2048), s2_tile=256, num_blocks=4096, max_blocks_per_seq=16, seed=3),
    4: MlaConfig("mla-sparse-b16-nq128-topk2048-seq4k-32k", B=16, s1=1, nq=128, topk=2048,
                 seq_range=(4096, 32768), num_blocks=4096, max_blocks_per_seq=256, seed=4),
}


def _gen(device, seed: int) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(int(seed))
    return g


def _draw_seq_lens(cfg, g, device) -> torch.Tensor:
    if cfg.seq_lens is not None:
        return torch.tensor(list(cfg.seq_lens), dtype=torch.int32)
    lo, hi = cfg.seq_range
    return torch.randint(lo, hi + 1, (cfg.B,), generator=g, device=device).to(torch.int32).cpu()


def _block_table(cfg, seqs: torch.Tensor, g, device, poison: bool):
    """Random permutation of the pool handed out in order; unused entries -1.

    Returns (block_table [B, max_blocks] int32 on cpu, owner[num_blocks] int64
    = batch owning each physical block or -1, used blocks per batch)."""
    bs = cfg.block_size
    need = [(int(s) + bs - 1) // bs for s in seqs.tolist()]
    assert all(n <= cfg.max_blocks_per_seq for n in need), "sequence longer than the table row"
    assert sum(need) <= cfg.num_blocks, "pool too small for the drawn lengths"
    perm = torch.randperm(cfg.num_blocks, generator=g, device=device).cpu()
    table = torch.full((cfg.B, cfg.max_blocks_per_seq), -1, dtype=torch.int32)
    owner = torch.full((cfg.num_blocks,), -1, dtype=torch.int64)
    pos = 0
    for b, n in enumerate(need):
        ids = perm[pos:pos + n]
        table[b, :n] = ids.to(torch.int32)
        owner[ids] = b
        pos += n
    if poison:
        # unused table entries hold arbitrary in-range ids; they must never be
        # read.  A separate generator keeps the valid data identical to the
        # unpoisoned draw of the same seed.
        gp = torch.Generator().manual_seed(0x5EED0000 + cfg.seed)
        extra = torch.randint(0, cfg.num_blocks, (cfg.B, cfg.max_blocks_per_seq),
                              generator=gp).to(torch.int32)
        unused = torch.arange(cfg.max_blocks_per_seq)[None, :] >= torch.tensor(need)[:, None]
        table = torch.where(unused, extra, table)
    return table, owner, need


def _slot_valid(cfg, seqs, table, need, device):
    """valid[num_blocks*bs] bool: slot holds a token p < seq of its owner."""
    bs = cfg.block_size
    valid = torch.zeros(cfg.num_blocks * bs, dtype=torch.bool)
    for b in range(cfg.B):
        n = need[b]
        if n == 0:
            continue
        ids = table[b, :n].to(torch.int64)
        slots = (ids[:, None] * bs + torch.arange(bs)[None, :]).reshape(-1)[: int(seqs[b])]
        valid[slots] = True
    return valid.to(device)


def _to_e4m3_codes(x: torch.Tensor) -> torch.Tensor:
    """torch's own float32 -> float8_e4m3fn cast, returned as raw uint8 codes."""
    return x.to(torch.float8_e4m3fn).view(torch.uint8)


def make_gqa_inputs(cfg: GqaConfig, device="cpu", seed: Optional[int] = None, poison: bool = False,
                    seq_lens: Optional[Sequence[int]] = None, keep_float: bool = False) -> dict:
    """Draw one seeded instance of ``cfg`` on ``device``.

    Recipe: Q ~ N(0,1) fp32 rounded to bf16; K, V ~ N(0,1) fp32 over the whole
    physical pool; a fraction ``outlier_frac`` of (kv-head, channel) pairs of K
    and (separately drawn) of V multiplied by ``outlier_gain``.  q_scale =
    amax|q| / 448 per (token, head); k_scale = amax|k| / 448 per (slot, kv
    head); v_scale = amax|v| / 448 per (batch, kv head, channel) over that
    batch's valid tokens.  Codes are torch's float8_e4m3fn cast of x / scale.
    With ``poison`` every slot that holds no valid token gets NaN codes
    (0x7F / 0xFF) and a NaN k_scale, and unused table entries get arbitrary
    in-range ids: the decode must not read any of them.
    """
    seed = cfg.seed if seed is None else seed
    if seq_lens is not None:
        cfg = replace(cfg, seq_lens=tuple(int(s) for s in seq_lens), seq_range=None)
    cfg = replace(cfg, seed=seed)
    g = _gen(device, seed)
    B, s1, nq, nkv, D, bs = cfg.B, cfg.s1, cfg.nq, cfg.nkv, cfg.D, cfg.block_size
    seqs = _draw_seq_lens(cfg, g, device)
    table, owner, need = _block_table(cfg, seqs, g, device, poison)
    nslots = cfg.num_blocks * bs

    q32 = torch.randn((B * s1, nq, D), generator=g, device=device, dtype=torch.float32)
    q = q32.to(torch.bfloat16)
    q_scale = q.float().abs().amax(dim=-1) / E4M3_MAX

    def outliers():
        n = int(round(cfg.outlier_frac * nkv * D))
        gain = torch.ones(nkv * D, device=device)
        if n:
            idx = torch.randperm(nkv * D, generator=g, device=device)[:n]
            gain[idx] = cfg.outlier_gain
        return gain.view(nkv, D)

    k = torch.randn((nslots, nkv, D), generator=g, device=device, dtype=torch.float32)
    k *= outliers()
    k_scale = k.abs().amax(dim=-1) / E4M3_MAX
    k_codes = _to_e4m3_codes(k / k_scale[..., None])
    k_float = k if keep_float else None
    del k

    v = torch.randn((nslots, nkv, D), generator=g, device=device, dtype=torch.float32)
    v *= outliers()
    valid = _slot_valid(cfg, seqs, table, need, device)
    owner_slot = owner.to(device).repeat_interleave(bs)
    owner_slot = torch.where(valid, owner_slot, torch.full_like(owner_slot, -1))
    amax = torch.zeros((B + 1, nkv, D), device=device)
    idx = (owner_slot + 1).clamp(min=0)                         # row 0 collects non-valid slots
    with warnings.catch_warnings():
        warnings.simplefilter("ignore")            # index_reduce is flagged beta
        amax.index_reduce_(0, idx, v.abs(), "amax", include_self=True)
    v_scale_all = amax / E4M3_MAX
    v_scale = v_scale_all[1:].contiguous()
    # A batch with no valid token has no data to scale; give it a unit scale.
    v_scale = torch.where(v_scale > 0, v_scale, torch.full_like(v_scale, 1.0 / E4M3_MAX))
    pool_scale = v.abs().amax(dim=0, keepdim=True) / E4M3_MAX   # for slots nobody owns
    per_slot = torch.where((owner_slot >= 0)[:, None, None], v_scale_all[idx], pool_scale)
    per_slot = torch.where(per_slot > 0, per_slot, pool_scale)
    v_codes = _to_e4m3_codes(v / per_slot)
    v_float = v if keep_float else None
    del v, per_slot

    if poison:
        bad = ~valid
        nan_codes = torch.where(torch.arange(D, device=device) % 2 == 0,
                                torch.tensor(0x7F, dtype=torch.uint8, device=device),
                                torch.tensor(0xFF, dtype=torch.uint8, device=device))
        k_codes[bad] = nan_codes
        v_codes[bad] = nan_codes
        k_scale[bad] = float("nan")

    return dict(
        cfg=cfg,
        q=q.contiguous(),
        q_scale=q_scale.contiguous(),
        k_cache=k_codes.view(cfg.num_blocks, bs, nkv, D).contiguous(),
        k_scale=k_scale.view(cfg.num_blocks, bs, nkv).contiguous(),
        v_cache=v_codes.view(cfg.num_blocks, bs, nkv, D).contiguous(),
        v_scale=v_scale.contiguous(),
        block_table=table.to(device),
        kv_act_seqs=seqs.to(device),
        softmax_scale=cfg.softmax_scale,
        k_float=None if k_float is None else k_float.view(cfg.num_blocks, bs, nkv, D),
        v_float=None if v_float is None else v_float.view(cfg.num_blocks, bs, nkv, D),
    )


def make_mla_inputs(cfg: MlaConfig, device="cpu", seed: Optional[int] = None,
                    seq_lens: Optional[Sequence[int]] = None) -> dict:
    """Draw one seeded MLA-style instance.

    Recipe: query nope/rope ~ N(0,1) rounded to bf16; per cache row the 512
    nope values ~ N(0,1) are quantised per 128-channel group with scale =
    amax/448 (torch's e4m3 cast), the 64 rope values ~ N(0,1) are stored as
    bf16; top-k indices per query token and KV head are drawn uniformly
    without replacement from [0, seq) (all of [0, seq) when seq <= topk,
    followed by -1 padding); topk is [B*s1, nkv*topk], KV head h's slice at
    columns [h*topk, (h+1)*topk).
    """
    seed = cfg.seed if seed is None else seed
    if seq_lens is not None:
        cfg = replace(cfg, seq_lens=tuple(int(s) for s in seq_lens), seq_range=None)
    g = _gen(device, seed)
    B, s1, nq, bs = cfg.B, cfg.s1, cfg.nq, cfg.block_size
    seqs = _draw_seq_lens(cfg, g, device)
    table, owner, need = _block_table(cfg, seqs, g, device, poison=False)
    nrows = cfg.num_blocks * bs

    qn = torch.randn((B * s1 * nq, MLA_NOPE), generator=g, device=device).to(torch.bfloat16)
    qr = torch.randn((B * s1 * nq, MLA_ROPE), generator=g, device=device).to(torch.bfloat16)

    kn = torch.randn((nrows, MLA_GROUPS, MLA_NOPE // MLA_GROUPS), generator=g, device=device)
    gscale = kn.abs().amax(dim=-1) / E4M3_MAX                  # [rows, 4]
    kn_codes = _to_e4m3_codes(kn / gscale[..., None]).view(nrows, MLA_NOPE)
    kr = torch.randn((nrows, MLA_ROPE), generator=g, device=device).to(torch.bfloat16)
    cache = torch.zeros((nrows, MLA_ROW_BYTES), dtype=torch.uint8, device=device)
    cache[:, :MLA_NOPE] = kn_codes
    cache[:, MLA_NOPE:MLA_NOPE + 2 * MLA_ROPE] = kr.view(torch.uint8).view(nrows, 2 * MLA_ROPE)
    cache[:, 640:656] = gscale.contiguous().view(torch.uint8).view(nrows, 16)
    del kn

    K = cfg.topk
    topk = torch.full((B * s1, cfg.nkv * K), -1, dtype=torch.int32)
    for b in range(B):
        sq = int(seqs[b])
        for s in range(s1):
            n = min(sq, K)
            if n == 0:
                continue
            for h in range(cfg.nkv):
                # uniform without replacement: first n of a random permutation
                sel = torch.randperm(sq, generator=g, device=device)[:n]
                topk[b * s1 + s, h * K:h * K + n] = sel.cpu().to(torch.int32)

    return dict(
        cfg=cfg,
        q_nope=qn.contiguous(),
        q_rope=qr.contiguous(),
        cache=cache,
        topk=topk.to(device),
        block_table=table.to(device),
        kv_act_seqs=seqs.to(device),
        softmax_scale=cfg.softmax_scale,
    )


def mla_kv_split(inp: dict) -> dict:
    """The same cache as [P2]'s kv_split sister operator holds it: three tensors
    (section 相关算子对比) -- kn_quant [rows, 512] e4m3 codes, kr [rows, 64] bf16,
    kn_scales [rows, 4] fp32 -- cut from the packed 672-byte rows (bytes
    0..511, 512..639 and 640..655)."""
    cache = inp["cache"]
    rows = cache.shape[0]
    return dict(inp,
                kn_quant=cache[:, :MLA_NOPE].contiguous(),
                kr=cache[:, MLA_NOPE:MLA_NOPE + 2 * MLA_ROPE].contiguous().view(torch.bfloat16).view(rows, MLA_ROPE),
                kn_scales=cache[:, 640:656].contiguous().view(torch.float32).view(rows, MLA_GROUPS))


def gqa_algorithmic_bytes(cfg: GqaConfig, seqs: Sequence[int]) -> int:
    """Bytes the decode must move at least once: for every valid (token, kv
    head) its K row, V row and k_scale; v_scale per (batch, kv head); Q
    (bf16) and q_scale and the bf16 output per query row; the block-table
    entries covering the valid tokens and the sequence lengths."""
    bs = cfg.block_size
    tok = sum(int(s) for s in seqs)
    blocks = sum((int(s) + bs - 1) // bs for s in seqs)
    return (tok * cfg.nkv * (2 * cfg.D + 4)
            + cfg.B * cfg.nkv * cfg.D * 4
            + cfg.B * cfg.s1 * cfg.nq * (2 * cfg.D + 4)
            + cfg.B * cfg.s1 * cfg.nq * 2 * cfg.D
            + 4 * blocks + 4 * cfg.B)


def mla_algorithmic_bytes(cfg: MlaConfig, seqs: Sequence[int]) -> int:
    """Gathered rows (656 used bytes each), the indices and table entries that
    address them, the bf16 queries (576 values) and bf16 outputs (512)."""
    n = 0
    for s in seqs:
        n += cfg.s1 * cfg.nkv * min(int(s), cfg.topk)
    rows = cfg.B * cfg.s1 * cfg.nq
    return n * (656 + 4 + 4) + rows * (MLA_NOPE + MLA_ROPE) * 2 + rows * MLA_NOPE * 2 + 4 * cfg.B


# ------------------------------------------------------------ cache writer

@dataclass(frozen=True)
class ScatterConfig:
    """Shape recipe of one call of the FP8 KV-cache writer ([P5])."""
    name: str
    num_tokens: int
    num_head: int
    k_head_size: int = 128
    v_head_size: int = 128
    num_blocks: int = 4
    block_size: int = BLOCK_SIZE
    layout: str = "BSND"          # BSND [nb, bs, H, d] (the decode's) or BNBD [nb, H, bs, d]
    slot_bits: int = 32
    skip: int = 0                 # tokens given a slot outside [0, num_blocks * block_size)
    seed: int = 0


def _random_codes(shape, g, device) -> torch.Tensor:
    """Uniform e4m3 codes without the two NaN codes (0x7F, 0xFF)."""
    c = torch.randint(0, 254, shape, generator=g, device=device, dtype=torch.int32)
    c = c + (c >= 0x7F).to(torch.int32)          # skip 0x7F; 0xFF is out of range already
    return c.to(torch.uint8)


def make_scatter_inputs(cfg: ScatterConfig, device="cpu", seed: Optional[int] = None) -> dict:
    """Draw one seeded writer call.

    Slots are distinct: the first num_tokens entries of a random permutation
    of the pool's slots.  ``skip`` randomly chosen tokens get a slot outside
    the pool instead (alternately -1 - k and num_slots + k - 1).  Keys and values
    are uniform e4m3 codes, key scales uniform in [1e-3, 1e-1), and the caches
    start filled with random bytes / values so that untouched positions are
    visible."""
    seed = cfg.seed if seed is None else seed
    g = _gen(device, seed)
    T, H, nb, bs = cfg.num_tokens, cfg.num_head, cfg.num_blocks, cfg.block_size
    nslots = nb * bs
    assert T <= nslots, "more tokens than cache slots"
    slots = torch.randperm(nslots, generator=g, device=device)[:T].to(torch.int64)
    if cfg.skip:
        which = torch.randperm(T, generator=g, device=device)[: cfg.skip]
        k = torch.arange(cfg.skip, device=device, dtype=torch.int64)
        slots[which] = torch.where(k % 2 == 0, -1 - k, nslots + k - 1)
    slots = slots.to(torch.int32 if cfg.slot_bits == 32 else torch.int64)
    key = _random_codes((T, H, cfg.k_head_size), g, device)
    value = _random_codes((T, H, cfg.v_head_size), g, device)
    key_scale = torch.rand((T, H), generator=g, device=device) * 0.099 + 0.001
    if cfg.layout == "BSND":
        kshape, vshape, sshape = (nb, bs, H, cfg.k_head_size), (nb, bs, H, cfg.v_head_size), (nb, bs, H)
    else:
        kshape, vshape, sshape = (nb, H, bs, cfg.k_head_size), (nb, H, bs, cfg.v_head_size), (nb, H, bs)
    key_cache = _random_codes(kshape, g, device)
    value_cache = _random_codes(vshape, g, device)
    key_scale_cache = torch.rand(sshape, generator=g, device=device)
    return dict(cfg=cfg, key=key, value=value, slot_mapping=slots, key_scale=key_scale,
                key_cache=key_cache, value_cache=value_cache, key_scale_cache=key_scale_cache)


def prefill_slots(cfg: GqaConfig, device="cpu", seed: Optional[int] = None) -> dict:
    """Slot mapping that writes every valid token of a GQA workload's sequences.

    Lengths and block table are drawn exactly as make_gqa_inputs draws them
    (same seed, same generator order), so writing per-token rows at these
    slots fills the pool positions the decode of that workload reads.  Token
    order is (batch, position); slot = table[b, p // 128] * 128 + p % 128."""
    seed = cfg.seed if seed is None else seed
    g = _gen(device, seed)
    seqs = _draw_seq_lens(cfg, g, device)
    table, _, need = _block_table(cfg, seqs, g, device, False)
    bs = cfg.block_size
    parts = []
    for b in range(cfg.B):
        n = int(seqs[b])
        if n == 0:
            continue
        p = torch.arange(n, dtype=torch.int64)
        parts.append(table[b, p // bs].to(torch.int64) * bs + p % bs)
    slots = torch.cat(parts) if parts else torch.zeros(0, dtype=torch.int64)
    return dict(slots=slots.to(torch.int32).to(device), seqs=seqs, block_table=table)


# ------------------------------------------------------- KvCompressEpilog

@dataclass(frozen=True)
class EpilogConfig:
    """Shape recipe of one KvCompressEpilog call ([P3])."""
    name: str
    num_tokens: int
    d: int
    block_num: int
    block_size: int
    head_dim: int
    quant_mode: int = 1
    round_scale: bool = True
    slot_bits: int = 32
    skip: int = 0                 # tokens given slot -1
    block_pad: int = 0            # extra bytes between blocks (a cache viewed inside a larger buffer)
    seed: int = 0


def make_epilog_inputs(cfg: EpilogConfig, device="cpu", seed: Optional[int] = None) -> dict:
    """Draw one seeded KvCompressEpilog call.

    x ~ N(0,1) in fp32 rounded to bf16, with per-(token, 64-column group) gains
    drawn log-uniformly over 2^-20 .. 2^20 (so the scales span many binades)
    and one group in 16 set to zero; slots are distinct (first tokens of a
    random permutation of the pool), ``skip`` of them -1; the cache starts as
    random bytes.  The cache is a flat byte buffer of block_num blocks of
    block_size * head_dim + block_pad bytes."""
    seed = cfg.seed if seed is None else seed
    g = _gen(device, seed)
    T, d = cfg.num_tokens, cfg.d
    nslots = cfg.block_num * cfg.block_size
    assert T <= nslots
    x = torch.randn((T, d // 64, 64), generator=g, device=device)
    gain = torch.exp2(torch.rand((T, d // 64, 1), generator=g, device=device) * 40 - 20)
    zero = torch.rand((T, d // 64, 1), generator=g, device=device) < 1 / 16
    x = torch.where(zero, torch.zeros_like(x), x * gain).reshape(T, d).to(torch.bfloat16)
    slots = torch.randperm(nslots, generator=g, device=device)[:T].to(torch.int64)
    if cfg.skip:
        which = torch.randperm(T, generator=g, device=device)[: cfg.skip]
        slots[which] = -1
    slots = slots.to(torch.int32 if cfg.slot_bits == 32 else torch.int64)
    block_stride = cfg.block_size * cfg.head_dim + cfg.block_pad
    cache = torch.randint(0, 256, (cfg.block_num * block_stride,), generator=g, device=device,
                          dtype=torch.int32).to(torch.uint8)
    return dict(cfg=cfg, x=x, slot_mapping=slots, cache=cache, block_stride=block_stride)
