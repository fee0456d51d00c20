"""Independent closed forms used to pin the oracle (test code only).

Nothing here calls the oracle.  E4M3 and BF16 rounding use torch's own
casts (library routines), the dense K/V gather copies whole blocks into a
contiguous per-sequence layout, and the attention sums are written in the
closed forms the online recurrence must reduce to:

  one tile   : out = vs * sum_p E4M3(448 e^{S_p - m}) v_p / (448 sum_p e^{S_p - m})
  many tiles : out = vs * sum_t e^{m_t - M} / 448 * sum_{p in t} E4M3(448 e^{S_p - m_t}) v_p
                       / sum_p e^{S_p - M}

with m_t the max of S over tile t and M the max over the sequence.  The
second holds because the per-row P scale of a tile is max_t P / 448, so the
FP8 weights of a tile only depend on that tile's own max (the running max
cancels).
"""
from __future__ import annotations

import numpy as np
import torch


def e4m3_round(x) -> np.ndarray:
    """Value of torch's float32 -> float8_e4m3fn cast (RNE), as float64."""
    t = torch.as_tensor(np.asarray(x, dtype=np.float32))
    return t.to(torch.float8_e4m3fn).to(torch.float32).double().numpy()


def e4m3_value(codes) -> np.ndarray:
    t = torch.as_tensor(np.asarray(codes, dtype=np.uint8)).view(torch.float8_e4m3fn)
    return t.to(torch.float32).double().numpy()


def bf16_value(t) -> np.ndarray:
    return t.detach().cpu().float().double().numpy()


def bf16_round(x) -> np.ndarray:
    t = torch.as_tensor(np.asarray(x, dtype=np.float32))
    return t.to(torch.bfloat16).float().double().numpy()


def dense_kv(inp, b):
    """Concatenate the blocks of sequence b into [seq, nkv, D] arrays
    (block-wise copy, the way a BSND rebuild of a paged cache is done)."""
    cfg = inp["cfg"]
    bs = cfg.block_size
    seq = int(inp["kv_act_seqs"][b])
    table = inp["block_table"][b].cpu().numpy()
    nblk = (seq + bs - 1) // bs
    kc = inp["k_cache"].cpu().numpy()
    vc = inp["v_cache"].cpu().numpy()
    ks = inp["k_scale"].cpu().numpy()
    K = np.concatenate([kc[max(int(table[i]), 0)] for i in range(nblk)], axis=0)[:seq] if nblk else np.zeros((0, cfg.nkv, cfg.D), np.uint8)
    V = np.concatenate([vc[max(int(table[i]), 0)] for i in range(nblk)], axis=0)[:seq] if nblk else np.zeros((0, cfg.nkv, cfg.D), np.uint8)
    KS = np.concatenate([ks[max(int(table[i]), 0)] for i in range(nblk)], axis=0)[:seq] if nblk else np.zeros((0, cfg.nkv), np.float32)
    return K, V, KS


def q_codes_value(inp, row_q):
    """E4M3 value of q / q_scale for query row (b*s1+s, qh): float32 divide then torch cast."""
    q = inp["q"].float()[row_q[0], row_q[1]]
    qs = inp["q_scale"][row_q[0], row_q[1]]
    return e4m3_round((q / qs).numpy())


def scores(inp, b, s, qh):
    """S_p for every valid token p of batch b, query position s, query head qh."""
    cfg = inp["cfg"]
    G = cfg.nq // cfg.nkv
    h = qh // G
    K, V, KS = dense_kv(inp, b)
    qv = q_codes_value(inp, (b * cfg.s1 + s, qh))
    qs = float(inp["q_scale"][b * cfg.s1 + s, qh])
    kv = e4m3_value(K[:, h, :])
    return (kv @ qv) * qs * KS[:, h].astype(np.float64) * float(inp["softmax_scale"]), V[:, h, :]


def closed_form_row(inp, b, s, qh, s2_tile):
    """Multi-tile closed form of the output row (FP64), its L and M."""
    cfg = inp["cfg"]
    G = cfg.nq // cfg.nkv
    h = qh // G
    S, V = scores(inp, b, s, qh)
    vs = inp["v_scale"][b, h].double().numpy()
    n = S.shape[0]
    if n == 0:
        return np.zeros(cfg.D), 0.0, -np.inf
    M = S.max()
    vv = e4m3_value(V)
    acc = np.zeros(cfg.D)
    for lo in range(0, n, s2_tile):
        St = S[lo:lo + s2_tile]
        mt = St.max()
        w = e4m3_round(448.0 * np.exp(St - mt))
        acc += np.exp(mt - M) / 448.0 * (w @ vv[lo:lo + s2_tile])
    L = np.exp(S - M).sum()
    return acc * vs / L, L, M


def exact_attention_row(inp, b, s, qh):
    """FP64 softmax attention on the unquantised fp32 K/V (needs keep_float inputs)."""
    cfg = inp["cfg"]
    G = cfg.nq // cfg.nkv
    h = qh // G
    bs = cfg.block_size
    seq = int(inp["kv_act_seqs"][b])
    table = inp["block_table"][b].cpu().numpy()
    kf = inp["k_float"].cpu().numpy()
    vf = inp["v_float"].cpu().numpy()
    nblk = (seq + bs - 1) // bs
    K = np.concatenate([kf[int(table[i])] for i in range(nblk)], axis=0)[:seq, h].astype(np.float64)
    V = np.concatenate([vf[int(table[i])] for i in range(nblk)], axis=0)[:seq, h].astype(np.float64)
    q = inp["q"].float()[b * cfg.s1 + s, qh].double().numpy()
    S = K @ q * float(inp["softmax_scale"])
    w = np.exp(S - S.max())
    return (w @ V) / w.sum()


# ------------------------------------------------------------------ MLA

def mla_dequant_rows(cache_rows: np.ndarray) -> np.ndarray:
    """[n, 672] bytes -> [n, 576] K = [kn | kr]: the page's reshape(-1, 128)
    times the per-group fp32 scale (fp32 multiply), cast to bf16; rope bytes
    reinterpreted as bf16."""
    n = cache_rows.shape[0]
    if n == 0:
        return np.zeros((0, 576))
    codes = torch.as_tensor(np.ascontiguousarray(cache_rows[:, :512]))
    kn32 = codes.view(torch.float8_e4m3fn).to(torch.float32).reshape(-1, 128)
    sc = torch.as_tensor(np.ascontiguousarray(cache_rows[:, 640:656])).view(torch.float32).reshape(-1, 1)
    kn = (kn32 * sc).to(torch.bfloat16).reshape(n, 512).double().numpy()
    kr = torch.as_tensor(np.ascontiguousarray(cache_rows[:, 512:640])).view(torch.bfloat16).double().numpy()
    return np.concatenate([kn, kr], axis=1)


def mla_gather(inp, b, s, h=0):
    """Dequantised K rows KV head h reads for query position s of batch b (its
    top-k slice is columns [h*topk, h*topk + n) of the index row)."""
    cfg = inp["cfg"]
    bs = cfg.block_size
    seq = int(inp["kv_act_seqs"][b])
    n = max(0, min(seq - cfg.s1 + 1 + s, cfg.topk))
    idx = inp["topk"][b * cfg.s1 + s, h * cfg.topk:h * cfg.topk + n].cpu().numpy().astype(np.int64)
    table = inp["block_table"][b].cpu().numpy().astype(np.int64)
    rows = table[idx // bs] * bs + idx % bs
    cache = inp["cache"].cpu().numpy()
    return mla_dequant_rows(cache[rows])


def mla_closed_form_row(inp, b, s, hq, s2_tile):
    cfg = inp["cfg"]
    K = mla_gather(inp, b, s, hq // (cfg.nq // cfg.nkv))
    r = (b * cfg.s1 + s) * cfg.nq + hq
    q = np.concatenate([inp["q_nope"][r].float().double().numpy(), inp["q_rope"][r].float().double().numpy()])
    n = K.shape[0]
    if n == 0:
        return np.zeros(512)
    S = (K @ q) * float(inp["softmax_scale"])
    M = S.max()
    acc = np.zeros(512)
    for lo in range(0, n, s2_tile):
        St = S[lo:lo + s2_tile]
        mt = St.max()
        pb = bf16_round(np.exp(St - mt))
        acc += np.exp(mt - M) * (pb @ K[lo:lo + s2_tile, :512])
    return acc / np.exp(S - M).sum()
