"""Thin ctypes binding of libpa_fp8.so (the C ABI in include/pa_fp8.h).

Argument marshalling only: shapes are read off the torch tensors, pointers
and sizes are passed through, and every step of the decode runs in the HIP
library.  There is no fallback: if the library is missing or the tensors are
not on a GPU, the call raises.
"""
from __future__ import annotations

import ctypes
import os

import torch

PKG = os.path.dirname(os.path.abspath(__file__))
# PA_FP8_LIB selects another build of the same library (e.g. a tuning variant).
LIB_PATH = os.environ.get("PA_FP8_LIB") or os.path.join(PKG, "libpa_fp8.so")

PA_OK, PA_ERR_NULLPTR, PA_ERR_INVALID, PA_ERR_UNSUPPORTED, PA_ERR_WORKSPACE, PA_ERR_HIP = range(6)

EXPORTS = ("pa_fp8_decode_workspace_size", "pa_fp8_decode", "pa_fp8_decode_noalloc", "pa_fp8_decode_debug",
           "pa_fp8_decode_causal",
           "pa_fp8_mla_workspace_size", "pa_fp8_mla_sparse_decode",
           "pa_fp8_mla_sparse_decode_kv_split", "pa_fp8_scatter_kv_cache",
           "pa_fp8_kv_compress_epilog_workspace_size", "pa_fp8_kv_compress_epilog",
           "pa_fp8_last_error_string", "pa_fp8_last_error", "pa_fp8_version")

PA_CACHE_BSND, PA_CACHE_BNBD = 0, 1


class PaError(RuntimeError):
    def __init__(self, code: int, msg: str):
        super().__init__(f"pa_fp8 status {code}: {msg}")
        self.code = code


_lib = None


def lib():
    """Load the built library (never builds, never falls back)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with fp8_paged_kv_amd.build.build()")
        L = ctypes.CDLL(LIB_PATH)
        P, I, F, Z = ctypes.c_void_p, ctypes.c_int, ctypes.c_float, ctypes.c_size_t
        gqa = [P] * 9 + [I] * 6 + [F] + [I] * 4 + [P, Z]
        L.pa_fp8_decode.argtypes = gqa + [P]
        L.pa_fp8_decode.restype = I
        L.pa_fp8_decode_noalloc.argtypes = [P] * 9 + [I] * 6 + [F] + [I] * 4 + [P]
        L.pa_fp8_decode_noalloc.restype = I
        L.pa_fp8_decode_causal.argtypes = [P] * 9 + [I] * 6 + [F] + [I] * 4 + [P, Z, P]
        L.pa_fp8_decode_causal.restype = I
        L.pa_fp8_decode_debug.argtypes = gqa + [P, P, P]
        L.pa_fp8_decode_debug.restype = I
        L.pa_fp8_decode_workspace_size.argtypes = [I] * 9 + [P, P]
        L.pa_fp8_decode_workspace_size.restype = I
        L.pa_fp8_mla_workspace_size.argtypes = [I] * 5 + [P]
        L.pa_fp8_mla_workspace_size.restype = I
        L.pa_fp8_mla_sparse_decode.argtypes = [P] * 7 + [I] * 8 + [F, I, P, Z, P]
        L.pa_fp8_mla_sparse_decode.restype = I
        L.pa_fp8_mla_sparse_decode_kv_split.argtypes = [P] * 9 + [I] * 8 + [F, I, P, Z, P]
        L.pa_fp8_mla_sparse_decode_kv_split.restype = I
        L.pa_fp8_scatter_kv_cache.argtypes = [P] * 7 + [I] * 8 + [ctypes.c_int64] * 4 + [P]
        L.pa_fp8_scatter_kv_cache.restype = I
        L.pa_fp8_kv_compress_epilog_workspace_size.argtypes = [I] * 5 + [ctypes.c_int64, I, I, P]
        L.pa_fp8_kv_compress_epilog_workspace_size.restype = I
        L.pa_fp8_kv_compress_epilog.argtypes = [P] * 3 + [I] * 5 + [ctypes.c_int64] + [I] * 4 + [F, P, Z, P]
        L.pa_fp8_kv_compress_epilog.restype = I
        L.pa_fp8_last_error_string.argtypes = []
        L.pa_fp8_last_error_string.restype = ctypes.c_char_p
        L.pa_fp8_last_error.argtypes = []
        L.pa_fp8_last_error.restype = ctypes.c_char_p
        L.pa_fp8_version.argtypes = []
        L.pa_fp8_version.restype = ctypes.c_char_p
        _lib = L
    return _lib


def _check(rc: int):
    if rc != PA_OK:
        raise PaError(rc, lib().pa_fp8_last_error_string().decode())


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def workspace_size(B, s1, nq, nkv, D, block_size, max_blocks_per_seq, s2_tile, num_splits=0):
    """(bytes, splits) the decode needs for these sizes."""
    n = ctypes.c_size_t(0)
    s = ctypes.c_int(0)
    _check(lib().pa_fp8_decode_workspace_size(B, s1, nq, nkv, D, block_size, max_blocks_per_seq, s2_tile,
                                              num_splits, ctypes.byref(n), ctypes.byref(s)))
    return n.value, s.value


def _shapes(q, k_cache, block_table, kv_act_seqs, s1):
    B = int(kv_act_seqs.shape[0])
    nq, D = int(q.shape[1]), int(q.shape[2])
    num_blocks, block_size, nkv = int(k_cache.shape[0]), int(k_cache.shape[1]), int(k_cache.shape[2])
    if s1 is None:
        if q.shape[0] % B:
            raise ValueError("q rows are not a multiple of the batch size")
        s1 = int(q.shape[0]) // B          # [P1] kernel signature: s1 = (B*S1) // B
    return B, s1, nq, nkv, D, block_size, num_blocks, int(block_table.shape[1])


def _checked_inputs(ts):
    for name, t in ts.items():
        if t is None:
            continue
        if not t.is_cuda:
            raise ValueError(f"{name} must be a GPU tensor")
        if not t.is_contiguous():
            raise ValueError(f"{name} must be contiguous")


def decode(q, q_scale, k_cache, k_scale, v_cache, v_scale, block_table, kv_act_seqs, softmax_scale,
           s2_tile, num_splits=0, out=None, workspace=None, stream=None, s1=None, causal=False):
    """FP8 paged decode; returns out [B*s1, nq, D] bf16 (allocated if not given).
    causal=True: pa_fp8_decode_causal (position s of s1 sees the first seq - s1 + 1 + s tokens)."""
    B, s1, nq, nkv, D, bs, nblk, mbps = _shapes(q, k_cache, block_table, kv_act_seqs, s1)
    _checked_inputs(dict(q=q, q_scale=q_scale, k_cache=k_cache, k_scale=k_scale, v_cache=v_cache,
                         v_scale=v_scale, block_table=block_table, kv_act_seqs=kv_act_seqs, out=out,
                         workspace=workspace))
    if out is None:
        out = torch.empty((B * s1, nq, D), dtype=torch.bfloat16, device=q.device)
    need, _ = workspace_size(B, s1, nq, nkv, D, bs, mbps, s2_tile, num_splits)
    if workspace is None and need:
        workspace = torch.zeros(need, dtype=torch.uint8, device=q.device)
    wbytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    if causal:
        _check(lib().pa_fp8_decode_causal(
            _ptr(q), _ptr(q_scale), _ptr(k_cache), _ptr(k_scale), _ptr(v_cache), _ptr(v_scale),
            _ptr(block_table), _ptr(kv_act_seqs), _ptr(out), B, s1, nq, nkv, D, bs, float(softmax_scale),
            int(s2_tile), mbps, nblk, int(num_splits), _ptr(workspace), wbytes, _stream(stream)))
        return out
    _check(lib().pa_fp8_decode(
        _ptr(q), _ptr(q_scale), _ptr(k_cache), _ptr(k_scale), _ptr(v_cache), _ptr(v_scale),
        _ptr(block_table), _ptr(kv_act_seqs), _ptr(out), B, s1, nq, nkv, D, bs, float(softmax_scale),
        int(s2_tile), mbps, nblk, int(num_splits), _ptr(workspace), wbytes, _stream(stream)))
    return out


def decode_noalloc(q, q_scale, k_cache, k_scale, v_cache, v_scale, block_table, kv_act_seqs, softmax_scale,
                   s2_tile, num_splits=0, out=None, stream=None, s1=None):
    """pa_fp8_decode_noalloc: the decode with the library's own scratch instead of a
    workspace (allocates nothing when ``out`` is given)."""
    B, s1, nq, nkv, D, bs, nblk, mbps = _shapes(q, k_cache, block_table, kv_act_seqs, s1)
    _checked_inputs(dict(q=q, q_scale=q_scale, k_cache=k_cache, k_scale=k_scale, v_cache=v_cache,
                         v_scale=v_scale, block_table=block_table, kv_act_seqs=kv_act_seqs, out=out))
    if out is None:
        out = torch.empty((B * s1, nq, D), dtype=torch.bfloat16, device=q.device)
    _check(lib().pa_fp8_decode_noalloc(
        _ptr(q), _ptr(q_scale), _ptr(k_cache), _ptr(k_scale), _ptr(v_cache), _ptr(v_scale),
        _ptr(block_table), _ptr(kv_act_seqs), _ptr(out), B, s1, nq, nkv, D, bs, float(softmax_scale),
        int(s2_tile), mbps, nblk, int(num_splits), _stream(stream)))
    return out


def decode_noalloc_inputs(inp: dict, num_splits=0, out=None, stream=None):
    """decode_noalloc() on a dict produced by fp8_paged_kv_amd.synth.make_gqa_inputs."""
    return decode_noalloc(inp["q"], inp["q_scale"], inp["k_cache"], inp["k_scale"], inp["v_cache"], inp["v_scale"],
                          inp["block_table"], inp["kv_act_seqs"], inp["softmax_scale"],
                          inp.get("s2_tile", inp["cfg"].s2_tile), num_splits=num_splits, out=out, stream=stream,
                          s1=inp["cfg"].s1)


def decode_debug(q, q_scale, k_cache, k_scale, v_cache, v_scale, block_table, kv_act_seqs, softmax_scale,
                 s2_tile, num_splits=0, stream=None, s1=None):
    """decode plus the in-kernel dumps: (out, rows [B, max_blocks*block_size] int32, q8 codes)."""
    B, s1, nq, nkv, D, bs, nblk, mbps = _shapes(q, k_cache, block_table, kv_act_seqs, s1)
    _checked_inputs(dict(q=q, k_cache=k_cache, block_table=block_table, kv_act_seqs=kv_act_seqs))
    out = torch.empty((B * s1, nq, D), dtype=torch.bfloat16, device=q.device)
    rows = torch.empty((B, mbps * bs), dtype=torch.int32, device=q.device)
    q8 = torch.zeros((B * s1, nq, D), dtype=torch.uint8, device=q.device)
    need, _ = workspace_size(B, s1, nq, nkv, D, bs, mbps, s2_tile, num_splits)
    workspace = torch.zeros(need, dtype=torch.uint8, device=q.device) if need else None
    _check(lib().pa_fp8_decode_debug(
        _ptr(q), _ptr(q_scale), _ptr(k_cache), _ptr(k_scale), _ptr(v_cache), _ptr(v_scale),
        _ptr(block_table), _ptr(kv_act_seqs), _ptr(out), B, s1, nq, nkv, D, bs, float(softmax_scale),
        int(s2_tile), mbps, nblk, int(num_splits), _ptr(workspace), need, _ptr(rows), _ptr(q8),
        _stream(stream)))
    return out, rows, q8


def decode_inputs(inp: dict, num_splits=0, out=None, workspace=None, stream=None):
    """decode() on a dict produced by fp8_paged_kv_amd.synth.make_gqa_inputs (inp["causal"] selects
    the causal variant)."""
    return decode(inp["q"], inp["q_scale"], inp["k_cache"], inp["k_scale"], inp["v_cache"], inp["v_scale"],
                  inp["block_table"], inp["kv_act_seqs"], inp["softmax_scale"],
                  inp.get("s2_tile", inp["cfg"].s2_tile), num_splits=num_splits, out=out, workspace=workspace,
                  stream=stream, s1=inp["cfg"].s1, causal=bool(inp.get("causal", False)))


def mla_workspace_size(B, s1, nq, topk, s2_tile):
    n = ctypes.c_size_t(0)
    _check(lib().pa_fp8_mla_workspace_size(B, s1, nq, topk, s2_tile, ctypes.byref(n)))
    return n.value


def mla_decode(q_nope, q_rope, cache, topk, block_table, kv_act_seqs, softmax_scale, s2_tile, s1,
               out=None, workspace=None, stream=None, block_size=128, nkv=1):
    """MLA sparse decode; topk [B*s1, nkv*topk]; returns out [B*s1*nq, 512] bf16 (allocated if not given)."""
    B = int(kv_act_seqs.shape[0])
    nq = int(q_nope.shape[0]) // (B * s1)
    K = int(topk.shape[1]) // nkv
    _checked_inputs(dict(q_nope=q_nope, q_rope=q_rope, cache=cache, topk=topk, block_table=block_table,
                         kv_act_seqs=kv_act_seqs, out=out, workspace=workspace))
    if out is None:
        out = torch.empty((B * s1 * nq, 512), dtype=torch.bfloat16, device=q_nope.device)
    need = mla_workspace_size(B, s1, nq, K, s2_tile)
    if workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=q_nope.device)
    _check(lib().pa_fp8_mla_sparse_decode(
        _ptr(q_nope), _ptr(q_rope), _ptr(cache), _ptr(topk), _ptr(block_table), _ptr(kv_act_seqs), _ptr(out),
        B, s1, nq, nkv, K, block_size, int(block_table.shape[1]), int(cache.shape[0]) // block_size,
        float(softmax_scale), int(s2_tile), _ptr(workspace), workspace.numel() * workspace.element_size(),
        _stream(stream)))
    return out


def mla_decode_kv_split(q_nope, q_rope, kn_quant, kr, kn_scales, topk, block_table, kv_act_seqs, softmax_scale,
                        s2_tile, s1, out=None, workspace=None, stream=None, block_size=128, nkv=1):
    """MLA sparse decode over the kv_split cache (kn_quant [rows, 512] uint8,
    kr [rows, 64] bf16, kn_scales [rows, 4] float32); returns out [B*s1*nq, 512] bf16."""
    B = int(kv_act_seqs.shape[0])
    nq = int(q_nope.shape[0]) // (B * s1)
    K = int(topk.shape[1]) // nkv
    _checked_inputs(dict(q_nope=q_nope, q_rope=q_rope, kn_quant=kn_quant, kr=kr, kn_scales=kn_scales, topk=topk,
                         block_table=block_table, kv_act_seqs=kv_act_seqs, out=out, workspace=workspace))
    if kn_quant.shape[1] != 512 or kr.shape[1] != 64 or kn_scales.shape[1] != 4:
        raise ValueError("kv_split planes must be [rows, 512], [rows, 64], [rows, 4]")
    if out is None:
        out = torch.empty((B * s1 * nq, 512), dtype=torch.bfloat16, device=q_nope.device)
    need = mla_workspace_size(B, s1, nq, K, s2_tile)
    if workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=q_nope.device)
    _check(lib().pa_fp8_mla_sparse_decode_kv_split(
        _ptr(q_nope), _ptr(q_rope), _ptr(kn_quant), _ptr(kr), _ptr(kn_scales), _ptr(topk), _ptr(block_table),
        _ptr(kv_act_seqs), _ptr(out), B, s1, nq, nkv, K, block_size, int(block_table.shape[1]),
        int(kn_quant.shape[0]) // block_size, float(softmax_scale), int(s2_tile), _ptr(workspace),
        workspace.numel() * workspace.element_size(), _stream(stream)))
    return out


def mla_decode_kv_split_inputs(inp: dict, out=None, workspace=None, stream=None):
    """mla_decode_kv_split() on a dict from synth.mla_kv_split(synth.make_mla_inputs(...))."""
    cfg = inp["cfg"]
    return mla_decode_kv_split(inp["q_nope"], inp["q_rope"], inp["kn_quant"], inp["kr"], inp["kn_scales"],
                               inp["topk"], inp["block_table"], inp["kv_act_seqs"], inp["softmax_scale"],
                               inp.get("s2_tile", cfg.s2_tile), cfg.s1, out=out, workspace=workspace,
                               stream=stream, block_size=cfg.block_size, nkv=cfg.nkv)


def mla_decode_inputs(inp: dict, out=None, workspace=None, stream=None):
    """mla_decode() on a dict produced by fp8_paged_kv_amd.synth.make_mla_inputs."""
    cfg = inp["cfg"]
    return mla_decode(inp["q_nope"], inp["q_rope"], inp["cache"], inp["topk"], inp["block_table"],
                      inp["kv_act_seqs"], inp["softmax_scale"], inp.get("s2_tile", cfg.s2_tile), cfg.s1,
                      out=out, workspace=workspace, stream=stream, block_size=cfg.block_size, nkv=cfg.nkv)


def scatter_kv_cache(key, value, key_cache, value_cache, slot_mapping, key_scale, key_scale_cache,
                     layout: str = "BSND", stream=None):
    """In-place FP8 KV-cache write (pa_fp8_scatter_kv_cache).

    key [T, H, dk] / value [T, H, dv]: uint8 or float8_e4m3fn, rows may be
    strided over tokens (each token's [H, d] block contiguous); key_scale
    [T, H] float32, any strides; slot_mapping [T] int32 / int64.
    layout "BSND": caches [nb, bs, H, d], key_scale_cache [nb, bs, H];
    layout "BNBD": caches [nb, H, bs, d], key_scale_cache [nb, H, bs] or [nb, H, bs, 1]."""
    T, H, dk = (int(x) for x in key.shape)
    dv = int(value.shape[2])
    for name, t, d in (("key", key, dk), ("value", value, dv)):
        if t.element_size() != 1 or t.stride(2) != 1 or t.stride(1) != d:
            raise ValueError(f"{name}: one-byte codes with each token's [H, d] block contiguous")
    for name, t in (("key_cache", key_cache), ("value_cache", value_cache), ("key_scale_cache", key_scale_cache)):
        if not t.is_contiguous():
            raise ValueError(f"{name} must be contiguous")
    if key_scale.dtype != torch.float32 or key_scale_cache.dtype != torch.float32:
        raise ValueError("key_scale and key_scale_cache must be float32")
    if slot_mapping.dtype not in (torch.int32, torch.int64):
        raise ValueError("slot_mapping must be int32 or int64")
    lay = {"BSND": PA_CACHE_BSND, "BNBD": PA_CACHE_BNBD}[layout]
    nb = int(key_cache.shape[0])
    bs = int(key_cache.shape[1] if lay == PA_CACHE_BSND else key_cache.shape[2])
    for name, t in (("key", key), ("value", value), ("key_scale", key_scale), ("slot_mapping", slot_mapping)):
        if not t.is_cuda:
            raise ValueError(f"{name} must be a GPU tensor")
    _checked_inputs(dict(key_cache=key_cache, value_cache=value_cache, key_scale_cache=key_scale_cache,
                         slot_mapping=slot_mapping))
    _check(lib().pa_fp8_scatter_kv_cache(
        _ptr(key), _ptr(value), _ptr(key_cache), _ptr(value_cache), _ptr(slot_mapping), _ptr(key_scale),
        _ptr(key_scale_cache), T, H, dk, dv, nb, bs, 32 if slot_mapping.dtype == torch.int32 else 64, lay,
        key.stride(0), value.stride(0), key_scale.stride(0), key_scale.stride(1), _stream(stream)))


def scatter_inputs(inp: dict, stream=None):
    """scatter_kv_cache() on a dict produced by fp8_paged_kv_amd.synth.make_scatter_inputs
    (updates the dict's caches in place)."""
    scatter_kv_cache(inp["key"], inp["value"], inp["key_cache"], inp["value_cache"], inp["slot_mapping"],
                     inp["key_scale"], inp["key_scale_cache"], inp["cfg"].layout, stream=stream)


def kv_compress_epilog(cache, x, slot_mapping, block_num, block_size, head_dim, block_stride=None, quant_mode=1,
                       round_scale=True, quant_group_size=64, x_scale=1.0, stream=None):
    """KvCompressEpilog modes 0/1 (pa_fp8_kv_compress_epilog), in place.

    cache: a uint8 tensor holding block_num blocks (block_stride bytes apart,
    default block_size * head_dim) of block_size rows of head_dim bytes --
    e.g. [block_num, block_size, 1, head_dim]; x [tokens, d] bf16;
    slot_mapping [tokens] int32 / int64."""
    T, d = (int(v) for v in x.shape)
    if x.dtype != torch.bfloat16 or not x.is_contiguous():
        raise ValueError("x must be a contiguous bf16 tensor")
    if cache.dtype != torch.uint8 or slot_mapping.dtype not in (torch.int32, torch.int64):
        raise ValueError("cache must be uint8, slot_mapping int32 or int64")
    stride = block_size * head_dim if block_stride is None else int(block_stride)
    if cache.numel() < (block_num - 1) * stride + block_size * head_dim:
        raise ValueError("cache smaller than its blocks")
    _checked_inputs(dict(cache=cache, x=x, slot_mapping=slot_mapping))
    n = ctypes.c_size_t(0)
    _check(lib().pa_fp8_kv_compress_epilog_workspace_size(T, d, block_num, block_size, head_dim, stride,
                                                          quant_group_size, quant_mode, ctypes.byref(n)))
    _check(lib().pa_fp8_kv_compress_epilog(
        _ptr(cache), _ptr(x), _ptr(slot_mapping), T, d, block_num, block_size, head_dim, stride,
        32 if slot_mapping.dtype == torch.int32 else 64, quant_group_size, quant_mode, 1 if round_scale else 0,
        float(x_scale), None, 0, _stream(stream)))


def epilog_inputs(inp: dict, stream=None):
    """kv_compress_epilog() on a dict from synth.make_epilog_inputs (updates inp["cache"] in place)."""
    c = inp["cfg"]
    kv_compress_epilog(inp["cache"], inp["x"], inp["slot_mapping"], c.block_num, c.block_size, c.head_dim,
                       block_stride=inp["block_stride"], quant_mode=c.quant_mode, round_scale=c.round_scale,
                       stream=stream)
