"""Python front of the C oracle (oracle/pa_oracle.c) — TEST INFRASTRUCTURE ONLY.

Only tests, the smoke check and the benchmark's CPU-baseline leg import this
module.  It marshals numpy arrays into the plain-C oracle through ctypes and
runs independent batches on a thread pool (the C calls release the GIL).
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from concurrent.futures import ThreadPoolExecutor

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "pa_oracle.c")
LIB = os.path.join(HERE, "liboracle.so")

_lib = None


def default_threads() -> int:
    """Worker threads: the CPUs this process may run on, at most 16 (one GPU's
    share of a shared host)."""
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:
        n = os.cpu_count() or 1
    return max(1, min(n, 16))


def build(force: bool = True) -> str:
    """Compile the oracle with gcc (no fast-math, no FMA contraction)."""
    if force or not os.path.exists(LIB):
        tmp = LIB + ".tmp"
        subprocess.check_call(["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-ffp-contract=off",
                               "-Wall", "-o", tmp, SRC, "-lm"])
        os.replace(tmp, LIB)
    return LIB


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(LIB):
            build(force=True)
        L = ctypes.CDLL(LIB)
        P = ctypes.c_void_p
        I = ctypes.c_int
        L.oracle_e4m3_decode.argtypes = [ctypes.c_uint8]
        L.oracle_e4m3_decode.restype = ctypes.c_double
        L.oracle_e4m3_encode.argtypes = [ctypes.c_double]
        L.oracle_e4m3_encode.restype = ctypes.c_uint8
        L.oracle_bf16_encode.argtypes = [ctypes.c_double]
        L.oracle_bf16_encode.restype = ctypes.c_uint16
        L.oracle_bf16_decode.argtypes = [ctypes.c_uint16]
        L.oracle_bf16_decode.restype = ctypes.c_double
        L.oracle_mla_dequant_row.argtypes = [P, P]
        L.oracle_mla_dequant_row.restype = None
        L.oracle_pa_fp8_decode.argtypes = [P] * 8 + [I] * 6 + [ctypes.c_double] + [I] * 6 + [P] * 6
        L.oracle_pa_fp8_decode.restype = I
        L.oracle_pa_fp8_decode_rows.argtypes = ([P] * 8 + [I] * 6 + [ctypes.c_double] + [I] * 4
                                                + [P, I] + [P] * 4)
        L.oracle_pa_fp8_decode_rows.restype = I
        L.oracle_mla_sparse_decode.argtypes = [P] * 6 + [I] * 8 + [ctypes.c_double] + [I] * 3 + [P] * 2
        L.oracle_mla_sparse_decode.restype = I
        L.oracle_kv_compress_row_bytes.argtypes = [I, I]
        L.oracle_kv_compress_row_bytes.restype = I
        L.oracle_kv_compress_cache_col.argtypes = [I, I]
        L.oracle_kv_compress_cache_col.restype = I
        L.oracle_kv_compress_epilog.argtypes = [P, P, P] + [I] * 5 + [ctypes.c_int64, I, I]
        L.oracle_kv_compress_epilog.restype = I
        L.oracle_scatter_kv_cache.argtypes = [P] * 7 + [I] * 7 + [ctypes.c_int64] * 4
        L.oracle_scatter_kv_cache.restype = I
        _lib = L
    return _lib


def _ptr(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _np(x, dtype):
    """torch tensor / numpy array -> contiguous numpy array of ``dtype`` (bit view for bf16)."""
    try:
        import torch
        if isinstance(x, torch.Tensor):
            x = x.detach().cpu()
            if x.dtype == torch.bfloat16:
                x = x.view(torch.int16)
            x = x.contiguous().numpy()
    except ImportError:
        pass
    x = np.ascontiguousarray(x)
    if x.dtype != dtype:
        x = x.view(dtype) if x.dtype.itemsize == np.dtype(dtype).itemsize and x.dtype.kind in "iu" else x.astype(dtype)
    return np.ascontiguousarray(x)


def e4m3_decode(codes) -> np.ndarray:
    L = lib()
    c = np.asarray(codes, dtype=np.uint8)
    return np.array([L.oracle_e4m3_decode(int(v)) for v in c.reshape(-1)]).reshape(c.shape)


def e4m3_encode(x) -> np.ndarray:
    L = lib()
    a = np.asarray(x, dtype=np.float64)
    return np.array([L.oracle_e4m3_encode(float(v)) for v in a.reshape(-1)], dtype=np.uint8).reshape(a.shape)


def bf16_encode(x) -> np.ndarray:
    L = lib()
    a = np.asarray(x, dtype=np.float64)
    return np.array([L.oracle_bf16_encode(float(v)) for v in a.reshape(-1)], dtype=np.uint16).reshape(a.shape)


def bf16_decode(h) -> np.ndarray:
    a = np.asarray(h, dtype=np.uint16).astype(np.uint32) << 16
    return a.view(np.float32).astype(np.float64)


def _gqa_arrays(inp):
    cfg = inp["cfg"]
    return dict(
        q=_np(inp["q"], np.uint16), q_scale=_np(inp["q_scale"], np.float32),
        k=_np(inp["k_cache"], np.uint8), ks=_np(inp["k_scale"], np.float32),
        v=_np(inp["v_cache"], np.uint8), vs=_np(inp["v_scale"], np.float32),
        table=_np(inp["block_table"], np.int32), seqs=_np(inp["kv_act_seqs"], np.int32),
        B=cfg.B, s1=cfg.s1, nq=cfg.nq, nkv=cfg.nkv, D=cfg.D, bs=cfg.block_size,
        scale=float(inp["softmax_scale"]), s2_tile=int(inp.get("s2_tile", cfg.s2_tile)),
        max_blocks=int(inp["block_table"].shape[1]), num_blocks=int(inp["k_cache"].shape[0]),
        causal=1 if inp.get("causal", False) else 0,
    )


def gqa_decode(inp, threads: int = None, b_range=None) -> dict:
    """Run the oracle over every batch (or ``b_range``) of a GQA input dict."""
    L = lib()
    a = _gqa_arrays(inp)
    B, s1, nq, D = a["B"], a["s1"], a["nq"], a["D"]
    out = np.zeros((B * s1, nq, D), dtype=np.float64)
    out_bf = np.zeros((B * s1, nq, D), dtype=np.uint16)
    q8 = np.zeros((B * s1, nq, D), dtype=np.uint8)
    M = np.zeros((B * s1, nq), dtype=np.float64)
    Ls = np.zeros((B * s1, nq), dtype=np.float64)
    rows = np.zeros((B, a["max_blocks"] * a["bs"]), dtype=np.int32)
    lo, hi = b_range if b_range is not None else (0, B)
    threads = threads or min(default_threads(), max(1, hi - lo))

    def run(rng):
        rc = L.oracle_pa_fp8_decode(
            _ptr(a["q"]), _ptr(a["q_scale"]), _ptr(a["k"]), _ptr(a["ks"]), _ptr(a["v"]), _ptr(a["vs"]),
            _ptr(a["table"]), _ptr(a["seqs"]), B, s1, nq, a["nkv"], D, a["bs"], a["scale"],
            a["s2_tile"], a["max_blocks"], a["num_blocks"], a["causal"], rng[0], rng[1],
            _ptr(out), _ptr(out_bf), _ptr(q8), _ptr(M), _ptr(Ls), _ptr(rows))
        if rc != 0:
            raise ValueError(f"oracle_pa_fp8_decode rc={rc}")

    chunks = [(b, b + 1) for b in range(lo, hi)]
    with ThreadPoolExecutor(max_workers=threads) as ex:
        list(ex.map(run, chunks))
    return dict(out=out, out_bf16=out_bf, q8=q8, M=M, L=Ls, rows=rows, threads=threads)


def gqa_decode_rows(inp, rows, threads: int = None) -> dict:
    """Oracle for the listed query rows only (row = (b*s1 + s)*nq + qh)."""
    L = lib()
    a = _gqa_arrays(inp)
    rows = np.ascontiguousarray(np.asarray(rows, dtype=np.int64))
    n, D = rows.shape[0], a["D"]
    out = np.zeros((n, D), dtype=np.float64)
    out_bf = np.zeros((n, D), dtype=np.uint16)
    M = np.zeros(n)
    Ls = np.zeros(n)
    threads = threads or min(default_threads(), max(1, n))
    # rows dealt round-robin in chunks of 8, so that threads share long and short sequences
    parts = [np.concatenate([np.arange(c, min(c + 8, n)) for c in range(8 * t, n, 8 * threads)] or
                            [np.zeros(0, dtype=np.int64)]) for t in range(threads)]

    def run(idx):
        if len(idx) == 0:
            return
        k = len(idx)
        sub = np.ascontiguousarray(rows[idx])
        o = np.zeros((k, D)); ob = np.zeros((k, D), dtype=np.uint16)
        m = np.zeros(k); l = np.zeros(k)
        rc = L.oracle_pa_fp8_decode_rows(
            _ptr(a["q"]), _ptr(a["q_scale"]), _ptr(a["k"]), _ptr(a["ks"]), _ptr(a["v"]), _ptr(a["vs"]),
            _ptr(a["table"]), _ptr(a["seqs"]), a["B"], a["s1"], a["nq"], a["nkv"], D, a["bs"], a["scale"],
            a["s2_tile"], a["max_blocks"], a["num_blocks"], a["causal"], _ptr(sub), k,
            _ptr(o), _ptr(ob), _ptr(m), _ptr(l))
        if rc != 0:
            raise ValueError(f"oracle_pa_fp8_decode_rows rc={rc}")
        out[idx] = o; out_bf[idx] = ob; M[idx] = m; Ls[idx] = l

    with ThreadPoolExecutor(max_workers=threads) as ex:
        list(ex.map(run, parts))
    return dict(out=out, out_bf16=out_bf, M=M, L=Ls, threads=threads)


def mla_decode(inp, threads: int = None, b_range=None) -> dict:
    """Run the MLA oracle over every batch (or ``b_range``) of an MLA input dict."""
    L = lib()
    cfg = inp["cfg"]
    qn = _np(inp["q_nope"], np.uint16)
    qr = _np(inp["q_rope"], np.uint16)
    cache = _np(inp["cache"], np.uint8)
    topk = _np(inp["topk"], np.int32)
    table = _np(inp["block_table"], np.int32)
    seqs = _np(inp["kv_act_seqs"], np.int32)
    B, s1, nq = cfg.B, cfg.s1, cfg.nq
    nkv = int(getattr(cfg, "nkv", 1))
    K = topk.shape[1] // nkv
    s2_tile = int(inp.get("s2_tile", cfg.s2_tile))
    out = np.zeros((B * s1 * nq, 512), dtype=np.float64)
    out_bf = np.zeros((B * s1 * nq, 512), dtype=np.uint16)
    lo, hi = b_range if b_range is not None else (0, B)
    threads = threads or min(default_threads(), max(1, hi - lo))

    def run(rng):
        rc = L.oracle_mla_sparse_decode(
            _ptr(qn), _ptr(qr), _ptr(cache), _ptr(topk), _ptr(table), _ptr(seqs),
            B, s1, nq, nkv, K, cfg.block_size, table.shape[1], cache.shape[0] // cfg.block_size,
            float(inp["softmax_scale"]), s2_tile, rng[0], rng[1], _ptr(out), _ptr(out_bf))
        if rc != 0:
            raise ValueError(f"oracle_mla_sparse_decode rc={rc}")

    with ThreadPoolExecutor(max_workers=threads) as ex:
        list(ex.map(run, [(b, b + 1) for b in range(lo, hi)]))
    return dict(out=out, out_bf16=out_bf, threads=threads)


def scatter_kv_cache(key, value, key_cache, value_cache, slot_mapping, key_scale, key_scale_cache,
                     layout: str = "BSND") -> dict:
    """The [P5] cache writer on copies of the given caches.

    ``key`` [T, H, dk] and ``value`` [T, H, dv] hold e4m3 codes (uint8 or
    float8 tensors / arrays), ``key_scale`` [T, H] float32 (any strides),
    ``slot_mapping`` [T] int32 or int64.  Caches: BSND ``[nb, bs, H, d]`` with
    scales ``[nb, bs, H]``, or BNBD ``[nb, H, bs, d]`` with scales
    ``[nb, H, bs]`` (a trailing axis of 1 is accepted).  Returns the updated
    copies and the number of tokens written.
    """
    k = _np(key, np.uint8)
    v = _np(value, np.uint8)
    kc = _np(key_cache, np.uint8).copy()
    vc = _np(value_cache, np.uint8).copy()
    slots = np.ascontiguousarray(_slots64(slot_mapping))
    ks = _np(key_scale, np.float32)
    ksc = _np(key_scale_cache, np.float32).copy()
    T, H, dk = k.shape
    dv = v.shape[2]
    lay = {"BSND": 0, "BNBD": 1}[layout]
    if lay == 0:
        nb, bs = kc.shape[0], kc.shape[1]
    else:
        nb, bs = kc.shape[0], kc.shape[2]
    n = lib().oracle_scatter_kv_cache(_ptr(k), _ptr(v), _ptr(kc), _ptr(vc), _ptr(slots), _ptr(ks), _ptr(ksc),
                                      T, H, dk, dv, nb, bs, lay, H * dk, H * dv, H, 1)
    if n < 0:
        raise ValueError("oracle_scatter_kv_cache rejected its arguments")
    return dict(key_cache=kc, value_cache=vc, key_scale_cache=ksc, written=n)


def _slots64(slot_mapping) -> np.ndarray:
    try:
        import torch
        if isinstance(slot_mapping, torch.Tensor):
            return slot_mapping.detach().cpu().to(torch.int64).numpy()
    except ImportError:
        pass
    return np.asarray(slot_mapping).astype(np.int64)


def kv_compress_row_bytes(d: int, mode: int) -> int:
    return lib().oracle_kv_compress_row_bytes(int(d), int(mode))


def kv_compress_cache_col(d: int, mode: int) -> int:
    return lib().oracle_kv_compress_cache_col(int(d), int(mode))


def kv_compress_epilog(cache, x, slot_mapping, mode: int, round_scale: bool = True, block_stride=None) -> dict:
    """[P3] KvCompressEpilog modes 0/1 on a copy of ``cache``.

    cache: [block_num, block_size, 1, head_dim] uint8 (a block stride in bytes
    may be given for a cache viewed inside a larger buffer: then ``cache`` is
    the flat buffer); x: [tokens, d] bf16 (or its int16 bits); slot_mapping
    [tokens] int32 / int64.  Returns the updated copy and the written count."""
    c = _np(cache, np.uint8).copy()
    xs = _np(x, np.uint16)
    slots = np.ascontiguousarray(_slots64(slot_mapping))
    T, d = xs.shape
    if block_stride is None:
        nb, bs, _, hd = c.shape
        stride = bs * hd
    else:
        nb, bs, hd, stride = block_stride
    n = lib().oracle_kv_compress_epilog(_ptr(c), _ptr(xs), _ptr(slots), T, d, nb, bs, hd, stride, int(mode),
                                        1 if round_scale else 0)
    if n < 0:
        raise ValueError("oracle_kv_compress_epilog rejected its arguments")
    return dict(cache=c, written=n)
