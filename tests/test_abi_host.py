"""CPU-only checks of the C ABI: the library loads, exports every declared
entry point, and rejects bad arguments on the host before any launch."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "pa_fp8.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(pa_fp8_\w+)\s*\(", text)))


@pytest.fixture(scope="module")
def lib():
    from fp8_paged_kv_amd import binding
    if not os.path.exists(binding.LIB_PATH):
        from fp8_paged_kv_amd import build
        build.build()
    return binding.lib()


def test_header_declares_expected_entry_points():
    from fp8_paged_kv_amd import binding
    assert set(declared_functions()) == set(binding.EXPORTS)


def test_library_exports_every_declared_symbol(lib):
    for name in declared_functions():
        assert hasattr(lib, name), name


def test_version(lib):
    assert lib.pa_fp8_version().decode().startswith("pa_fp8")


FAKE = ctypes.c_void_p(0x1000)      # never dereferenced: validation fails first


def call(lib, **over):
    a = dict(q=FAKE, qs=FAKE, k=FAKE, ks=FAKE, v=FAKE, vs=FAKE, table=FAKE, seqs=FAKE, out=FAKE,
             B=2, s1=1, nq=8, nkv=2, D=128, bs=128, scale=0.088, tile=256, mbps=6, nblocks=8, splits=1,
             ws=None, wsb=0, stream=None)
    a.update(over)
    return lib.pa_fp8_decode(a["q"], a["qs"], a["k"], a["ks"], a["v"], a["vs"], a["table"], a["seqs"], a["out"],
                             a["B"], a["s1"], a["nq"], a["nkv"], a["D"], a["bs"], a["scale"], a["tile"],
                             a["mbps"], a["nblocks"], a["splits"], a["ws"], a["wsb"], a["stream"])


@pytest.mark.parametrize("over,code", [
    (dict(q=None), 1), (dict(out=None), 1), (dict(table=None), 1),
    (dict(B=0), 2), (dict(nq=7), 2), (dict(tile=200), 2), (dict(splits=-1), 2), (dict(nblocks=0), 2),
    (dict(scale=0.0), 2), (dict(scale=float("inf")), 2), (dict(scale=float("nan")), 2),
    (dict(D=64), 3), (dict(bs=64, tile=256), 3), (dict(tile=384), 3), (dict(s1=65536 * 16, nq=4, nkv=2), 3),
    (dict(splits=2, ws=None), 4), (dict(splits=2, ws=FAKE, wsb=16), 4),
])
def test_host_validation_codes(lib, over, code):
    assert call(lib, **over) == code
    assert len(lib.pa_fp8_last_error_string()) > 0


def test_workspace_query(lib):
    from fp8_paged_kv_amd import binding
    n, s = binding.workspace_size(2, 1, 8, 2, 128, 128, 6, 256, 1)
    assert (n, s) == (0, 1)
    n, s = binding.workspace_size(2, 1, 8, 2, 128, 128, 6, 256, 3)
    assert s == 3 and n >= 2 * 8 * 3 * (128 * 4 + 8)
    n, s = binding.workspace_size(4, 1, 96, 8, 128, 128, 1024, 512, 0)
    assert 1 <= s <= 256 and n > 0
    with pytest.raises(binding.PaError):
        binding.workspace_size(2, 1, 8, 3, 128, 128, 6, 256, 1)


ALIGNED = ctypes.c_void_p(0x10000)   # 16-byte aligned, never dereferenced


def scatter(lib, **over):
    a = dict(k=ALIGNED, v=ALIGNED, kc=ALIGNED, vc=ALIGNED, slots=ALIGNED, ks=ALIGNED, ksc=ALIGNED,
             T=4, H=8, dk=128, dv=128, nb=2, bs=16, bits=32, layout=1, kst=1024, vst=1024, kst_s=8, ksh_s=1,
             stream=None)
    a.update(over)
    return lib.pa_fp8_scatter_kv_cache(a["k"], a["v"], a["kc"], a["vc"], a["slots"], a["ks"], a["ksc"], a["T"],
                                       a["H"], a["dk"], a["dv"], a["nb"], a["bs"], a["bits"], a["layout"],
                                       a["kst"], a["vst"], a["kst_s"], a["ksh_s"], a["stream"])


@pytest.mark.parametrize("over,code", [
    (dict(k=None), 1), (dict(slots=None), 1), (dict(ksc=None), 1),
    (dict(T=0), 2), (dict(H=0), 2), (dict(nb=0), 2), (dict(bs=-1), 2), (dict(bits=16), 2), (dict(layout=2), 2),
    (dict(kst=512), 2), (dict(vst=1000), 2), (dict(kst_s=-1), 2),
    (dict(dk=120, kst=960), 3), (dict(kst=1032), 3), (dict(k=ctypes.c_void_p(0x10008)), 3),
    (dict(bits=64, slots=ctypes.c_void_p(0x10004)), 3),
])
def test_scatter_host_validation_codes(lib, over, code):
    assert scatter(lib, **over) == code
    assert len(lib.pa_fp8_last_error_string()) > 0


def epilog(lib, **over):
    a = dict(cache=ALIGNED, x=ALIGNED, slots=ALIGNED, T=1024, d=256, nb=128, bs=16, hd=384, bstride=16 * 384,
             bits=32, gs=64, mode=1, rs=1, xs=1.0, stream=None)
    a.update(over)
    return lib.pa_fp8_kv_compress_epilog(a["cache"], a["x"], a["slots"], a["T"], a["d"], a["nb"], a["bs"], a["hd"],
                                         a["bstride"], a["bits"], a["gs"], a["mode"], a["rs"], a["xs"], None, 0,
                                         a["stream"])


@pytest.mark.parametrize("over,code", [
    (dict(cache=None), 1), (dict(x=None), 1), (dict(slots=None), 1),
    (dict(T=0), 2), (dict(d=200), 2), (dict(d=64), 2), (dict(d=8256), 2), (dict(hd=322), 2),
    (dict(mode=0, hd=326), 2), (dict(mode=3), 2), (dict(bits=8), 2), (dict(bstride=100), 2),
    (dict(mode=2, gs=8), 2), (dict(mode=2), 3), (dict(x=ctypes.c_void_p(0x10008)), 3),
])
def test_epilog_host_validation_codes(lib, over, code):
    assert epilog(lib, **over) == code
    assert len(lib.pa_fp8_last_error_string()) > 0


def test_epilog_page_row_sizes_accepted(lib):
    """The page's worked values: head_dim 323 (d = 256) and 583 (d = 512) are
    exactly enough in mode 1, one byte less is rejected."""
    n = ctypes.c_size_t(7)
    for d, col in ((256, 323), (512, 583)):
        assert lib.pa_fp8_kv_compress_epilog_workspace_size(4, d, 2, 16, col, 16 * col, 64, 1, ctypes.byref(n)) == 0
        assert n.value == 0
        assert lib.pa_fp8_kv_compress_epilog_workspace_size(4, d, 2, 16, col - 1, 16 * col, 64, 1,
                                                            ctypes.byref(n)) == 2


def causal(lib, **over):
    a = dict(B=2, s1=2, nq=64, nkv=2, tile=256, mbps=6, nblocks=8, splits=3, ws=None, wsb=0, q=FAKE)
    a.update(over)
    return lib.pa_fp8_decode_causal(a["q"], FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, a["B"], a["s1"], a["nq"],
                                    a["nkv"], 128, 128, 0.088, a["tile"], a["mbps"], a["nblocks"], a["splits"],
                                    a["ws"], a["wsb"], None)


@pytest.mark.parametrize("over,code", [
    (dict(q=None), 1), (dict(splits=-1), 2), (dict(nq=63), 2),
    (dict(s1=65536 * 32), 3),                      # more query rows per KV head than the row blocks cover
    (dict(ws=None), 4),                            # per-head path with 3 splits needs a workspace
    (dict(s1=512, nq=96, nkv=8, splits=2, ws=FAKE, wsb=1024), 4),
])
def test_causal_host_validation_codes(lib, over, code):
    """Causal decode takes the per-head path too (any number of query rows per
    KV head, explicit splits); its arguments are checked like pa_fp8_decode's."""
    assert causal(lib, **over) == code
    assert len(lib.pa_fp8_last_error_string()) > 0


def test_prefill_workspace_grows_with_row_blocks(lib):
    """More than 64 query rows per KV head: blocks of 32 rows, each (batch, KV
    head, row block) with its own partials and arrival counter."""
    from fp8_paged_kv_amd import binding
    n1, s1_ = binding.workspace_size(2, 8, 64, 2, 128, 128, 16, 256, 3)     # 256 rows per KV head: 8 blocks
    n2, _ = binding.workspace_size(2, 4, 64, 2, 128, 128, 16, 256, 3)      # 128 rows: 4 blocks
    assert s1_ == 3 and n1 > n2 > 0
    units = 2 * 2 * 8
    assert n1 >= units * 3 * 32 * (128 + 2) * 4


def mla(lib, **over):
    a = dict(qn=ALIGNED, qr=ALIGNED, cache=ALIGNED, topk=ALIGNED, table=ALIGNED, seqs=ALIGNED, out=ALIGNED,
             B=2, s1=1, nq=64, nkv=2, K=512, bs=128, mbps=8, nb=16, scale=0.04, tile=512, ws=ALIGNED,
             wsb=1 << 30, stream=None)
    a.update(over)
    return lib.pa_fp8_mla_sparse_decode(a["qn"], a["qr"], a["cache"], a["topk"], a["table"], a["seqs"], a["out"],
                                        a["B"], a["s1"], a["nq"], a["nkv"], a["K"], a["bs"], a["mbps"], a["nb"],
                                        a["scale"], a["tile"], a["ws"], a["wsb"], a["stream"])


@pytest.mark.parametrize("over,code", [
    (dict(qn=None), 1), (dict(topk=None), 1), (dict(cache=None), 1),
    (dict(B=0), 2), (dict(nkv=0), 2), (dict(nkv=3), 2), (dict(K=0), 2), (dict(scale=-1.0), 2),
    (dict(nkv=4), 3), (dict(nq=48, nkv=1), 3), (dict(tile=1024), 3), (dict(bs=64), 3),
    (dict(out=ctypes.c_void_p(0x10008)), 3), (dict(ws=None), 4), (dict(wsb=16), 4),
])
def test_mla_host_validation_codes(lib, over, code):
    """nq / nkv query heads per KV head must come in blocks of 32 (nkv = 4 with
    nq = 64 leaves 16); nkv must divide nq."""
    assert mla(lib, **over) == code
    assert len(lib.pa_fp8_last_error_string()) > 0


def test_last_error_names_agree(lib):
    assert call(lib, B=0) == 2
    assert lib.pa_fp8_last_error_string() == lib.pa_fp8_last_error()


def noalloc(lib, **over):
    a = dict(q=FAKE, qs=FAKE, k=FAKE, ks=FAKE, v=FAKE, vs=FAKE, table=FAKE, seqs=FAKE, out=FAKE,
             B=2, s1=1, nq=8, nkv=2, D=128, bs=128, scale=0.088, tile=256, mbps=6, nblocks=8, splits=1, stream=None)
    a.update(over)
    return lib.pa_fp8_decode_noalloc(a["q"], a["qs"], a["k"], a["ks"], a["v"], a["vs"], a["table"], a["seqs"],
                                     a["out"], a["B"], a["s1"], a["nq"], a["nkv"], a["D"], a["bs"], a["scale"],
                                     a["tile"], a["mbps"], a["nblocks"], a["splits"], a["stream"])


@pytest.mark.parametrize("over,code", [
    (dict(q=None), 1), (dict(seqs=None), 1), (dict(B=0), 2), (dict(nq=7), 2), (dict(D=64), 3),
    # per-head path with 64 splits of 64 rows for 64 sequences: about 136 MB of partials
    (dict(B=64, nq=64, nkv=1, mbps=1024, splits=64), 4),
])
def test_noalloc_host_validation_codes(lib, over, code):
    """The no-allocation entry point rejects bad arguments, and a call whose
    workspace exceeds the library's scratch, before touching the device."""
    assert noalloc(lib, **over) == code
    msg = lib.pa_fp8_last_error_string()
    assert len(msg) > 0
    if code == 4:
        assert b"scratch" in msg


def test_lds_probe_rejects_out_of_range_patterns():
    """The LDS read-pattern probe (a measurement tool beside the library) checks on the
    host that every lane's address stays inside its 64 KB buffer: a stride that would
    leave it, a stride not a multiple of 8, a bad width or pattern returns
    hipErrorInvalidValue (1) before anything is launched."""
    from fp8_paged_kv_amd import build
    if not os.path.exists(build.PROBE_LIB):
        build.build_probe()
    P = ctypes.CDLL(build.PROBE_LIB)
    P.pa_probe_lds_pattern.argtypes = [ctypes.c_int] * 5 + [ctypes.c_void_p, ctypes.c_void_p]
    P.pa_probe_lds_pattern.restype = ctypes.c_int
    bad = [(3, 528, 16),     # 63 lanes x 528 bytes > 32 KB base range
           (1, 2200, 16),    # 15 rows x 2200 bytes
           (1, 272, 12),     # width neither 8 nor 16
           (4, 16, 16),      # no such pattern
           (1, 270, 16),     # stride not a multiple of 8
           (0, 0, 0)]
    for pat, stride, width in bad:
        assert P.pa_probe_lds_pattern(pat, stride, width, 512, 16, None, None) == 1, (pat, stride, width)
    assert P.pa_probe_lds_pattern(0, 0, 16, 0, 16, None, None) == 1          # empty grid
