"""The C ABI without a GPU: the library loads, exports every function include/idx.h
declares, and its host-side checks reject bad arguments before any launch (each
call here fails a check, so nothing reaches the device).

With IDX_TEST_LIB naming the ABI layer built for the host under AddressSanitizer and
UndefinedBehaviorSanitizer (tests/host_asan, run by tests/test_host_asan.py), the same
tests run against that build, and the tests at the end also pretend a gfx950 is present:
every valid call then reaches exactly its kernel launchers (stand-ins that check the
arguments the kernels rely on) and no rejected call reaches one."""

import ctypes
import os
import re

import pytest

from sparse_attention_indexer_mxfp4_amd import _abi

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "idx.h")
HOST_LIB = os.environ.get("IDX_TEST_LIB")


def _gpu_visible():
    if HOST_LIB:
        return False  # the host build reports no device unless a test asks for one
    import torch

    return torch.cuda.is_available()

OK, NULL, SHAPE, STRIDE, FORMAT, WORKSPACE, LAUNCH, DEVICE = range(8)
P = 0x10000  # an aligned, never-dereferenced stand-in address


@pytest.fixture(scope="module")
def lib():
    if HOST_LIB:
        handle = ctypes.CDLL(HOST_LIB)
        _abi._declare(handle)
        return handle
    if _gpu_visible():
        # some calls here pass every host check with stand-in addresses (P): with a
        # device present they would launch kernels on memory that does not exist
        pytest.skip("argument-check tests use stand-in device addresses; they run where no GPU is visible")
    return _abi.lib()


def _declared():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"^\s*(?:const\s+)?[\w\s\*]*?\b(idx_\w+)\s*\(", text, re.M)))


def test_exports_every_declared_function(lib):
    names = _declared()
    assert "idx_mqa_logits" in names and "idx_topk" in names
    for name in names:
        assert hasattr(lib, name), name
    assert sorted(names) == sorted(_abi.EXPORTS)


@pytest.mark.skipif(bool(HOST_LIB), reason="the measurement library is not part of the ABI layer")
def test_calibration_library_exports():
    # the measurement kernels bench.py reports beside the spec peaks (include/idx_calib.h)
    text = open(os.path.join(ROOT, "include", "idx_calib.h")).read()
    names = sorted(set(re.findall(r"^\s*int32_t\s+(idx_calib_\w+)\s*\(", text, re.M)))
    assert names == ["idx_calib_copy", "idx_calib_mfma", "idx_calib_mfma_sink_words", "idx_calib_read",
                     "idx_calib_read_sink_words"]
    calib = ctypes.CDLL(os.path.join(ROOT, "sparse_attention_indexer_mxfp4_amd", "libidx_calib.so"))
    for name in names:
        assert hasattr(calib, name), name
    assert calib.idx_calib_read_sink_words() == 8192 and calib.idx_calib_mfma_sink_words() == 8192
    # argument checks come before any device call
    calib.idx_calib_copy.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p]
    assert calib.idx_calib_copy(P, P, 15, None) != 0
    assert calib.idx_calib_copy(None, P, 16, None) != 0


@pytest.mark.skipif(bool(HOST_LIB), reason="the debug library is a separate build of the whole library")
def test_debug_library_exports_and_flags(lib):
    # libidx_debug.so: the same sources built with -DIDX_DEBUG, the same exports
    dbg = ctypes.CDLL(_abi.DEBUG_LIB_PATH)
    _abi._declare(dbg)
    for name in _declared():
        assert hasattr(dbg, name), name
    assert dbg.idx_debug_build() == 1 and lib.idx_debug_build() == 0
    assert dbg.idx_abi_version() == lib.idx_abi_version()
    flags = ctypes.c_uint32(7)
    # the release build records nothing and asks nothing of the device
    assert lib.idx_debug_flags(ctypes.byref(flags), 1) == OK and flags.value == 0
    assert lib.idx_debug_flags(None, 1) == NULL and dbg.idx_debug_flags(None, 0) == NULL
    if not _gpu_visible():
        # the debug build waits for the device first: without one that fails
        assert dbg.idx_debug_flags(ctypes.byref(flags), 0) == LAUNCH
    assert (_abi.DBG_LENGTH, _abi.DBG_PAGE, _abi.DBG_SLOT, _abi.DBG_POSITION, _abi.DBG_SEQ) == tuple(
        int(re.search(rf"#define {n}\s+(\d+)u", open(HEADER).read()).group(1))
        for n in ("IDX_DBG_LENGTH", "IDX_DBG_PAGE", "IDX_DBG_SLOT", "IDX_DBG_POSITION", "IDX_DBG_SEQ"))


def test_version_and_status_text(lib):
    assert lib.idx_abi_version() == 1
    for s in range(8):
        assert lib.idx_status_str(s).decode().startswith(_abi.STATUS_NAMES[s])
    assert lib.idx_status_str(99) == b"unknown idx_status"


def test_page_bytes(lib):
    assert lib.idx_page_bytes(0, 64, 128) == 64 * 132
    assert lib.idx_page_bytes(1, 64, 128) == 64 * 68
    assert lib.idx_page_bytes(7, 64, 128) == 0


def _mqa(lib, **kw):
    a = dict(q=P, qs=64 * 128, k=P, ks=128, ksc=P, w=P, ws=64, rs=P, re=P, M=8, N=100, H=64, D=128, out=P, os=100)
    a.update(kw)
    return lib.idx_mqa_logits(a["q"], a["qs"], a["k"], a["ks"], a["ksc"], a["w"], a["ws"], a["rs"], a["re"], a["M"],
                              a["N"], a["H"], a["D"], a["out"], a["os"], None)


def test_mqa_logits_checks(lib):
    assert _mqa(lib, D=64) == SHAPE
    assert _mqa(lib, H=0) == SHAPE
    assert _mqa(lib, H=129) == SHAPE
    assert _mqa(lib, M=-1) == SHAPE
    assert _mqa(lib, M=0) == OK  # empty: nothing launched
    assert _mqa(lib, N=0, q=None) == OK
    assert _mqa(lib, q=None) == NULL
    assert _mqa(lib, ksc=None) == NULL
    assert _mqa(lib, out=None) == NULL
    assert _mqa(lib, qs=64 * 128 - 16) == STRIDE
    assert _mqa(lib, q=P + 8) == STRIDE
    assert _mqa(lib, ks=100) == STRIDE
    assert _mqa(lib, os=99) == STRIDE
    assert _mqa(lib, os=102) == STRIDE
    assert _mqa(lib, out=P + 4) == STRIDE
    assert _mqa(lib, ws=10) == STRIDE


def _cache(fmt=0, ps=64, npg=10, hd=128, stride=None, base=P):
    pb = ps * (hd + 4) if fmt == 0 else ps * (hd // 2 + hd // 32)
    return _abi.PagedCache(fmt=fmt, page_size=ps, num_pages=npg, head_dim=hd,
                           page_stride_bytes=pb if stride is None else stride, base=base)


def _paged(lib, cache=None, **kw):
    a = dict(q=P, qsc=None, w=P, ctx=P, per_row=0, bt=P, bts=8, mb=8, B=4, nn=1, H=64, out=P, os=512, width=512,
             ends=None, ws=None, wsb=0)
    a.update(kw)
    c = _cache() if cache is None else cache
    return lib.idx_paged_mqa_logits(ctypes.byref(c), a["q"], a["qsc"], a["w"], a["ctx"], a["per_row"], a["bt"],
                                    a["bts"], a["mb"], a["B"], a["nn"], a["H"], a["out"], a["os"], a["width"],
                                    a["ends"], a["ws"], a["wsb"], None)


def test_paged_checks(lib):
    assert lib.idx_paged_mqa_logits(None, P, None, P, P, 0, P, 8, 8, 4, 1, 64, P, 512, 512, None, None, 0,
                                    None) == NULL
    assert _paged(lib, cache=_cache(fmt=3)) == FORMAT
    assert _paged(lib, cache=_cache(hd=64)) == SHAPE
    assert _paged(lib, cache=_cache(ps=40)) == SHAPE
    assert _paged(lib, cache=_cache(ps=2048)) == SHAPE
    assert _paged(lib, cache=_cache(npg=0)) == SHAPE
    assert _paged(lib, cache=_cache(stride=64 * 132 - 16)) == STRIDE
    assert _paged(lib, cache=_cache(stride=64 * 132 + 4)) == STRIDE
    assert _paged(lib, cache=_cache(base=None)) == NULL
    assert _paged(lib, cache=_cache(base=P + 4)) == STRIDE
    assert _paged(lib, nn=0) == SHAPE
    assert _paged(lib, nn=5) == SHAPE
    assert _paged(lib, B=8193) == SHAPE
    assert _paged(lib, H=200) == SHAPE
    assert _paged(lib, width=-1) == SHAPE
    assert _paged(lib, B=8192, width=2 ** 31 - 1) == SHAPE  # chunk offsets would overflow int32
    assert _paged(lib, B=0, q=None) == OK
    assert _paged(lib, q=None) == NULL
    assert _paged(lib, ctx=None) == NULL
    assert _paged(lib, bt=None) == NULL
    assert _paged(lib, out=None) == NULL
    assert _paged(lib, qsc=P) == FORMAT  # fp8 carries no query scale
    assert _paged(lib, cache=_cache(fmt=1)) == NULL  # MXFP4 needs one
    assert _paged(lib, bts=7) == STRIDE
    assert _paged(lib, os=510) == STRIDE
    assert _paged(lib, out=P + 8) == STRIDE
    assert _paged(lib, q=P + 1) == STRIDE


def test_workspace_queries(lib):
    c = _cache()
    assert lib.idx_paged_mqa_logits_workspace(4, 1, 64, ctypes.byref(c)) == 0
    # top-k: 4096 workgroup records of 16 bytes and one 28736-byte record per row, for
    # 1..256 rows (several workgroups per row); none beyond
    assert lib.idx_topk_workspace(4, 1000, 16) == 2048 * 16 + 4 * 36928
    assert lib.idx_topk_workspace(256, 1000, 16) == 2048 * 16 + 256 * 36928
    assert lib.idx_topk_workspace(257, 1000, 16) == 0
    assert lib.idx_topk_workspace(0, 1000, 16) == 0


WS4 = 2048 * 16 + 4 * 36928  # idx_topk_workspace for 4 rows


def _topk(lib, **kw):
    a = dict(L=P, ls=1000, rows=4, width=1000, rs=None, re=P, k=16, out=P, os=16, ws=P, wsb=WS4)
    a.update(kw)
    return lib.idx_topk(a["L"], a["ls"], a["rows"], a["width"], a["rs"], a["re"], a["k"], a["out"], a["os"], a["ws"],
                        a["wsb"], None)


def test_topk_checks(lib):
    assert _topk(lib, k=0) == SHAPE
    assert _topk(lib, k=65537) == SHAPE
    assert _topk(lib, rows=-1) == SHAPE
    assert _topk(lib, rows=0, L=None, re=None, out=None) == OK
    assert _topk(lib, re=None) == NULL
    assert _topk(lib, out=None) == NULL
    assert _topk(lib, L=None) == NULL
    assert _topk(lib, ls=999) == STRIDE
    assert _topk(lib, os=15) == STRIDE
    assert _topk(lib, out=P + 2) == STRIDE
    assert _topk(lib, wsb=WS4 - 1) == WORKSPACE
    assert _topk(lib, ws=None) == NULL
    assert _topk(lib, rows=300, ws=None, wsb=0) != WORKSPACE  # many rows: no workspace needed


def test_k_store_and_q_quant_checks(lib):
    c = _cache()
    assert lib.idx_k_store(ctypes.byref(c), P, 2, 128, P, 10, None) == FORMAT
    assert lib.idx_k_store(ctypes.byref(c), P, 0, 128, P, -1, None) == SHAPE
    assert lib.idx_k_store(ctypes.byref(c), None, 0, 128, None, 0, None) == OK
    assert lib.idx_k_store(ctypes.byref(c), None, 0, 128, P, 10, None) == NULL
    assert lib.idx_k_store(ctypes.byref(c), P, 0, 127, P, 10, None) == STRIDE
    assert lib.idx_k_store(ctypes.byref(c), P + 2, 0, 128, P, 10, None) == STRIDE
    assert lib.idx_k_store(ctypes.byref(c), P, 0, 128, P + 4, 10, None) == STRIDE
    assert lib.idx_q_quant(P, 0, 128, 4, 1, 128, 5, P, None, None) == FORMAT
    assert lib.idx_q_quant(P, 3, 128, 4, 1, 128, 0, P, None, None) == FORMAT
    assert lib.idx_q_quant(P, 0, 128, 4, 1, 64, 0, P, None, None) == SHAPE
    assert lib.idx_q_quant(None, 0, 128, 0, 1, 128, 0, None, None, None) == OK
    assert lib.idx_q_quant(P, 0, 128, 4, 1, 128, 1, P, None, None) == NULL
    assert lib.idx_q_quant(P, 0, 128, 4, 1, 128, 0, P, P, None) == FORMAT
    assert lib.idx_q_quant(P, 0, 100, 4, 1, 128, 0, P, None, None) == STRIDE


def test_fused_producer_checks(lib):
    c = _cache()
    kn = lib.idx_k_norm_rope_store
    # (cache, k, dtype, stride, positions, cos_sin, max_position, rope_dim, weight, eps, slots, N, stream)
    assert kn(ctypes.byref(c), P, 0, 128, P, P, 16, 3, P, 1e-6, P, 10, None) == SHAPE  # odd rope_dim
    assert kn(ctypes.byref(c), P, 0, 128, P, P, 16, 130, P, 1e-6, P, 10, None) == SHAPE  # rope_dim > D
    assert kn(ctypes.byref(c), P, 0, 128, None, P, 16, 64, P, 1e-6, P, 10, None) == NULL
    assert kn(ctypes.byref(c), P, 0, 128, P, None, 16, 64, P, 1e-6, P, 10, None) == NULL
    assert kn(ctypes.byref(c), P, 0, 128, P, P, 0, 64, P, 1e-6, P, 10, None) == SHAPE  # empty table
    assert kn(ctypes.byref(c), P, 0, 128, P, P, 16, 64, P, 0.0, P, 10, None) == SHAPE  # eps must be > 0
    assert kn(ctypes.byref(c), P, 0, 128, P, P, 16, 64, P + 4, 1e-6, P, 10, None) == STRIDE  # weight alignment
    assert kn(ctypes.byref(c), P, 0, 128, P + 4, P, 16, 64, P, 1e-6, P, 10, None) == STRIDE  # positions alignment
    assert kn(ctypes.byref(c), None, 0, 128, None, None, 0, 0, None, 1e-6, None, 0, None) == OK  # N = 0
    qr = lib.idx_q_rope_quant
    # (q, dtype, stride, positions, cos_sin, max_position, rope_dim, weights, w_stride, scale, T, H, D, fmt,
    #  q_out, q_scale_out, weights_out, stream)
    assert qr(P, 0, 128, P, P, 16, 5, P, 1, 1.0, 4, 1, 128, 0, P, None, P, None) == SHAPE
    assert qr(P, 0, 128, P, P, 16, 64, None, 1, 1.0, 4, 1, 128, 0, P, None, P, None) == NULL
    assert qr(P, 0, 128, P, P, 16, 64, P, 1, 1.0, 4, 1, 128, 0, P, None, None, None) == NULL
    assert qr(P, 0, 128, P, P, 16, 64, P, 0, 1.0, 4, 1, 128, 0, P, None, P, None) == STRIDE  # weights stride < H
    assert qr(P, 0, 128, P, P, 16, 64, P, 1, 1.0, 4, 1, 128, 0, P + 4, None, P, None) == STRIDE  # fp8 q_out
    assert qr(P, 0, 128, P, P, 16, 64, P, 1, 1.0, 4, 1, 128, 1, P, None, P, None) == NULL  # MXFP4 needs scales
    assert qr(None, 0, 128, None, None, 0, 0, None, 1, 1.0, 0, 1, 128, 0, None, None, None, None) == OK  # T = 0


def test_topk_to_slots_checks(lib):
    f = lib.idx_topk_to_slots
    # (topk, stride, rows, k, row_seq, next_n, B, row_valid, bt, bt_stride, max_blocks, P, slots, indptr, lens, s)
    assert f(P, 8, 4, 8, None, 1, 0, None, P, 4, 4, 16, P, P, None, None) == SHAPE  # B < 1
    assert f(P, 8, 4, 8, None, 0, 2, None, P, 4, 4, 16, P, P, None, None) == SHAPE  # next_n < 1 without row_seq
    assert f(P, 8, 4, 8, None, 1, 2, None, P, 4, 4, 16, P, None, None, None) == NULL  # indptr
    assert f(P, 8, 4, 8, None, 1, 2, None, None, 4, 4, 16, P, P, None, None) == NULL  # block table
    assert f(P, 4, 4, 8, None, 1, 2, None, P, 4, 4, 16, P, P, None, None) == STRIDE  # topk stride < k
    assert f(P, 8, 4, 8, None, 1, 2, None, P, 3, 4, 16, P, P, None, None) == STRIDE  # bt stride < max_blocks
    assert f(P + 2, 8, 4, 8, None, 1, 2, None, P, 4, 4, 16, P, P, None, None) == STRIDE
    assert f(P, 8, -1, 8, None, 1, 2, None, P, 4, 4, 16, P, P, None, None) == SHAPE


def test_two_level_checks(lib):
    c = _cache()
    bm = lib.idx_paged_mqa_logits_block_max

    def _bm(**kw):
        a = dict(bmp=P, bms=32, bs=16, B=4)
        a.update(kw)
        return bm(ctypes.byref(c), P, None, P, P, 0, P, 8, 8, a["B"], 1, 64, P, 512, 512, None, a["bmp"], a["bms"],
                  a["bs"], None, 0, None)
    assert _bm(bs=8) == SHAPE  # block maxima need 16, 32 or 64
    assert _bm(bs=128) == SHAPE
    assert _bm(bmp=None) == NULL
    assert _bm(bms=31) == STRIDE  # 512 / 16 blocks per row
    assert _bm(bmp=P + 2) == STRIDE
    assert _bm(B=0) == OK
    assert _bm(bs=0, bmp=None, B=0) == OK  # no block maxima asked for

    g = lib.idx_paged_mqa_logits_gather

    def _g(**kw):
        a = dict(cand=P, cs=8, n=8, bs=64, rr=1, out=P, os=512, B=4, nn=1)
        a.update(kw)
        return g(ctypes.byref(c), P, None, P, P, 0, P, 8, 8, a["B"], a["nn"], 64, a["cand"], a["cs"], a["n"],
                 a["bs"], a["rr"], a["out"], a["os"], a.get("ends", P), None)
    assert _g(bs=8) == SHAPE  # a 16-key group must sit inside one pool block
    assert _g(bs=48) == SHAPE  # not a power of two
    assert _g(n=0) == SHAPE
    assert _g(rr=0) == SHAPE
    assert _g(B=4096, nn=4) == SHAPE  # rows kept in LDS
    assert _g(cand=None) == NULL
    assert _g(cs=7) == STRIDE
    assert _g(os=510) == STRIDE  # the pool row is n * block = 512 wide
    assert _g(out=None) == NULL
    assert _g(ends=None) == NULL  # the pool lengths pass through it
    assert _g(ends=P + 2) == STRIDE
    assert _g(B=0) == OK

    cb = lib.idx_candidate_blocks
    assert cb(P, 32, 4, 32, P, 48, 8, P, 8, None, 0, None) == SHAPE  # block size a power of two
    assert cb(P, 31, 4, 32, P, 16, 8, P, 8, None, 0, None) == STRIDE
    assert cb(P, 32, 4, 32, None, 16, 8, P, 8, None, 0, None) == NULL
    assert cb(P, 32, 0, 32, None, 16, 8, None, 8, None, 0, None) == OK

    m = lib.idx_apply_candidate_mask
    assert m(P, 512, 4, 512, P, P, 8, 8, 24, 1, None) == SHAPE
    assert m(P, 512, 4, 2 ** 20, P, P, 8, 8, 1, 1, None) == SHAPE  # one LDS byte per block
    assert m(P, 510, 4, 510, P, P, 8, 8, 16, 1, None) == STRIDE
    assert m(P + 4, 512, 4, 512, P, P, 8, 8, 16, 1, None) == STRIDE
    assert m(P, 512, 4, 512, P, None, 8, 8, 16, 1, None) == NULL
    assert m(P, 512, 4, 512, P, P, 7, 8, 16, 1, None) == STRIDE
    assert m(P, 512, 4, 512, P, P, 8, 8, 16, 0, None) == SHAPE

    r = lib.idx_remap_compact_topk
    assert r(P, 8, 4, 16, P, 8, 8, 16, 1, None) == STRIDE
    assert r(None, 16, 4, 16, P, 8, 8, 16, 1, None) == NULL
    assert r(P, 16, 4, 16, P, 8, 8, 12, 1, None) == SHAPE
    assert r(P, 16, 0, 16, P, 8, 8, 16, 1, None) == OK


def test_paged_prefill_checks(lib):
    f = lib.idx_paged_prefill_logits

    def _pf(cache=None, **kw):
        a = dict(q=P, qsc=None, w=P, ends=P, bt=P, mb=8, M=64, H=64, out=P, os=512, width=512)
        a.update(kw)
        c = _cache() if cache is None else cache
        return f(ctypes.byref(c), a["q"], a["qsc"], a["w"], a["ends"], a["bt"], a["mb"], a["M"], a["H"], a["out"],
                 a["os"], a["width"], None)
    assert _pf(M=-1) == SHAPE
    assert _pf(M=0, q=None) == OK
    assert _pf(q=None) == NULL
    assert _pf(ends=None) == NULL
    assert _pf(bt=None) == NULL
    assert _pf(out=None) == NULL
    assert _pf(cache=_cache(fmt=1)) == NULL  # MXFP4 needs query scales
    assert _pf(qsc=P) == FORMAT
    assert _pf(os=510) == STRIDE
    assert _pf(q=P + 4) == STRIDE
    assert _pf(H=0) == SHAPE
    assert _pf(M=2 ** 20, width=2 ** 20) == SHAPE  # past the row limit
    assert _pf(M=16385) == SHAPE  # 16384 rows at most
    assert _pf(H=129) == SHAPE
    assert _pf(width=0, out=None) == OK  # nothing to write, nothing launched


@pytest.mark.skipif(_gpu_visible(), reason="checks the no-device path; a GPU is visible")
def test_paged_prefill_empty_table_passes_host_checks(lib):
    # an fp8 chunk with no block-table entries (NULL table, max_blocks 0) but rows that
    # end past 0 is a valid call: every column is -inf. It must pass the host checks and
    # reach the device query (the GPU test runs it); the kernel chosen for fp8 pages
    # is then the paged one, which reads neither the table nor a page when no key exists
    f = lib.idx_paged_prefill_logits
    c = _cache()
    assert f(ctypes.byref(c), P, None, P, P, None, 0, 64, 64, P, 512, 512, None) == DEVICE
    assert f(ctypes.byref(_cache(fmt=1)), P, P, P, P, None, 0, 64, 64, P, 512, 512, None) == DEVICE


@pytest.mark.skipif(_gpu_visible(), reason="checks the no-device path; a GPU is visible")
def test_valid_call_without_device_reports_device_error(lib):
    # arguments pass every host check, so the call reaches the device query, which
    # fails here because this machine has no GPU; nothing is launched
    assert _topk(lib) == DEVICE


# ---- host build only: a pretend gfx950 behind the ABI layer ---------------------------

host_only = pytest.mark.skipif(not HOST_LIB, reason="needs the host build of the ABI layer (tests/host_asan)")


@pytest.fixture
def device(lib):
    lib.idx_host_set_device(1)
    yield lib
    lib.idx_host_set_device(0)


def _launches(lib, call, what=""):
    """(status, launches) of one call, with no launcher check failing."""
    n0, v0 = lib.idx_host_launches(), lib.idx_host_violations()
    s = call()
    assert lib.idx_host_violations() == v0, f"{what}: a launcher was reached with arguments its kernels cannot use"
    return s, lib.idx_host_launches() - n0


@host_only
def test_host_valid_calls_reach_their_launchers(device):
    lib = device
    c8, c4 = _cache(), _cache(fmt=1)
    kn, qr = lib.idx_k_norm_rope_store, lib.idx_q_rope_quant
    calls = {
        "mqa": lambda: _mqa(lib),
        "paged fp8": lambda: _paged(lib),
        "paged mxfp4": lambda: _paged(lib, cache=c4, qsc=P),
        "paged per-row lengths": lambda: _paged(lib, per_row=1, nn=2),
        "topk": lambda: _topk(lib),
        "topk many rows": lambda: _topk(lib, rows=300, ws=None, wsb=0),
        "topk noalloc": lambda: lib.idx_topk_noalloc(P, 1000, 4, 1000, None, P, 16, P, 16, None),
        "k store": lambda: lib.idx_k_store(ctypes.byref(c8), P, 0, 128, P, 10, None),
        "q quant fp8": lambda: lib.idx_q_quant(P, 0, 128, 4, 1, 128, 0, P, None, None),
        "q quant mxfp4": lambda: lib.idx_q_quant(P, 0, 128, 4, 1, 128, 1, P, P, None),
        "k norm rope store": lambda: kn(ctypes.byref(c8), P, 0, 128, P, P, 16, 64, P, 1e-6, P, 10, None),
        "q rope quant": lambda: qr(P, 0, 128, P, P, 16, 64, P, 1, 1.0, 4, 1, 128, 0, P, None, P, None),
        "slots": lambda: lib.idx_topk_to_slots(P, 8, 4, 8, None, 1, 2, None, P, 4, 4, 16, P, P, None, None),
        "block max": lambda: lib.idx_paged_mqa_logits_block_max(ctypes.byref(c8), P, None, P, P, 0, P, 8, 8, 4, 1,
                                                                64, P, 512, 512, None, P, 32, 16, None, 0, None),
        "gather": lambda: lib.idx_paged_mqa_logits_gather(ctypes.byref(c8), P, None, P, P, 0, P, 8, 8, 4, 1, 64, P,
                                                          8, 8, 64, 1, P, 512, P, None),
        "candidate blocks": lambda: lib.idx_candidate_blocks(P, 32, 4, 32, P, 16, 8, P, 8, P, WS4, None),
        "candidate mask": lambda: lib.idx_apply_candidate_mask(P, 512, 4, 512, P, P, 8, 8, 16, 1, None),
        "remap": lambda: lib.idx_remap_compact_topk(P, 16, 4, 16, P, 8, 8, 16, 1, None),
    }
    pf = lib.idx_paged_prefill_logits
    calls.update({
        "prefill fp8 pages": lambda: pf(ctypes.byref(c8), P, None, P, P, P, 8, 64, 64, P, 512, 512, None),
        "prefill mxfp4 pages": lambda: pf(ctypes.byref(c4), P, P, P, P, P, 8, 64, 64, P, 512, 512, None),
        "prefill mxfp4 pages, 128 heads": lambda: pf(ctypes.byref(c4), P, P, P, P, P, 8, 64, 128, P, 512, 512,
                                                     None),
        # no block-table entries: the fp8 chunk must take the paged kernel with no key
        # to read (a NULL table is valid then), never the contiguous one
        "prefill fp8, empty table": lambda: pf(ctypes.byref(c8), P, None, P, P, None, 0, 64, 64, P, 512, 512, None),
        "prefill mxfp4, empty table": lambda: pf(ctypes.byref(c4), P, P, P, P, None, 0, 64, 64, P, 512, 512, None),
    })
    for name, call in calls.items():
        s, n = _launches(lib, call, name)
        assert s == OK, (name, s)
        assert n >= 1, f"{name}: nothing launched"


@host_only
@pytest.mark.parametrize("check,launches", [
    (test_mqa_logits_checks, 0), (test_paged_checks, 0), (test_topk_checks, 1),
    (test_k_store_and_q_quant_checks, 0), (test_fused_producer_checks, 0), (test_topk_to_slots_checks, 0),
    (test_two_level_checks, 0), (test_paged_prefill_checks, 0)])
def test_host_rejected_calls_launch_nothing(device, check, launches):
    # the argument checks above, now with a device present: every rejected or empty call
    # returns before any launcher (test_topk_checks holds one valid call, 300 rows)
    s, n = _launches(device, lambda: check(device), check.__name__)
    assert n == launches, check.__name__
