"""ctypes view of libidx.so (include/idx.h). Loading fails loudly if the library is
missing: there is no fallback implementation."""

from __future__ import annotations

import contextlib
import ctypes
import os

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libidx.so")
DEBUG_LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libidx_debug.so")

IDX_OK = 0
IDX_KV_FP8_E4M3 = 0
IDX_KV_MXFP4_E2M1 = 1
IDX_IN_F32 = 0
IDX_IN_BF16 = 1
ABI_VERSION = 1

STATUS_NAMES = {
    0: "IDX_OK", 1: "IDX_ERR_NULL", 2: "IDX_ERR_SHAPE", 3: "IDX_ERR_STRIDE", 4: "IDX_ERR_FORMAT",
    5: "IDX_ERR_WORKSPACE", 6: "IDX_ERR_LAUNCH", 7: "IDX_ERR_DEVICE",
}

# every function include/idx.h declares
EXPORTS = (
    "idx_page_bytes", "idx_mqa_logits", "idx_paged_mqa_logits", "idx_paged_mqa_logits_workspace", "idx_topk",
    "idx_topk_workspace", "idx_k_store", "idx_q_quant", "idx_k_norm_rope_store", "idx_q_rope_quant",
    "idx_topk_to_slots", "idx_paged_mqa_logits_block_max", "idx_candidate_blocks", "idx_apply_candidate_mask",
    "idx_paged_mqa_logits_gather", "idx_remap_compact_topk", "idx_paged_prefill_logits", "idx_topk_noalloc",
    "idx_debug_flags", "idx_debug_build", "idx_status_str", "idx_abi_version",
)

# idx_debug_flags bits: device-resident values the kernels had to clamp or drop
DBG_LENGTH, DBG_PAGE, DBG_SLOT, DBG_POSITION, DBG_SEQ = 1, 2, 4, 8, 16


class PagedCache(ctypes.Structure):
    """idx_paged_cache."""

    _fields_ = [
        ("fmt", ctypes.c_int32),
        ("page_size", ctypes.c_int32),
        ("num_pages", ctypes.c_int32),
        ("head_dim", ctypes.c_int32),
        ("page_stride_bytes", ctypes.c_int64),
        ("base", ctypes.c_void_p),
    ]


class IdxError(RuntimeError):
    def __init__(self, status: int, text: str):
        super().__init__(text)
        self.status = status


_lib = None

_P = ctypes.c_void_p
_I32 = ctypes.c_int32
_I64 = ctypes.c_int64
_SZ = ctypes.c_size_t
_F32 = ctypes.c_float


def _declare(lib: ctypes.CDLL) -> None:
    cache_p = ctypes.POINTER(PagedCache)
    sig = {
        "idx_page_bytes": (_SZ, [_I32, _I32, _I32]),
        "idx_mqa_logits": (_I32, [_P, _I64, _P, _I64, _P, _P, _I64, _P, _P, _I32, _I32, _I32, _I32, _P, _I64, _P]),
        "idx_paged_mqa_logits": (_I32, [cache_p, _P, _P, _P, _P, _I32, _P, _I64, _I32, _I32, _I32, _I32, _P, _I64,
                                        _I32, _P, _P, _SZ, _P]),
        "idx_paged_mqa_logits_workspace": (_SZ, [_I32, _I32, _I32, cache_p]),
        "idx_topk": (_I32, [_P, _I64, _I32, _I32, _P, _P, _I32, _P, _I64, _P, _SZ, _P]),
        "idx_topk_workspace": (_SZ, [_I32, _I32, _I32]),
        "idx_topk_noalloc": (_I32, [_P, _I64, _I32, _I32, _P, _P, _I32, _P, _I64, _P]),
        "idx_k_store": (_I32, [cache_p, _P, _I32, _I64, _P, _I32, _P]),
        "idx_q_quant": (_I32, [_P, _I32, _I64, _I32, _I32, _I32, _I32, _P, _P, _P]),
        "idx_k_norm_rope_store": (_I32, [cache_p, _P, _I32, _I64, _P, _P, _I32, _I32, _P, _F32, _P, _I32, _P]),
        "idx_q_rope_quant": (_I32, [_P, _I32, _I64, _P, _P, _I32, _I32, _P, _I64, _F32, _I32, _I32, _I32, _I32, _P,
                                    _P, _P, _P]),
        "idx_topk_to_slots": (_I32, [_P, _I64, _I32, _I32, _P, _I32, _I32, _P, _P, _I64, _I32, _I32, _P, _P, _P, _P]),
        "idx_paged_mqa_logits_block_max": (_I32, [cache_p, _P, _P, _P, _P, _I32, _P, _I64, _I32, _I32, _I32, _I32,
                                                  _P, _I64, _I32, _P, _P, _I64, _I32, _P, _SZ, _P]),
        "idx_candidate_blocks": (_I32, [_P, _I64, _I32, _I32, _P, _I32, _I32, _P, _I64, _P, _SZ, _P]),
        "idx_apply_candidate_mask": (_I32, [_P, _I64, _I32, _I32, _P, _P, _I64, _I32, _I32, _I32, _P]),
        "idx_paged_mqa_logits_gather": (_I32, [cache_p, _P, _P, _P, _P, _I32, _P, _I64, _I32, _I32, _I32, _I32, _P,
                                               _I64, _I32, _I32, _I32, _P, _I64, _P, _P]),
        "idx_remap_compact_topk": (_I32, [_P, _I64, _I32, _I32, _P, _I64, _I32, _I32, _I32, _P]),
        "idx_paged_prefill_logits": (_I32, [cache_p, _P, _P, _P, _P, _P, _I32, _I32, _I32, _P, _I64, _I32, _P]),
        "idx_debug_flags": (_I32, [ctypes.POINTER(ctypes.c_uint32), _I32]),
        "idx_debug_build": (_I32, []),
        "idx_status_str": (ctypes.c_char_p, [_I32]),
        "idx_abi_version": (_I32, []),
    }
    for name, (res, args) in sig.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args


def _load(path: str) -> ctypes.CDLL:
    if not os.path.exists(path):
        raise ImportError(f"{path} is missing: build it with `python -m sparse_attention_indexer_mxfp4_amd.build`")
    handle = ctypes.CDLL(path)
    _declare(handle)
    if handle.idx_abi_version() != ABI_VERSION:
        raise ImportError(f"{os.path.basename(path)} ABI {handle.idx_abi_version()} != {ABI_VERSION}")
    return handle


def lib() -> ctypes.CDLL:
    """The loaded library (loaded once). Raises if libidx.so has not been built."""
    global _lib, _release
    if _lib is None:
        _release = _load(LIB_PATH)
        _lib = _release
    return _lib


_release = None
_debug = None


@contextlib.contextmanager
def debug_build():
    """Within the block, every call goes to libidx_debug.so (the -DIDX_DEBUG build),
    which yields the same results and records clamped device-resident values for
    idx_debug_flags. Not thread-safe: the switch is process-wide."""
    global _lib, _debug
    if _debug is None:
        _debug = _load(DEBUG_LIB_PATH)
        if _debug.idx_debug_build() != 1:
            raise ImportError(f"{DEBUG_LIB_PATH} is not a debug build")
    lib()
    _lib = _debug
    try:
        yield _debug
    finally:
        _lib = _release


def check(status: int) -> None:
    if status != IDX_OK:
        raise IdxError(status, lib().idx_status_str(status).decode())
