"""ctypes view of libidx.so (include/idx.h). Loading fails loudly if the library is
missing: there is no fallback implementation."""

from __future__ import annotations

import ctypes
import os

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libidx.so")

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
    "idx_status_str", "idx_abi_version",
)


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
        "idx_status_str": (ctypes.c_char_p, [_I32]),
        "idx_abi_version": (_I32, []),
    }
    for name, (res, args) in sig.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args


def lib() -> ctypes.CDLL:
    """The loaded library (loaded once). Raises if libidx.so has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(
                f"{LIB_PATH} is missing: build it with `python -m sparse_attention_indexer_mxfp4_amd.build`")
        handle = ctypes.CDLL(LIB_PATH)
        _declare(handle)
        if handle.idx_abi_version() != ABI_VERSION:
            raise ImportError(f"libidx ABI {handle.idx_abi_version()} != {ABI_VERSION}")
        _lib = handle
    return _lib


def check(status: int) -> None:
    if status != IDX_OK:
        raise IdxError(status, lib().idx_status_str(status).decode())
