"""idx_topk_noalloc (the top-k entry point that allocates nothing, for callers under
graph capture or in tight serving loops) against idx_topk with a caller workspace, both
through the C ABI, on the same logits: bit for bit (index work).

Two calls in a row on the path that keeps its records in the library's own array (rows
of more than 65536 columns), the second with fewer and shorter rows, so the second call
reads the array as the first left it; then one call on the one-workgroup-per-row path,
which uses no scratch.
"""

import ctypes

import numpy as np
import pytest
import torch

from oracle import indexer
from sparse_attention_indexer_mxfp4_amd import _abi, ops

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def _noalloc(logits, ends, k):
    rows, width = logits.shape
    out = torch.full((rows, k), -7, dtype=torch.int32, device=DEV)
    st = _abi.lib().idx_topk_noalloc(logits.data_ptr(), logits.stride(0), rows, width, None, ends.data_ptr(), k,
                                     out.data_ptr(), out.stride(0), torch.cuda.current_stream().cuda_stream)
    _abi.check(st)
    return out


def _with_workspace(logits, ends, k):
    rows, width = logits.shape
    lib = _abi.lib()
    need = lib.idx_topk_workspace(rows, width, k)
    ws = torch.zeros(max(need, 1), dtype=torch.uint8, device=DEV)  # a workspace of its own
    out = torch.empty((rows, k), dtype=torch.int32, device=DEV)
    _abi.check(lib.idx_topk(logits.data_ptr(), logits.stride(0), rows, width, None, ends.data_ptr(), k,
                            out.data_ptr(), out.stride(0), ctypes.c_void_p(ws.data_ptr()), need,
                            torch.cuda.current_stream().cuda_stream))
    return out


@pytest.mark.parametrize("rows,width,k,seed", [(64, 131072, 2048, 1), (8, 70000, 512, 2), (300, 4000, 256, 3)])
def test_noalloc_matches_topk(rows, width, k, seed):
    rng = np.random.default_rng(seed)
    L = rng.standard_normal((rows, width)).astype(np.float32)
    ends = rng.integers(1, width + 1, rows).astype(np.int32)
    ends[0] = width
    lt = torch.from_numpy(L).to(DEV)
    en = torch.from_numpy(ends).to(DEV)
    print(f"noalloc rows={rows} width={width} k={k}", flush=True)
    got = _noalloc(lt, en, k)
    want = _with_workspace(lt, en, k)
    torch.cuda.synchronize()
    got, want = got.cpu().numpy(), want.cpu().numpy()
    np.testing.assert_array_equal(got, want)
    sample = np.arange(0, rows, max(1, rows // 8))
    np.testing.assert_array_equal(got[sample], indexer.topk(L[sample].astype(np.float64), None, ends[sample], k))
