"""GPU parity of idx_topk: on the same fp32 logits the GPU and the oracle take every
decision in the same precision, so the indices must match exactly (index work),
ties and signed zeros included."""

import numpy as np
import pytest
import torch

from oracle import indexer
from sparse_attention_indexer_mxfp4_amd import ops

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def _run(logits, starts, ends, k):
    lt = torch.from_numpy(np.ascontiguousarray(logits, dtype=np.float32)).to(DEV)
    st = None if starts is None else torch.from_numpy(np.asarray(starts, np.int32)).to(DEV)
    en = torch.from_numpy(np.asarray(ends, np.int32)).to(DEV)
    out = ops.idx_topk(lt, st, en, k)
    torch.cuda.synchronize()
    return out.cpu().numpy()


@pytest.mark.parametrize("width,k", [(100, 16), (3000, 64), (5000, 2048), (20000, 512), (40000, 2048),
                                     (70000, 1000)])
def test_topk_random_rows(width, k):
    rng = np.random.default_rng(width + k)
    rows = 12
    L = rng.standard_normal((rows, width)).astype(np.float32)
    L[0] = np.round(L[0] * 2) / 2  # heavy ties
    L[1] = 0.0
    L[1, ::3] = -0.0  # signed zeros tie
    L[2] = 1.0  # all equal
    L[3, : width // 2] = -np.inf  # -inf inside the range ranks last
    starts = rng.integers(0, width // 4, rows)
    ends = rng.integers(width // 2, width + 1, rows)
    starts[4], ends[4] = 0, width
    starts[5], ends[5] = 10, 10  # empty
    ends[6] = starts[6] + k  # exactly k
    ends[7] = starts[7] + k - 1  # one short
    ends[8] = width + 50  # clamped to the width
    got = _run(L, starts, ends, k)
    want = indexer.topk(L.astype(np.float64), starts, ends, k)
    np.testing.assert_array_equal(got, want)


def test_topk_no_start_and_large_k():
    rng = np.random.default_rng(3)
    L = rng.standard_normal((5, 300)).astype(np.float32)
    ends = np.array([300, 0, 150, 299, 1])
    got = _run(L, None, ends, 400)
    np.testing.assert_array_equal(got, indexer.topk(L.astype(np.float64), None, ends, 400))


def test_topk_many_rows():
    rng = np.random.default_rng(4)
    rows, width, k = 600, 2048, 256
    L = rng.standard_normal((rows, width)).astype(np.float32)
    ends = rng.integers(0, width + 1, rows)
    got = _run(L, np.zeros(rows, np.int32), ends, k)
    np.testing.assert_array_equal(got, indexer.topk(L.astype(np.float64), None, ends, k))
