"""The indexer step under HIP graph capture: the calls neither allocate nor
synchronise, so a captured logits + top-k step must replay to exactly the eager
result, replay after replay, with unrelated eager work in between."""

import numpy as np
import pytest
import torch

from sparse_attention_indexer_mxfp4_amd import ops, workloads
from tests import _inputs

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


@pytest.mark.parametrize("fmt", ["fp8", "mxfp4"])
def test_graph_replay_matches_eager(fmt):
    wl = workloads.paged(seed=21, B=6, next_n=2, H=64, ctx_lo=50, ctx_hi=3000, width=3072, topk=256, fmt=fmt)
    pi = _inputs.paged_inputs(wl)
    f = ops.FP8 if fmt == "fp8" else ops.MXFP4
    pool = torch.from_numpy(pi.pool).to(DEV)
    q = torch.from_numpy(pi.q).to(DEV)
    qs = None if pi.q_scale is None else torch.from_numpy(pi.q_scale).to(DEV)
    w = torch.from_numpy(wl.w).to(DEV)
    ctx = torch.from_numpy(wl.context_lens).to(DEV)
    bt = torch.from_numpy(wl.block_table).to(DEV)
    logits = torch.empty((wl.rows, wl.width), dtype=torch.float32, device=DEV)
    ends = torch.empty(wl.rows, dtype=torch.int32, device=DEV)
    out = torch.empty((wl.rows, wl.topk), dtype=torch.int32, device=DEV)

    def step():
        ops.idx_paged_mqa_logits(pool, f, wl.page_size, q, qs, w, ctx, bt, wl.width, logits=logits, row_end_out=ends)
        ops.idx_topk(logits, None, ends, wl.topk, out=out)

    step()
    torch.cuda.synchronize()
    ref_logits, ref_ends, ref_out = logits.clone(), ends.clone(), out.clone()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step()
    scratch = torch.randn(1 << 20, device=DEV)
    for rep in range(4):
        logits.fill_(7.0)
        ends.fill_(-5)
        out.fill_(-9)
        scratch.mul_(1.0001)  # unrelated eager work between replays
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(logits, ref_logits), f"replay {rep}: logits differ"
        assert torch.equal(ends, ref_ends), f"replay {rep}: row ends differ"
        assert torch.equal(out, ref_out), f"replay {rep}: top-k differs"
