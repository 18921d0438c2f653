"""The debug build (libidx_debug.so, the kernels compiled with -DIDX_DEBUG) against the
release build on the same inputs.

The kernels trust device-resident values (lengths, row bounds, block-table entries,
slots, rotary positions, sequence ids) and clamp or drop any that fall outside their
range; the debug build also records each kind in a bit that idx_debug_flags reads back.
Here every entry point runs under both builds: on valid inputs (block-table entries
past each sequence's pages set to -1, which no kernel may read) the debug build
records nothing, and each kind of out-of-range value, all of which the release kernels
clamp or skip by construction, sets exactly its own bit. In every case the two builds'
outputs agree bit for bit."""

import numpy as np
import pytest
import torch

from sparse_attention_indexer_mxfp4_amd import _abi, ops, workloads
from tests import _inputs

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def _dev(x):
    return torch.from_numpy(np.ascontiguousarray(x)).to(DEV)


def _bits(outs):
    """Every output tensor as host bytes (NaN-safe, -0.0 distinct)."""
    if isinstance(outs, torch.Tensor):
        outs = (outs,)
    return [o.contiguous().view(torch.uint8).cpu().numpy().copy() for o in outs if o is not None]


def both(call, what):
    """(flags the debug build recorded, outputs) after running call() under each build;
    asserts the outputs agree byte for byte. call() must build its own outputs (and
    copies of anything it updates in place)."""
    assert ops.idx_debug_flags() == 0  # the release build records nothing
    want = call()
    torch.cuda.synchronize()
    want = _bits(want)
    with ops.debug_build():
        ops.idx_debug_flags(clear=True)
        got = call()
        flags = ops.idx_debug_flags(clear=True)
        got = _bits(got)
    assert len(got) == len(want)
    for i, (g, w) in enumerate(zip(got, want)):
        assert np.array_equal(g, w), f"{what}: output {i} differs between the debug and release builds"
    return flags


def _padded_copy(logits):
    """A copy with a row stride that is a multiple of 4 (what the in-place mask needs)."""
    rows, width = logits.shape
    out = torch.empty((rows, -(-width // 4) * 4), dtype=logits.dtype, device=logits.device)[:, :width]
    out.copy_(logits)
    return out


def _unused_entries_to_minus_one(wl):
    bt = wl.block_table.copy()
    used = -(-wl.context_lens.astype(np.int64) // wl.page_size)
    for b in range(bt.shape[0]):
        bt[b, used[b]:] = -1
    return bt


def _paged(fmt, next_n=2):
    lens = np.array([0, 1, 63, 65, 300, 1000, 7])
    wl = workloads.paged(seed=60 + next_n, B=len(lens), next_n=next_n, H=64, ctx_lo=0, ctx_hi=0, width=1101,
                         topk=33, fmt=fmt, context_lens=lens)
    pi = _inputs.paged_inputs(wl)
    return wl, pi


def _args(wl, pi, fmt, ctx=None, bt=None):
    f = ops.FP8 if fmt == "fp8" else ops.MXFP4
    ctx = wl.context_lens if ctx is None else ctx
    bt = _unused_entries_to_minus_one(wl) if bt is None else bt
    return (_dev(pi.pool), f, wl.page_size, _dev(pi.q), None if pi.q_scale is None else _dev(pi.q_scale),
            _dev(wl.w), _dev(ctx.astype(np.int32)), _dev(bt))


def test_release_library_reports_release():
    assert _abi.lib().idx_debug_build() == 0
    with ops.debug_build() as dbg:
        assert dbg.idx_debug_build() == 1
        assert _abi.lib() is dbg
    assert _abi.lib().idx_debug_build() == 0


@pytest.mark.parametrize("fmt", ["fp8", "mxfp4"])
def test_valid_inputs_record_nothing(fmt):
    wl, pi = _paged(fmt)
    args = _args(wl, pi, fmt)
    block, n_cand, k = 32, 7, 40

    def decode():
        logits, ends = ops.idx_paged_mqa_logits(*args, wl.width)
        idx = ops.idx_topk(logits, None, ends, k)
        slots, indptr, lens = ops.idx_topk_to_slots(idx, args[-1], wl.page_size, next_n=wl.next_n)
        return logits, ends, idx, slots, indptr, lens

    def per_row():
        ctx = np.repeat(wl.context_lens, wl.next_n) - np.tile(np.arange(wl.next_n)[::-1], wl.B)
        a = _args(wl, pi, fmt, ctx=np.maximum(ctx, 0))
        return ops.idx_paged_mqa_logits(*a, wl.width, ctx_per_row=True)

    def two_level():
        logits, ends, bm = ops.idx_paged_mqa_logits_block_max(*args, wl.width, block)
        cand = ops.idx_candidate_blocks(bm, ends, block, n_cand)
        masked = ops.idx_apply_candidate_mask(_padded_copy(logits), ends, cand, block)
        pool, pend = ops.idx_paged_mqa_logits_gather(*args, cand, block)
        tk = ops.idx_topk(pool, None, pend, k)
        remapped = ops.idx_remap_compact_topk(tk.clone(), cand, block)
        return logits, ends, bm, cand, masked, pool, pend, tk, remapped

    for name, call in (("decode", decode), ("per-row lengths", per_row), ("two-level", two_level)):
        assert both(call, f"{fmt} {name}") == 0, f"{fmt} {name}: a valid input was recorded as clamped"


@pytest.mark.parametrize("fmt", ["fp8", "mxfp4"])
def test_valid_prefill_and_producers_record_nothing(fmt):
    f = ops.FP8 if fmt == "fp8" else ops.MXFP4
    wl = workloads.paged_prefill(seed=71, M=45, N=900, H=64, width=1024, topk=16, fmt=fmt)
    pi = _inputs.paged_inputs(wl)
    bt = _unused_entries_to_minus_one(wl)[0]

    def prefill():
        return ops.idx_paged_prefill_logits(_dev(pi.pool), f, wl.page_size, _dev(pi.q),
                                            None if pi.q_scale is None else _dev(pi.q_scale), _dev(wl.w),
                                            _dev(wl.row_end), _dev(bt), wl.width)

    assert both(prefill, f"{fmt} prefill") == 0

    rng = np.random.default_rng(72)
    N, P, maxp, rope_dim, T, H = 300, 64, 4096, 64, 37, 64
    k = rng.standard_normal((N, 128)).astype(np.float32)
    slots = rng.permutation(((N + P - 1) // P + 2) * P)[:N].astype(np.int64)
    slots[::23] = -1  # padding
    pos = rng.integers(0, maxp, N).astype(np.int64)
    table = rng.uniform(-1.0, 1.0, (maxp, rope_dim)).astype(np.float32)
    wgt = rng.uniform(0.5, 1.5, 128).astype(np.float32)
    pb = ops.page_bytes(f, P)
    num_pages = (N + P - 1) // P + 2

    def store():
        pool = torch.zeros((num_pages, pb), dtype=torch.uint8, device=DEV)
        ops.idx_k_store(pool, f, P, _dev(k), _dev(slots))
        pool2 = torch.zeros_like(pool)
        ops.idx_k_norm_rope_store(pool2, f, P, _dev(k), _dev(slots), _dev(pos), _dev(table), rope_dim, _dev(wgt),
                                  1e-6)
        return pool, pool2

    q = rng.standard_normal((T, H, 128)).astype(np.float32)
    w = rng.standard_normal((T, H)).astype(np.float32)
    assert both(store, f"{fmt} k store") == 0
    assert both(lambda: ops.idx_q_rope_quant(_dev(q), f, _dev(pos[:T]), _dev(table), rope_dim, _dev(w), 0.01),
                f"{fmt} q rope quant") == 0


def test_mqa_logits_valid_records_nothing():
    M, N, H = 37, 301, 64
    starts = np.arange(M, dtype=np.int32) * 3
    wl = workloads.contiguous(seed=5, M=M, N=N, H=H, starts=starts, ends=np.minimum(starts + 250, N))
    ci = _inputs.contig_inputs(wl)
    args = (_dev(ci.q), _dev(ci.k), _dev(ci.k_scale), _dev(wl.w), _dev(wl.ks), _dev(wl.ke))

    def call():
        logits = ops.idx_mqa_logits(*args)
        return logits, ops.idx_topk(logits, args[4], args[5], 20)

    assert both(call, "mqa") == 0


# ---- each kind of out-of-range device value sets its own bit -----------------------


@pytest.mark.parametrize("fmt", ["fp8", "mxfp4"])
def test_lengths_are_recorded(fmt):
    wl, pi = _paged(fmt)
    # shared lengths: one sequence longer than the block table reaches, one negative
    # (the workload's own block table here: entries past a sequence's pages name a
    # valid page, so the longer length reads no entry outside the pool)
    ctx = wl.context_lens.copy()
    ctx[3], ctx[6] = 5000, -4
    bt = wl.block_table
    assert both(lambda: ops.idx_paged_mqa_logits(*_args(wl, pi, fmt, ctx=ctx, bt=bt), wl.width),
                "shared") == _abi.DBG_LENGTH
    # the gathered walk's own reading of the lengths
    block, n_cand = 32, 7
    _, ends, bm = ops.idx_paged_mqa_logits_block_max(*_args(wl, pi, fmt), wl.width, block)
    cand = ops.idx_candidate_blocks(bm, ends, block, n_cand)
    assert both(lambda: ops.idx_paged_mqa_logits_gather(*_args(wl, pi, fmt, ctx=ctx, bt=bt), cand, block),
                "gather") == _abi.DBG_LENGTH
    # row bounds of the top-k and of the candidate steps
    logits, ends = ops.idx_paged_mqa_logits(*_args(wl, pi, fmt), wl.width)
    bad_end = ends.clone()
    bad_end[2] = wl.width + 50
    assert both(lambda: ops.idx_topk(logits, None, bad_end, 16), "topk end") == _abi.DBG_LENGTH
    starts = torch.zeros_like(ends)
    starts[4] = -3
    assert both(lambda: ops.idx_topk(logits, starts, ends, 16), "topk start") == _abi.DBG_LENGTH
    assert both(lambda: ops.idx_candidate_blocks(bm, bad_end, block, n_cand), "candidates") == _abi.DBG_LENGTH
    assert both(lambda: ops.idx_apply_candidate_mask(_padded_copy(logits), bad_end, cand, block),
                "mask") == _abi.DBG_LENGTH


def test_mqa_and_prefill_lengths_are_recorded():
    M, N, H = 37, 301, 64
    starts = np.arange(M, dtype=np.int32) * 3
    ends = np.minimum(starts + 250, N).astype(np.int32)
    wl = workloads.contiguous(seed=5, M=M, N=N, H=H, starts=starts, ends=ends)
    ci = _inputs.contig_inputs(wl)
    ke = ends.copy()
    ke[5] = N + 9
    ks = starts.copy()
    ks[7] = -2
    for s, e, what in ((starts, ke, "end past N"), (ks, ends, "negative start")):
        args = (_dev(ci.q), _dev(ci.k), _dev(ci.k_scale), _dev(wl.w), _dev(s), _dev(e))
        assert both(lambda: ops.idx_mqa_logits(*args), what) == _abi.DBG_LENGTH
    for fmt in ("fp8", "mxfp4"):
        f = ops.FP8 if fmt == "fp8" else ops.MXFP4
        pw = workloads.paged_prefill(seed=74, M=45, N=900, H=64, width=1024, topk=16, fmt=fmt)
        pi = _inputs.paged_inputs(pw)
        re = pw.row_end.copy()
        re[3] = 5000
        assert both(lambda: ops.idx_paged_prefill_logits(
            _dev(pi.pool), f, pw.page_size, _dev(pi.q), None if pi.q_scale is None else _dev(pi.q_scale),
            _dev(pw.w), _dev(re), _dev(pw.block_table[0]), pw.width), f"prefill {fmt}") == _abi.DBG_LENGTH


@pytest.mark.parametrize("fmt", ["fp8", "mxfp4"])
def test_block_table_entries_are_recorded(fmt):
    wl, pi = _paged(fmt)
    for bad in (-2, wl.num_pages + 3):
        bt = _unused_entries_to_minus_one(wl)
        bt[5, 3] = bad  # a page the sequence of 1000 keys reads
        assert both(lambda: ops.idx_paged_mqa_logits(*_args(wl, pi, fmt, bt=bt), wl.width),
                    f"decode entry {bad}") == _abi.DBG_PAGE
        block, n_cand = 32, 31
        _, ends, bm = ops.idx_paged_mqa_logits_block_max(*_args(wl, pi, fmt), wl.width, block)
        cand = ops.idx_candidate_blocks(bm, ends, block, n_cand)  # 31 of 32 blocks: page 3 is in the pool
        assert both(lambda: ops.idx_paged_mqa_logits_gather(*_args(wl, pi, fmt, bt=bt), cand, block),
                    f"gather entry {bad}") == _abi.DBG_PAGE
    f = ops.FP8 if fmt == "fp8" else ops.MXFP4
    pw = workloads.paged_prefill(seed=75, M=45, N=900, H=64, width=1024, topk=16, fmt=fmt)
    pp = _inputs.paged_inputs(pw)
    bt = _unused_entries_to_minus_one(pw)[0]
    bt[13] = pw.num_pages + 1  # the last page: rows reach it
    assert both(lambda: ops.idx_paged_prefill_logits(
        _dev(pp.pool), f, pw.page_size, _dev(pp.q), None if pp.q_scale is None else _dev(pp.q_scale),
        _dev(pw.w), _dev(pw.row_end), _dev(bt), pw.width), f"prefill {fmt}") == _abi.DBG_PAGE


@pytest.mark.parametrize("fmt", ["fp8", "mxfp4"])
def test_slots_positions_and_sequences_are_recorded(fmt):
    f = ops.FP8 if fmt == "fp8" else ops.MXFP4
    rng = np.random.default_rng(76)
    N, P, maxp, rope_dim = 200, 64, 1024, 64
    num_pages = (N + P - 1) // P + 1
    k = rng.standard_normal((N, 128)).astype(np.float32)
    slots = rng.permutation(num_pages * P)[:N].astype(np.int64)
    slots[9] = num_pages * P + 5  # past the pool: dropped
    pos = rng.integers(0, maxp, N).astype(np.int64)
    table = rng.uniform(-1.0, 1.0, (maxp, rope_dim)).astype(np.float32)
    wgt = rng.uniform(0.5, 1.5, 128).astype(np.float32)
    pb = ops.page_bytes(f, P)

    def store(kind):
        pool = torch.zeros((num_pages, pb), dtype=torch.uint8, device=DEV)
        if kind == "plain":
            ops.idx_k_store(pool, f, P, _dev(k), _dev(slots))
        else:
            ops.idx_k_norm_rope_store(pool, f, P, _dev(k), _dev(slots), _dev(pos), _dev(table), rope_dim, _dev(wgt),
                                      1e-6)
        return pool

    assert both(lambda: store("plain"), "slot") == _abi.DBG_SLOT
    assert both(lambda: store("fused"), "slot, fused") == _abi.DBG_SLOT
    slots[9] = -1  # padding is not recorded
    assert both(lambda: store("fused"), "padding") == 0
    pos[4] = maxp + 7
    assert both(lambda: store("fused"), "k position") == _abi.DBG_POSITION
    T, H = 20, 64
    q = rng.standard_normal((T, H, 128)).astype(np.float32)
    w = rng.standard_normal((T, H)).astype(np.float32)
    qpos = rng.integers(0, maxp, T).astype(np.int64)
    qpos[3] = -1
    assert both(lambda: ops.idx_q_rope_quant(_dev(q), f, _dev(qpos), _dev(table), rope_dim, _dev(w), 0.01),
                "q position") == _abi.DBG_POSITION
    # sequence ids of top-k rows
    rows, kk, B, mb = 6, 16, 3, 4
    topk = rng.integers(-1, mb * P, (rows, kk)).astype(np.int32)
    bt = rng.integers(0, 50, (B, mb)).astype(np.int32)
    seq = np.array([0, 1, 2, 2, B + 2, 1], np.int32)
    assert both(lambda: ops.idx_topk_to_slots(_dev(topk), _dev(bt), P, row_seq=_dev(seq)), "row_seq") == _abi.DBG_SEQ


def test_flags_persist_until_cleared():
    wl, pi = _paged("fp8")
    ctx = wl.context_lens.copy()
    ctx[0] = -1
    with ops.debug_build():
        ops.idx_debug_flags(clear=True)
        ops.idx_paged_mqa_logits(*_args(wl, pi, "fp8", ctx=ctx), wl.width)
        assert ops.idx_debug_flags(clear=False) == _abi.DBG_LENGTH
        ops.idx_paged_mqa_logits(*_args(wl, pi, "fp8"), wl.width)  # valid: adds nothing, clears nothing
        assert ops.idx_debug_flags(clear=False) == _abi.DBG_LENGTH
        assert ops.idx_debug_flags(clear=True) == _abi.DBG_LENGTH
        assert ops.idx_debug_flags() == 0
