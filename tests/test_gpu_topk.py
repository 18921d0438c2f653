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


@pytest.mark.parametrize("width,k", [(8192, 2048), (3001, 64), (300, 256)])
def test_topk_many_rows_in_registers(width, k):
    # 1024 rows or more of at most 8192 columns: one 256-thread workgroup per row, keys
    # in registers. Rows of every length class: empty, shorter than k, exactly k, k + 1,
    # full; unaligned starts; heavy ties; all equal; -inf inside the range
    rng = np.random.default_rng(width + k + 1)
    rows = 1500
    L = rng.standard_normal((rows, width)).astype(np.float32)
    L[0::7] = np.round(L[0::7] * 2) / 2
    L[1::7] = 0.5
    L[2::7, : width // 3] = -np.inf
    starts = rng.integers(0, 9, rows)
    ends = rng.integers(0, width + 1, rows)
    ends[3::11] = np.minimum(starts[3::11] + k, width)
    ends[4::11] = np.minimum(starts[4::11] + k + 1, width)
    ends[5::11] = width
    ends[6::11] = starts[6::11]
    np.testing.assert_array_equal(_run(L, starts, ends, k), indexer.topk(L.astype(np.float64), starts, ends, k))


# ---- several workgroups per row (up to 256 rows of more than 65536 columns, 16-byte aligned)
def _oracle(L, starts, ends, k):
    return indexer.topk(L.astype(np.float64), starts, ends, k)


def test_topk_coop_repeated_calls():
    # the per-row records in the workspace must come back zeroed after every call:
    # three calls in a row on different data and row counts, each against the oracle
    rng = np.random.default_rng(11)
    for rows, width, k in ((32, 100000, 2048), (7, 70000, 700), (64, 131072, 512)):
        L = rng.standard_normal((rows, width)).astype(np.float32)
        ends = rng.integers(1, width + 1, rows)
        ends[0] = width
        ends[1] = k  # a row of exactly k keys: no selection
        ends[2] = 70000  # one unit may hold it whole
        starts = rng.integers(0, 7, rows)
        np.testing.assert_array_equal(_run(L, starts, ends, k), _oracle(L, starts, ends, k))


def test_topk_coop_full_rows_several_passes():
    # 256 rows of 131072 keys: more units than the device holds at once would be needed
    # for units that fit the registers, so every phase re-reads its columns in passes
    rng = np.random.default_rng(12)
    rows, width, k = 256, 131072, 2048
    L = rng.standard_normal((rows, width)).astype(np.float32)
    ends = np.full(rows, width)
    ends[::5] = rng.integers(k + 1, width, ends[::5].size)
    np.testing.assert_array_equal(_run(L, None, ends, k), _oracle(L, None, ends, k))


@pytest.mark.parametrize("ties", [False, True])
def test_topk_coop_one_long_row(ties):
    # one row of a million keys spread over hundreds of workgroups
    rng = np.random.default_rng(13)
    width, k = 1_000_000, 2048
    L = rng.standard_normal((1, width)).astype(np.float32)
    if ties:
        L = np.round(L * 4) / 4
    ends = np.array([width - 3])
    starts = np.array([5])
    np.testing.assert_array_equal(_run(L, starts, ends, k), _oracle(L, starts, ends, k))


@pytest.mark.parametrize("shared_prefix", [False, True])
def test_topk_coop_crowded_bin(shared_prefix):
    # The k-th key sits in a crowd of keys sharing its top 11 bits - more than the
    # per-row list holds - so the units meet again over a second row histogram. With
    # distinct 22-bit prefixes (values 1 + i 2^-13) the crowd's prefix of T is small and
    # goes to the list; with one shared prefix (values 1 + j 2^-23, j < 1024) it
    # overflows too, and T comes from a third histogram. 500 keys lie above the crowd;
    # ties go to the lowest columns.
    rng = np.random.default_rng(14 + shared_prefix)
    rows, width, k = 3, 100000, 2048
    L = rng.standard_normal((rows, width)).astype(np.float32) - 10.0
    for r in range(rows):
        cols = rng.choice(width, 6000, replace=False)
        step, top = (2.0 ** -23, 1024) if shared_prefix else (2.0 ** -13, 2048)
        L[r, cols] = (1.0 + rng.integers(0, top, 6000) * step).astype(np.float32)
        L[r, rng.choice(np.setdiff1d(np.arange(width), cols), 500, replace=False)] = 5.0
    ends = np.full(rows, width)
    np.testing.assert_array_equal(_run(L, None, ends, k), _oracle(L, None, ends, k))


@pytest.mark.parametrize("rows,width,k", [(32, 100000, 2048), (5, 300000, 64)])
def test_topk_coop_matches_one_workgroup_per_row(rows, width, k):
    # the same rows through both kernels: a row pointer off 16-byte alignment takes the
    # one-workgroup-per-row kernel
    rng = np.random.default_rng(rows + k)
    L = rng.standard_normal((rows, width + 1)).astype(np.float32)
    ends = rng.integers(0, width + 1, rows)
    lt = torch.from_numpy(L).to(DEV)
    en = torch.from_numpy(ends.astype(np.int32)).to(DEV)
    aligned = torch.empty((rows, -(-width // 4) * 4), dtype=torch.float32, device=DEV)[:, :width]
    aligned.copy_(lt[:, 1:])
    off = lt[:, 1:]  # rows start 4 bytes past a 16-byte boundary
    a = ops.idx_topk(aligned, None, en, k)
    b = ops.idx_topk(off, None, en, k)
    torch.cuda.synchronize()
    want = _oracle(L[:, 1:], None, ends, k)
    np.testing.assert_array_equal(a.cpu().numpy(), want)
    np.testing.assert_array_equal(b.cpu().numpy(), want)


@pytest.mark.parametrize("next_n,valid", [(1, False), (2, True)])
def test_topk_to_slots_matches_oracle(next_n, valid):
    from oracle import indexer as oi
    rng = np.random.default_rng(410 + next_n)
    B, P, mb, k = 9, 16, 12, 40
    rows = B * next_n
    bt = rng.permutation(B * mb + 5)[:B * mb].reshape(B, mb).astype(np.int32)
    topk = rng.integers(-1, P * mb + 3, (rows, k)).astype(np.int32)  # pads and out-of-table entries too
    topk[0, :] = -1
    rv = (rng.random(rows) > 0.3).astype(np.uint8) if valid else None
    slots, indptr, lens = ops.idx_topk_to_slots(torch.from_numpy(topk).to(DEV), torch.from_numpy(bt).to(DEV), P,
                                                next_n=next_n,
                                                row_valid=None if rv is None else torch.from_numpy(rv).to(DEV))
    want_s, want_p, want_l = oi.topk_to_slots(topk, np.arange(rows) // next_n, bt, P, rv)
    ip = indptr.cpu().numpy()
    np.testing.assert_array_equal(ip, want_p)
    np.testing.assert_array_equal(lens.cpu().numpy(), want_l)
    np.testing.assert_array_equal(slots.cpu().numpy()[: ip[-1]], want_s)


def test_topk_to_slots_after_topk_and_empty():
    # the real chain: paged-style rows through idx_topk, then to slots; and no rows
    rng = np.random.default_rng(420)
    rows, width, k, P = 6, 300, 32, 16
    L = torch.from_numpy(rng.standard_normal((rows, width)).astype(np.float32)).to(DEV)
    ends = torch.tensor([300, 10, 0, 150, 299, 33], dtype=torch.int32, device=DEV)
    out = ops.idx_topk(L, None, ends, k)
    bt = torch.from_numpy(rng.permutation(200)[: rows * 19].reshape(rows, 19).astype(np.int32)).to(DEV)
    slots, indptr, lens = ops.idx_topk_to_slots(out, bt, P)
    from oracle import indexer as oi
    want_s, want_p, _ = oi.topk_to_slots(out.cpu().numpy(), np.arange(rows), bt.cpu().numpy(), P)
    np.testing.assert_array_equal(indptr.cpu().numpy(), want_p)
    np.testing.assert_array_equal(slots.cpu().numpy()[: want_p[-1]], want_s)
    e_slots, e_indptr, e_lens = ops.idx_topk_to_slots(torch.zeros((0, k), dtype=torch.int32, device=DEV), bt, P)
    assert e_indptr.cpu().tolist() == [0] and e_lens.numel() == 0


@pytest.mark.parametrize("rows,width,k", [(1100, 4100, 300), (20, 40000, 2048)])
def test_topk_aligned_rows(rows, width, k):
    # rows starting on 16-byte boundaries take the vector first pass: lengths that are
    # not multiples of 4 or of a 256-key step, the 256-thread variant (>= 1024 rows),
    # rows whose selected bin is too large for the candidate list (all equal, or few
    # distinct values), and rows longer than the key cache
    rng = np.random.default_rng(rows + width)
    L = rng.standard_normal((rows, width)).astype(np.float32)
    L[0] = 2.5
    L[1] = np.round(L[1])
    L[2, ::2] = -np.inf
    L[3] = np.float32(1e-3) * rng.integers(0, 3, width)
    starts = 4 * rng.integers(0, width // 16, rows)
    ends = np.minimum(starts + rng.integers(1, width, rows), width)
    starts[:6], ends[:6] = 0, width
    ends[6] = starts[6] + k + 1
    ends[7] = starts[7] + 3
    ends[8] = starts[8] + 257
    got = _run(L, starts, ends, k)
    np.testing.assert_array_equal(got, indexer.topk(L.astype(np.float64), starts, ends, k))


def _long_rows(rng, rows, width, k):
    """Rows of up to 65536 keys: lengths from 0 to the width (log-spread, with the key
    cache's size and the k-boundaries among them), ties across the middle of a row, a
    row's best keys all in one half, -inf over a half, signed zeros."""
    L = rng.standard_normal((rows, width)).astype(np.float32)
    lens = np.exp(rng.uniform(np.log(1), np.log(width), rows)).astype(np.int64)
    special = np.minimum([width, width - 1, 32768, 32769, 8192, 8193, 2 * k + 8, 2 * k + 9, k, k + 1, 0, 1], width)
    m = min(len(special), rows - 6)
    lens[6:6 + m] = special[:m]
    L[0] = 0.75  # every key ties: the k lowest columns
    L[1] = np.round(L[1] * 2) / 2  # heavy ties
    half = width // 2
    L[2, half:] += 8.0  # the row's best keys all in the second half
    L[3, :half] += 8.0  # ... all in the first half
    L[4, :half] = -np.inf
    L[5, ::2] = -0.0
    L[5, 1::2] = 0.0
    lens[:6] = width
    return L, lens


@pytest.mark.parametrize("rows,width,k", [(12, 30000, 2048), (40, 65536, 512), (129, 40000, 2048),
                                          (256, 65536, 2048)])
def test_topk_long_rows(rows, width, k):
    # decode-shaped steps: up to 256 rows of up to 65536 keys, rows longer than the key
    # cache keeping 16-bit prefixes; unaligned starts take the unaligned read
    rng = np.random.default_rng(rows + width + k)
    L, lens = _long_rows(rng, rows, width, k)
    starts = np.zeros(rows, np.int64)
    starts[6::9] = 3
    ends = np.minimum(starts + lens, width)
    got = _run(L, starts, ends, k)
    np.testing.assert_array_equal(got, indexer.topk(L.astype(np.float64), starts, ends, k))


def test_topk_kernels_alternate_on_one_workspace():
    # the one-workgroup and several-workgroups kernels alternate on the same workspace,
    # which the latter must leave clear
    rng = np.random.default_rng(11)
    for rows, width, k in [(256, 65536, 2048), (8, 70000, 2048), (40, 50000, 2048), (8, 131072, 512),
                           (256, 60000, 1024)]:
        L, lens = _long_rows(rng, rows, width, k)
        ends = np.minimum(lens, width)
        got = _run(L, None, ends, k)
        np.testing.assert_array_equal(got, indexer.topk(L.astype(np.float64), None, ends, k),
                                      err_msg=f"rows {rows} width {width} k {k}")
