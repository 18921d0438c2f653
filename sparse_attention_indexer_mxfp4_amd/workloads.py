"""Seeded synthetic workloads for the indexer (NumPy only).

This module draws the raw inputs of an indexer call: full-precision query and key
rows, head weights, context lengths, the row ranges of a contiguous chunk, and the
page assignment of a paged K cache (block table and slot mapping). It holds none of
the indexer's arithmetic: no quantisation, no scoring, no masking, no top-k. Both the
GPU library's callers (tests, bench) and the CPU oracle's tests consume what it draws;
each side quantises and scores with its own code.

Shapes and distributions follow the workloads the vLLM pages describe for the
DeepSeek lightning indexer (pages ``vllm.v1.attention.ops.rocm_aiter_mla_sparse``,
functions ``fp8_mqa_logits_torch`` and ``rocm_fp8_paged_mqa_logits``; page
``vllm.v1.attention.ops.rocm_paged_mxfp4_indexer``, function
``rocm_mxfp4_sparse_attn_indexer``): D = 128, 64 heads (4 in the tiny case), pages of
64 keys, queries and keys drawn N(0, 1), head weights N(0, 1)/sqrt(H).
"""

from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np

FP8 = "fp8"
MXFP4 = "mxfp4"


@dataclass
class ContiguousWorkload:
    """One contiguous chunk: M query rows scored against N keys of one sequence."""

    name: str
    seed: int
    q: np.ndarray  # [M, H, D] float32
    k: np.ndarray  # [N, D] float32
    w: np.ndarray  # [M, H] float32
    ks: np.ndarray  # [M] int32, first valid key (inclusive)
    ke: np.ndarray  # [M] int32, end of valid keys (exclusive)
    topk: int

    @property
    def M(self) -> int:
        return self.q.shape[0]

    @property
    def H(self) -> int:
        return self.q.shape[1]

    @property
    def D(self) -> int:
        return self.q.shape[2]

    @property
    def N(self) -> int:
        return self.k.shape[0]


@dataclass
class PagedWorkload:
    """A decode / MTP step: B sequences, next_n query rows each, over a paged K cache.

    ``context_lens[b]`` is the number of keys sequence b holds in the cache (already
    divided by the compression ratio where the cache is compressed). Keys of sequence
    b are rows ``key_offsets[b] : key_offsets[b] + context_lens[b]`` of ``k``, in
    sequence order. Logical page p of sequence b lives in physical page
    ``block_table[b, p]``; entries past a sequence's last page name ``poison_page``, a
    page that holds no key of any sequence.
    """

    name: str
    seed: int
    fmt: str
    B: int
    next_n: int
    H: int
    D: int
    page_size: int
    width: int
    topk: int
    compress_ratio: int
    context_lens: np.ndarray  # [B] int32
    block_table: np.ndarray  # [B, max_blocks] int32
    num_pages: int  # pages in the pool, poison page included
    poison_page: int
    key_offsets: np.ndarray  # [B] int64
    slot_mapping: np.ndarray  # [sum(context_lens)] int64: physical page * page_size + offset
    q: np.ndarray  # [B, next_n, H, D] float32
    k: np.ndarray  # [sum(context_lens), D] float32
    w: np.ndarray  # [B * next_n, H] float32
    tokens: np.ndarray = field(default=None)  # [B] int64 uncompressed lengths (informational)

    @property
    def rows(self) -> int:
        return self.B * self.next_n

    @property
    def max_blocks(self) -> int:
        return self.block_table.shape[1]


def contiguous(
    seed: int,
    M: int,
    N: int,
    H: int,
    D: int = 128,
    topk: int = 16,
    causal_offset: int | None = None,
    starts: np.ndarray | None = None,
    ends: np.ndarray | None = None,
    name: str = "contiguous",
) -> ContiguousWorkload:
    """Draw a contiguous chunk. Row t's valid keys are [ks[t], ke[t]).

    By default the rows are the last M tokens of an N-token sequence: ks = 0 and
    ke = N - M + t + 1 (``causal_offset`` = N - M). Explicit ``starts``/``ends``
    override that.
    """
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((M, H, D), dtype=np.float32)
    k = rng.standard_normal((N, D), dtype=np.float32)
    w = (rng.standard_normal((M, H), dtype=np.float32) / np.float32(np.sqrt(H))).astype(np.float32)
    if ends is None:
        off = N - M if causal_offset is None else causal_offset
        ends = off + np.arange(M, dtype=np.int64) + 1
    if starts is None:
        starts = np.zeros(M, dtype=np.int64)
    return ContiguousWorkload(
        name=name,
        seed=seed,
        q=q,
        k=k,
        w=w,
        ks=np.asarray(starts, dtype=np.int32),
        ke=np.asarray(ends, dtype=np.int32),
        topk=topk,
    )


def paged(
    seed: int,
    B: int,
    next_n: int,
    H: int,
    ctx_lo: int,
    ctx_hi: int,
    width: int,
    topk: int,
    fmt: str = FP8,
    dist: str = "uniform",
    compress_ratio: int = 1,
    D: int = 128,
    page_size: int = 64,
    context_lens: np.ndarray | None = None,
    name: str = "paged",
) -> PagedWorkload:
    """Draw a paged decode / MTP step.

    Token lengths are drawn uniform on [ctx_lo, ctx_hi] (``dist="uniform"``) or
    log-uniform (``dist="loguniform"``, rounded), then divided by ``compress_ratio``
    to give the keys each sequence holds. Physical pages are a random permutation
    of the pool; one extra page (the poison page) fills block-table entries past a
    sequence's last page.
    """
    rng = np.random.default_rng(seed)
    if context_lens is None:
        if dist == "uniform":
            tokens = rng.integers(ctx_lo, ctx_hi + 1, size=B).astype(np.int64)
        elif dist == "loguniform":
            tokens = np.rint(np.exp(rng.uniform(np.log(ctx_lo), np.log(ctx_hi), size=B))).astype(np.int64)
        else:
            raise ValueError(dist)
        lens = tokens // compress_ratio
    else:
        lens = np.asarray(context_lens, dtype=np.int64)
        tokens = lens * compress_ratio
    max_blocks = -(-width // page_size)
    pages_per_seq = -(-lens // page_size)
    if np.any(pages_per_seq > max_blocks):
        raise ValueError("a sequence holds more keys than the logits width")
    used = int(pages_per_seq.sum())
    num_pages = used + 1
    poison = used
    perm = rng.permutation(used).astype(np.int64)
    block_table = np.full((B, max_blocks), poison, dtype=np.int32)
    key_offsets = np.zeros(B, dtype=np.int64)
    slot_parts = []
    p0 = 0
    k_off = 0
    for b in range(B):
        npg = int(pages_per_seq[b])
        block_table[b, :npg] = perm[p0 : p0 + npg]
        p0 += npg
        key_offsets[b] = k_off
        s = np.arange(int(lens[b]), dtype=np.int64)
        slot_parts.append(block_table[b, s // page_size].astype(np.int64) * page_size + s % page_size)
        k_off += int(lens[b])
    slot_mapping = np.concatenate(slot_parts) if slot_parts else np.zeros(0, dtype=np.int64)
    q = rng.standard_normal((B, next_n, H, D), dtype=np.float32)
    k = rng.standard_normal((int(lens.sum()), D), dtype=np.float32)
    w = (rng.standard_normal((B * next_n, H), dtype=np.float32) / np.float32(np.sqrt(H))).astype(np.float32)
    return PagedWorkload(
        name=name,
        seed=seed,
        fmt=fmt,
        B=B,
        next_n=next_n,
        H=H,
        D=D,
        page_size=page_size,
        width=width,
        topk=topk,
        compress_ratio=compress_ratio,
        context_lens=lens.astype(np.int32),
        block_table=block_table,
        num_pages=num_pages,
        poison_page=poison,
        key_offsets=key_offsets,
        slot_mapping=slot_mapping,
        q=q,
        k=k,
        w=w,
        tokens=tokens,
    )


@dataclass
class PagedPrefillWorkload(PagedWorkload):
    """A prefill chunk of one sequence over a paged K cache: ``q`` is [M, H, D], ``w``
    [M, H], and row t scores keys [0, row_end[t]) of the sequence (B = 1)."""

    row_end: np.ndarray = field(default=None)  # [M] int32

    @property
    def rows(self) -> int:
        return self.q.shape[0]

    @property
    def M(self) -> int:
        return self.q.shape[0]


def paged_prefill(seed: int, M: int, N: int, H: int, width: int, topk: int, fmt: str = MXFP4, D: int = 128,
                  page_size: int = 64, name: str = "paged prefill") -> PagedPrefillWorkload:
    """One sequence of N cached keys in pages (random physical order) and M query rows
    at its end: row t ends at N - M + t + 1 (causal)."""
    base = paged(seed=seed, B=1, next_n=1, H=H, ctx_lo=0, ctx_hi=0, width=width, topk=topk, fmt=fmt, D=D,
                 page_size=page_size, context_lens=np.array([N]), name=name)
    rng = np.random.default_rng(seed + 1000)
    q = rng.standard_normal((M, H, D), dtype=np.float32)
    w = (rng.standard_normal((M, H), dtype=np.float32) / np.float32(np.sqrt(H))).astype(np.float32)
    row_end = (N - M + 1 + np.arange(M)).astype(np.int32)
    fields = {f: getattr(base, f) for f in base.__dataclass_fields__}
    fields.update(q=q, w=w)
    return PagedPrefillWorkload(**fields, row_end=row_end)


def config6() -> PagedPrefillWorkload:
    """Paged MXFP4 prefill chunk: one sequence, 8192 rows x 8192 keys in pages of 64,
    causal, H = 64, top-2048 (the prefill chunk of the contiguous workload, read off
    the paged MXFP4 cache)."""
    return paged_prefill(seed=5, M=8192, N=8192, H=64, width=8192, topk=2048, fmt=MXFP4,
                         name="paged mxfp4 prefill causal M=N=8192 H=64")


# The five workloads the indexer is measured on.
def config1() -> ContiguousWorkload:
    """Contiguous fp8, one sequence: T = 4 rows, S = 256 keys, H = 4; row t ends at S - T + t + 1; top-16."""
    return contiguous(seed=0, M=4, N=256, H=4, topk=16, name="contiguous fp8 T=4 S=256 H=4")


def config2() -> PagedWorkload:
    """Paged fp8 decode: 32 sequences, lengths U[1024, 16384], width 32768, top-2048."""
    return paged(seed=1, B=32, next_n=1, H=64, ctx_lo=1024, ctx_hi=16384, width=32768, topk=2048,
                 fmt=FP8, name="paged fp8 decode B=32 ctx U[1024,16384] H=64")


def config3() -> PagedWorkload:
    """Paged fp8 MTP decode: 128 sequences x 2 rows, lengths log-uniform [4096, 65536], width 65536, top-2048."""
    return paged(seed=2, B=128, next_n=2, H=64, ctx_lo=4096, ctx_hi=65536, width=65536, topk=2048,
                 fmt=FP8, dist="loguniform", name="paged fp8 MTP B=128 next_n=2 ctx logU[4096,65536] H=64")


def config4() -> ContiguousWorkload:
    """Contiguous fp8 prefill chunk: 8192 rows x 8192 keys, causal (row t sees [0, t]), H = 64, top-2048."""
    return contiguous(seed=3, M=8192, N=8192, H=64, topk=2048, causal_offset=0,
                      name="prefill fp8 causal M=N=8192 H=64")


def config5() -> PagedWorkload:
    """Paged MXFP4 decode: 64 sequences, tokens U[8192, 131072] compressed 4:1, width 32768, top-512."""
    return paged(seed=4, B=64, next_n=1, H=64, ctx_lo=8192, ctx_hi=131072, width=32768, topk=512,
                 fmt=MXFP4, compress_ratio=4, name="paged mxfp4 decode B=64 ctx U[8192,131072]/4 H=64")


CONFIGS = {1: config1, 2: config2, 3: config3, 4: config4, 5: config5}
# further workloads measured the same way (a second workload on the same kernels)
EXTRA = {6: config6}
