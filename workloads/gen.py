"""Seeded synthetic inputs for paged-KV decode and chunked prefill.

Every array here is either a float32 standard-normal draw or an integer
layout (lengths, page permutation, block tables, slot mapping).  Nothing in
this module converts to a storage dtype or computes any part of attention.

Draw order for one workload, from ``numpy.random.Generator(PCG64(seed))``:
context (or prefix) lengths -> page permutation of the pool -> q -> K -> V.
Sequence ``b`` owns the next ``ceil(ctx_b / 16)`` pages of the permutation, in
order; the first page of the permutation that no sequence owns is the
*sentinel* page, and every unused block-table entry points at it (tests poison
that page, so a kernel that reads past a sequence's pages shows up).

The five named shapes are the attention shapes of the small models the pages
run (Qwen2.5-1.5B, Stories110M, TinyLlama-1.1B) at 16-token pages; they stand
in for the pages' trace-driven workloads, which are not used.
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import Optional, Sequence

import numpy as np

PAGE_SIZE = 16


@dataclass
class Workload:
    name: str
    kind: str                  # "decode" or "prefill"
    batch: int
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    kv_dtype: str              # "f32" | "bf16" | "f16" | "i8"
    q_dtype: str               # "f32" | "bf16" | "f16"
    out_dtype: str             # "f32" | "bf16" | "f16"
    num_pages: int
    sentinel_page: int
    context_lens: np.ndarray   # int32 [B]; includes the query tokens
    q_lens: np.ndarray         # int32 [B]; 1 per sequence for decode
    cu_q_lens: np.ndarray      # int32 [B+1]
    block_tables: np.ndarray   # int32 [B, max_blocks_per_seq]
    token_offsets: np.ndarray  # int64 [B+1]; start of sequence b in k/v/slots
    slot_mapping: np.ndarray   # int64 [sum ctx]; slot of every context token
    q: np.ndarray              # float32 [B, Hq, d] (decode) or [T, Hq, d]
    k: np.ndarray              # float32 [sum ctx, Hkv, d]
    v: np.ndarray              # float32 [sum ctx, Hkv, d]
    scale: float               # a float32 value
    seed: int = 0
    meta: dict = field(default_factory=dict)

    @property
    def page_size(self) -> int:
        return PAGE_SIZE

    @property
    def max_blocks_per_seq(self) -> int:
        return int(self.block_tables.shape[1])

    @property
    def max_context_len(self) -> int:
        return int(self.context_lens.max()) if self.batch else 0

    @property
    def max_q_len(self) -> int:
        return int(self.q_lens.max()) if self.batch else 0

    @property
    def num_query_tokens(self) -> int:
        return int(self.cu_q_lens[-1])

    def new_token_rows(self) -> np.ndarray:
        """Rows of k/v/slot_mapping holding the tokens whose queries run:
        the last token of each sequence (decode) or its whole chunk
        (prefill).  These are the tokens appended right before the call."""
        rows = []
        for b in range(self.batch):
            end = int(self.token_offsets[b + 1])
            rows.append(np.arange(end - int(self.q_lens[b]), end, dtype=np.int64))
        return np.concatenate(rows) if rows else np.zeros(0, np.int64)


def _build(name, kind, rng, ctx, q_lens, num_q_heads, num_kv_heads, head_dim,
           kv_dtype, q_dtype, out_dtype, num_pages, table_width, seed,
           scale=None, meta=None) -> Workload:
    ctx = np.asarray(ctx, dtype=np.int64)
    q_lens = np.asarray(q_lens, dtype=np.int64)
    batch = int(ctx.shape[0])
    nblocks = (ctx + PAGE_SIZE - 1) // PAGE_SIZE
    needed = int(nblocks.sum())
    if num_pages is None:
        num_pages = needed + 1            # exactly the needed pages + sentinel
    if needed + 1 > num_pages:
        raise ValueError(f"pool of {num_pages} pages cannot hold {needed} + sentinel")
    if table_width is None:
        table_width = max(1, int(nblocks.max()) if batch else 1)
    if batch and int(nblocks.max()) > table_width:
        raise ValueError("block table too narrow")
    perm = rng.permutation(num_pages).astype(np.int32)
    sentinel = int(perm[needed])
    block_tables = np.full((batch, table_width), sentinel, dtype=np.int32)
    offsets = np.zeros(batch + 1, dtype=np.int64)
    offsets[1:] = np.cumsum(ctx)
    slots = np.zeros(int(offsets[-1]), dtype=np.int64)
    page_cursor = 0
    for b in range(batch):
        nb = int(nblocks[b])
        block_tables[b, :nb] = perm[page_cursor:page_cursor + nb]
        page_cursor += nb
        t = np.arange(int(ctx[b]), dtype=np.int64)
        slots[offsets[b]:offsets[b + 1]] = (
            block_tables[b, t // PAGE_SIZE].astype(np.int64) * PAGE_SIZE + t % PAGE_SIZE)
    cu_q = np.zeros(batch + 1, dtype=np.int32)
    cu_q[1:] = np.cumsum(q_lens)
    total = int(offsets[-1])
    if kind == "decode":
        q = rng.standard_normal((batch, num_q_heads, head_dim), dtype=np.float32)
    else:
        q = rng.standard_normal((int(cu_q[-1]), num_q_heads, head_dim), dtype=np.float32)
    k = rng.standard_normal((total, num_kv_heads, head_dim), dtype=np.float32)
    v = rng.standard_normal((total, num_kv_heads, head_dim), dtype=np.float32)
    if scale is None:
        scale = float(np.float32(1.0) / np.sqrt(np.float32(head_dim)))
    return Workload(
        name=name, kind=kind, batch=batch, num_q_heads=num_q_heads,
        num_kv_heads=num_kv_heads, head_dim=head_dim, kv_dtype=kv_dtype,
        q_dtype=q_dtype, out_dtype=out_dtype, num_pages=int(num_pages),
        sentinel_page=sentinel, context_lens=ctx.astype(np.int32),
        q_lens=q_lens.astype(np.int32), cu_q_lens=cu_q,
        block_tables=block_tables, token_offsets=offsets, slot_mapping=slots,
        q=q, k=k, v=v, scale=float(np.float32(scale)), seed=seed,
        meta=dict(meta or {}))


def _c1(seed):
    rng = np.random.Generator(np.random.PCG64(seed))
    ctx = [17, 64, 133, 200]
    return _build("C1", "decode", rng, ctx, [1] * 4, 9, 3, 64, "f32", "f32", "f32",
                  64, 13, seed, scale=0.125,
                  meta={"desc": "paged decode, fp32 q/KV/out, B=4, 9/3 heads, d=64"})


def _c2(seed):
    rng = np.random.Generator(np.random.PCG64(seed))
    ctx = rng.integers(512, 4096, size=64, endpoint=True)
    return _build("C2", "decode", rng, ctx, [1] * 64, 12, 2, 128, "bf16", "f32", "f32",
                  20000, 256, seed,
                  meta={"desc": "paged decode, bf16 KV, Qwen2.5-1.5B shape, B=64, 12/2 heads, d=128"})


def _f1(seed):
    """The C2 draw (same seed, same values) stored as FP8 E4M3 codes."""
    w = _c2(seed)
    w.name, w.kv_dtype = "F1", "fp8"
    w.meta = {"desc": "paged decode, FP8 E4M3 KV + per-token-head fp32 scales, Qwen2.5-1.5B shape, B=64, 12/2 heads, d=128"}
    return w


def _c3(seed):
    rng = np.random.Generator(np.random.PCG64(seed))
    ctx = rng.integers(64, 1024, size=384, endpoint=True)
    return _build("C3", "decode", rng, ctx, [1] * 384, 12, 12, 64, "f16", "f32", "f32",
                  None, 64, seed,
                  meta={"desc": "paged decode, fp16 KV, Stories110M shape, B=384, 12/12 heads, d=64"})


def _c4(seed):
    rng = np.random.Generator(np.random.PCG64(seed))
    prefix = rng.integers(0, 3584, size=8, endpoint=True)
    chunk = np.full(8, 512)
    return _build("C4", "prefill", rng, prefix + chunk, chunk, 12, 2, 128, "bf16", "bf16",
                  "f32", 20000, 256, seed,
                  meta={"desc": "chunked causal prefill, bf16 q/KV, 8 x 512-token chunks, 12/2 heads, d=128",
                        "prefix_lens": prefix.astype(np.int32)})


def _c5(seed):
    rng = np.random.Generator(np.random.PCG64(seed))
    ctx = np.full(128, 2048)
    return _build("C5", "decode", rng, ctx, [1] * 128, 32, 4, 64, "i8", "f32", "f32",
                  None, 128, seed,
                  meta={"desc": "paged decode, int8 KV + per-token-head fp32 scales, TinyLlama-1.1B shape, B=128, 32/4 heads, d=64"})


EVICTED = -1   # block-table entry of a page a window-bounded cache has recycled


def _w1(seed):
    """Decode with a sliding window over long contexts, laid out the way a
    cache whose storage the window bounds holds it: only the pages that
    overlap each sequence's window (its last `window` positions) are
    allocated and drawn; block-table entries of earlier pages are EVICTED.
    k/v/slot_mapping hold the window tokens only (token_offsets delimit each
    sequence's), in position order.  Draw order: context lengths -> page
    permutation -> q -> K -> V."""
    window = 4096
    rng = np.random.Generator(np.random.PCG64(seed))
    ctx = rng.integers(16384, 65536, size=64, endpoint=True)
    batch, hq, hkv, d = 64, 12, 2, 128
    first = ctx - window
    p0 = first // PAGE_SIZE
    p1 = (ctx + PAGE_SIZE - 1) // PAGE_SIZE
    needed = int((p1 - p0).sum())
    num_pages = 20000
    perm = rng.permutation(num_pages).astype(np.int32)
    sentinel = int(perm[needed])
    table_width = int(p1.max())
    block_tables = np.full((batch, table_width), sentinel, dtype=np.int32)
    offsets = np.zeros(batch + 1, dtype=np.int64)
    offsets[1:] = np.cumsum(ctx - first)
    slots = np.zeros(int(offsets[-1]), dtype=np.int64)
    cursor = 0
    for b in range(batch):
        n = int(p1[b] - p0[b])
        block_tables[b, :p0[b]] = EVICTED
        block_tables[b, p0[b]:p1[b]] = perm[cursor:cursor + n]
        cursor += n
        t = np.arange(int(first[b]), int(ctx[b]), dtype=np.int64)
        slots[offsets[b]:offsets[b + 1]] = (
            block_tables[b, t // PAGE_SIZE].astype(np.int64) * PAGE_SIZE + t % PAGE_SIZE)
    q = rng.standard_normal((batch, hq, d), dtype=np.float32)
    k = rng.standard_normal((int(offsets[-1]), hkv, d), dtype=np.float32)
    v = rng.standard_normal((int(offsets[-1]), hkv, d), dtype=np.float32)
    return Workload(
        name="W1", kind="decode", batch=batch, num_q_heads=hq, num_kv_heads=hkv, head_dim=d,
        kv_dtype="bf16", q_dtype="f32", out_dtype="f32", num_pages=num_pages,
        sentinel_page=sentinel, context_lens=ctx.astype(np.int32),
        q_lens=np.ones(batch, dtype=np.int32), cu_q_lens=np.arange(batch + 1, dtype=np.int32),
        block_tables=block_tables, token_offsets=offsets, slot_mapping=slots, q=q, k=k, v=v,
        scale=float(np.float32(1.0) / np.sqrt(np.float32(d))), seed=seed,
        meta={"desc": "sliding-window decode, bf16 KV, Qwen2.5-1.5B shape, B=64, ctx U[16384,65536], window 4096, only window pages held",
              "window": window, "first_pos": first.astype(np.int64)})


def _mixed(name, seed):
    """A mixed batch in one varlen call: the C2 decode batch (64 one-token
    chunks at its context lengths) followed by prefill chunks: M1 takes the
    C4 chunks (8 x 512 tokens over its prefixes), M2 four 64-token chunks
    over 1024-token prefixes (a decode-heavy batch whose chunks are short).
    Qwen2.5-1.5B heads, bf16 q and KV, 20k-page pool, values drawn afresh
    from `seed`."""
    w2 = _c2(2)
    if name == "M1":
        w4 = _c4(4)
        chunks = [(int(c), int(q)) for c, q in zip(w4.context_lens, w4.q_lens)]
    else:
        chunks = [(1024 + 64, 64)] * 4
    ctx = [int(x) for x in w2.context_lens] + [c for c, _ in chunks]
    q_lens = [1] * w2.batch + [q for _, q in chunks]
    rng = np.random.Generator(np.random.PCG64(seed))
    return _build(name, "prefill", rng, ctx, q_lens, 12, 2, 128, "bf16", "bf16", "f32",
                  20000, 256, seed,
                  meta={"desc": f"mixed batch {name}: the C2 decode rows + "
                                + ("the C4 chunks" if name == "M1" else "4 x 64-token chunks over 1024-token prefixes")})


CONFIGS = {"C1": (_c1, 1), "C2": (_c2, 2), "C3": (_c3, 3), "C4": (_c4, 4), "C5": (_c5, 5),
           "W1": (_w1, 8), "F1": (_f1, 2), "M1": (lambda s: _mixed("M1", s), 6),
           "M2": (lambda s: _mixed("M2", s), 7)}


def make_workload(name: str, seed: Optional[int] = None) -> Workload:
    fn, default_seed = CONFIGS[name]
    return fn(default_seed if seed is None else seed)


def custom_workload(*, kind: str = "decode", context_lens: Sequence[int],
                    q_lens: Optional[Sequence[int]] = None, num_q_heads: int,
                    num_kv_heads: int, head_dim: int, kv_dtype: str = "f32",
                    q_dtype: str = "f32", out_dtype: str = "f32",
                    num_pages: Optional[int] = None, table_width: Optional[int] = None,
                    scale: Optional[float] = None, seed: int = 0,
                    name: str = "custom") -> Workload:
    """A small workload with explicit lengths (tests).  For prefill,
    ``q_lens[b] <= context_lens[b]``: the chunk is the last q_lens[b] tokens."""
    rng = np.random.Generator(np.random.PCG64(seed))
    ctx = list(context_lens)
    if q_lens is None:
        q_lens = [1 if c > 0 else 0 for c in ctx] if kind == "decode" else list(ctx)
    for c, ql in zip(ctx, q_lens):
        if ql > c:
            raise ValueError("query chunk longer than its context")
    return _build(name, kind, rng, ctx, list(q_lens), num_q_heads, num_kv_heads,
                  head_dim, kv_dtype, q_dtype, out_dtype, num_pages, table_width,
                  seed, scale=scale)
