"""Seeded synthetic inputs for the sparse-attention consumer of the indexer.

Like the rest of this package it only draws random inputs and lays them out;
it holds none of the attention's arithmetic (no dot products, no softmax).

Layout (BF16, TND queries, PA_BBND caches with one latent KV head):
  - queries q [T, H, D] BF16 bits;
  - the compressed cache is the KV member of the shared pages the indexer's
    K lives in (ratio 1: 128 rows of 1024 B at a 147712-byte page stride,
    ratio 2: 64 rows at 131072 bytes; the KV rows start at byte 0 of the
    page), D = 512 BF16 values per row;
  - the raw cache (sliding-window stage) is a pool of its own: 128 rows of
    D BF16 values per page, pages back to back;
  - block tables of shuffled page ids for both caches;
  - indices [T, topk]: request-local compressed positions in ascending
    order with -1 padding at the tail, as the indexer returns them;
  - sinks: one FP32 logit per head.
Value distributions: q and KV values N(0, 1) rounded to BF16; sinks uniform
on [-2, 2]; softmax scale 1/sqrt(D).  Unused rows of the pools keep a
poison value (BF16 of 1e4) so that a stray read changes results.
"""
from __future__ import annotations

from dataclasses import dataclass
import math

import numpy as np

from . import _rng, bf16_bits, page_layout

ATTN_DIM = 512             # D: key/value width of a cache entry (1024 B rows)
RAW_PAGE_ROWS = 128
POISON_KV = np.uint16(0x461C)  # BF16 1.0e4 (exactly 9984)

_TID_AQ, _TID_AKV, _TID_ARAW, _TID_AIDX, _TID_ASINK, _TID_ABT = range(40, 46)


@dataclass
class AttnProblem:
    name: str
    num_heads: int
    head_dim: int
    topk: int
    window: int
    scale: float
    q: np.ndarray              # uint16 [T, H, D]
    query_start_loc: np.ndarray  # int32 [B + 1]
    c_lens: np.ndarray         # int32 [B]
    r_lens: np.ndarray         # int32 [B]
    c_pages: np.ndarray        # uint8 [num_c_pages, c_page_stride]
    c_page_rows: int
    c_page_stride: int
    c_bt: np.ndarray           # int32 [B, c_bt_stride]
    r_pages: np.ndarray        # uint8 [num_r_pages, r_page_stride]
    r_page_rows: int
    r_page_stride: int
    r_bt: np.ndarray           # int32 [B, r_bt_stride]
    indices: np.ndarray        # int32 [T, topk]
    sinks: np.ndarray | None   # float32 [H]

    @property
    def num_tokens(self):
        return int(self.q.shape[0])

    @property
    def batch(self):
        return int(len(self.c_lens))


def _shuffled_table(seed, tid, pages_per_req):
    pages_per_req = np.asarray(pages_per_req, dtype=np.int64)
    total = max(int(pages_per_req.sum()), 1)
    perm = _rng(seed, tid).permutation(total).astype(np.int32)
    stride = max(int(pages_per_req.max()) if len(pages_per_req) else 1, 1)
    bt = np.full((len(pages_per_req), stride), -1, dtype=np.int32)
    off = 0
    for b, p in enumerate(pages_per_req):
        bt[b, :p] = perm[off:off + p]
        off += int(p)
    return bt, total


def _bf16_normal(rng, shape):
    return bf16_bits(rng.normal(0.0, 1.0, size=shape).astype(np.float32))


def _fill_rows(pages, bt, rows_per_page, D, lens, seed, tid, positions=None):
    """Random BF16 rows at each request's positions (all of [0, len) unless
    ``positions[b]`` lists the rows that will be read)."""
    view = pages.view(np.uint16)
    words_per_page = pages.shape[1] // 2
    for b, L in enumerate(np.asarray(lens)):
        pos = np.arange(int(L), dtype=np.int64) if positions is None else \
            np.unique(np.asarray(positions[b], dtype=np.int64))
        if len(pos) == 0:
            continue
        vals = _bf16_normal(_rng(seed, tid, b), (len(pos), D))
        page = bt[b, pos // rows_per_page].astype(np.int64)
        start = page * words_per_page + (pos % rows_per_page) * D
        flat = view.reshape(-1)
        for d0 in range(0, D, 64):  # scatter in column blocks (bounded temporaries)
            idx = start[:, None] + np.arange(d0, min(D, d0 + 64))[None, :]
            flat[idx] = vals[:, d0:d0 + idx.shape[1]]


def make_indices(seed, q_counts, c_lens, topk, layer=0, pad_frac=0.0, sparse_rows=None):
    """Per token: min(topk, visible) distinct positions of its request in
    ascending order, -1 after; ``pad_frac`` of the tokens keep only part of
    them.  Every compressed position of a request counts as visible (the
    attention reads what the indexer selected; the indexer's causality is
    its own concern)."""
    rng = _rng(seed, _TID_AIDX, layer)
    rows = []
    for b, (n, L) in enumerate(zip(np.asarray(q_counts), np.asarray(c_lens))):
        for _ in range(int(n)):
            k = min(topk, int(L))
            if pad_frac > 0 and rng.random() < pad_frac:
                k = int(rng.integers(0, k + 1))
            sel = np.sort(rng.choice(int(L), size=k, replace=False)) if k > 0 else np.zeros(0, np.int64)
            row = np.full(topk, -1, dtype=np.int32)
            row[:k] = sel
            rows.append(row)
    return np.stack(rows) if rows else np.zeros((0, topk), np.int32)


def build_attn_problem(name, seed, q_counts, c_lens, r_lens, ratio, num_heads, topk, window,
                       sinks=True, indices=None, pad_frac=0.0, fill_all=False, extra_indices=(),
                       window_pages_only=False):
    """An attention call over requests with q_counts[b] query tokens, compressed
    lengths c_lens[b] and raw lengths r_lens[b]; the compressed cache uses the
    indexer's shared page layout for ``ratio``.  The rows of ``extra_indices``
    (other index sets of the same shape, for timing with rotated inputs) are
    drawn too.  ``window_pages_only``: raw pages wholly before every token's
    window (never read) all map to one poisoned page, so the raw pool holds
    only the pages the window reaches."""
    q_counts = np.asarray(q_counts, dtype=np.int64)
    c_lens = np.asarray(c_lens, dtype=np.int64)
    r_lens = np.asarray(r_lens, dtype=np.int64)
    B = len(q_counts)
    T = int(q_counts.sum())
    D = ATTN_DIM
    qsl = np.zeros(B + 1, dtype=np.int32)
    qsl[1:] = np.cumsum(q_counts)
    c_rows, c_stride = page_layout(ratio)[:2]
    c_bt, c_np = _shuffled_table(seed, _TID_ABT, -(-c_lens // c_rows))
    if window_pages_only:
        first = np.maximum(0, r_lens - q_counts - window) // RAW_PAGE_ROWS  # first page a window reaches
        n_pages = -(-r_lens // RAW_PAGE_ROWS)
        live, _ = _shuffled_table(seed, _TID_ABT + 100, n_pages - first)
        r_np = int((n_pages - first).sum()) + 1
        r_bt = np.full((B, max(int(n_pages.max()), 1)), -1, dtype=np.int32)
        for b in range(B):
            r_bt[b, :first[b]] = r_np - 1          # the shared poisoned page
            r_bt[b, first[b]:n_pages[b]] = live[b, :n_pages[b] - first[b]]
    else:
        r_bt, r_np = _shuffled_table(seed, _TID_ABT + 100, -(-r_lens // RAW_PAGE_ROWS))
    if indices is None:
        indices = make_indices(seed, q_counts, c_lens, topk, pad_frac=pad_frac)
    indices = np.ascontiguousarray(indices, dtype=np.int32)
    # only the rows the call reads are drawn (the rest stays poisoned)
    c_pos = None
    r_pos = None
    if not fill_all:
        c_pos, r_pos = [], []
        for b in range(B):
            sel = np.concatenate([x[qsl[b]:qsl[b + 1]].reshape(-1) for x in (indices, *extra_indices)])
            c_pos.append(sel[(sel >= 0) & (sel < c_lens[b])])
            p_last = int(r_lens[b]) - 1
            p_first = int(r_lens[b]) - int(q_counts[b]) - window + 1
            r_pos.append(np.arange(max(0, p_first), p_last + 1) if window > 0 else np.zeros(0, np.int64))
    c_pages = np.empty((c_np, c_stride), dtype=np.uint8)
    c_pages.view(np.uint16)[:] = POISON_KV
    r_stride = RAW_PAGE_ROWS * D * 2
    r_pages = np.empty((r_np, r_stride), dtype=np.uint8)
    r_pages.view(np.uint16)[:] = POISON_KV
    _fill_rows(c_pages, c_bt, c_rows, D, c_lens, seed, _TID_AKV, c_pos)
    _fill_rows(r_pages, r_bt, RAW_PAGE_ROWS, D, r_lens, seed, _TID_ARAW, r_pos)
    q = _bf16_normal(_rng(seed, _TID_AQ), (T, num_heads, D))
    sk = _rng(seed, _TID_ASINK).uniform(-2.0, 2.0, size=num_heads).astype(np.float32) if sinks else None
    return AttnProblem(name=name, num_heads=num_heads, head_dim=D, topk=topk, window=window,
                       scale=1.0 / math.sqrt(D), q=q, query_start_loc=qsl,
                       c_lens=c_lens.astype(np.int32), r_lens=r_lens.astype(np.int32),
                       c_pages=c_pages, c_page_rows=c_rows, c_page_stride=c_stride, c_bt=c_bt,
                       r_pages=r_pages, r_page_rows=RAW_PAGE_ROWS, r_page_stride=r_stride, r_bt=r_bt,
                       indices=indices, sinks=sk)


def attn_decode(index_sets=1):
    """Decode attention after the decode_source indexer call: 64 requests x
    1 token, 32768 compressed positions (ratio 1, the indexer's 128-row pages
    at 147712 B), 2048 selected positions per token, a 128-position window
    over the raw cache, 64 heads, D = 512, sinks.  With index_sets > 1 the
    rows of that many independent index sets are drawn; returns the problem
    and the list of index sets (the problem's own first)."""
    B = 64
    q, c, r = [1] * B, np.full(B, 32768), np.full(B, 32768)
    extra = [make_indices(11 + 1000 * s, q, c, 2048) for s in range(1, index_sets)]
    ap = build_attn_problem("attn_decode", 11, q, c, r, 1, 64, 2048, 128, extra_indices=extra,
                            window_pages_only=True)
    return (ap, [ap.indices] + extra) if index_sets > 1 else ap


def attn_small():
    """A small mixed call: 5 requests (one without queries), ratio 2, 64
    heads, topk 96 (some rows padded), window 40."""
    return build_attn_problem("attn_small", 12, [3, 0, 1, 6, 2], [70, 40, 300, 129, 8], [141, 80, 601, 259, 17],
                              2, 64, 96, 40, pad_frac=0.3)
