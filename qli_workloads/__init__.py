"""Seeded synthetic inputs for the quantized lightning indexer (QLI).

This module only draws random inputs and lays them out the way the
DeepSeek V4.1 QLI developer guide describes its caches ("Data flow"
section: TND queries, PA_BBND paged index K with an FP16 per-token scale
packed after the KV inside four-slot shared pages; ratio-2 views hold 64
rows at a 131072-byte page stride, ratio-1 views 128 rows at 147712 bytes).
It holds none of the indexer's arithmetic: no dot products, no rounding of
scores, no selection.  Both the oracle and the GPU path consume what it
returns.

Distributions (the five named workloads): Q and K int8 uniform on
[-127, 127]; q_scale and k_scale fp16 uniform on [1e-3, 1e-2]; head weights
fp16 N(0, 0.1).  Float draws are made in float64 and rounded to fp16 by
numpy (round-to-nearest-even).

Page layout inside one shared page (the developer guide only says the index
K and its scale sit after the KV; the split below follows from
147712 = 128 * (1024 + 128 + 2)):
    ratio 1: [KV 128 x 1024 B][K 128 x 128 B @131072][scale 128 x 2 B @147456]
    ratio 2: [KV  64 x 1024 B][K  64 x 128 B @ 65536][scale  64 x 2 B @ 73728]
             (page padded to 131072 B by larger aliased members)
Unused rows and pages are poisoned (K byte 127, scale 60000.0) so that a
stray read changes results.
"""
from __future__ import annotations

from dataclasses import dataclass, field
import math

import numpy as np

HEAD_DIM = 128
BLOCK_POSITIONS = 8          # positions per candidate block
RAW_TOKENS_PER_PAGE = 128    # --block-size 128: one block id per 128 raw tokens

POISON_K = np.int8(127)
POISON_S = np.float16(60000.0).view(np.uint16)

# tensor ids for independent streams
_TID_Q, _TID_QS, _TID_W, _TID_K, _TID_KS, _TID_BT, _TID_CAND, _TID_REQ, _TID_XQ, _TID_XK, \
    _TID_WF, _TID_SLOT = range(12)


def page_layout(ratio: int):
    """(page_rows, page_stride_bytes, k_offset, s_offset) for one ratio."""
    if ratio == 1:
        return 128, 147712, 131072, 147456
    if ratio == 2:
        return 64, 131072, 65536, 73728
    raise ValueError("ratio must be 1 or 2")


def _rng(seed: int, *ids: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, *ids])))


def _int8_uniform(rng, shape):
    return rng.integers(-127, 128, size=shape, dtype=np.int8)


def _f16_uniform(rng, shape, lo=1e-3, hi=1e-2):
    return rng.uniform(lo, hi, size=shape).astype(np.float16).view(np.uint16)


def _f16_normal(rng, shape, std=0.1):
    return rng.normal(0.0, std, size=shape).astype(np.float16).view(np.uint16)


@dataclass
class Problem:
    """One indexer call: metadata, queries, paged K and scalars.

    K lives in a host-side compact pool ``k_pages[num_pages, R, 128]`` /
    ``s_pages[num_pages, R]`` (page stride R*128 and R*2 bytes).  The device
    pool re-lays the same pages at the real strides (``page_bytes``,
    ``k_offset``, ``s_offset``); the indexer only sees base pointers and
    strides, so both layouts describe the same cache.
    """
    name: str
    ratio: int
    num_heads: int
    mode: int                    # 1 plain, 2 candidate source, 3 candidate consumer
    topk: int
    cand_blocks: int             # output candidate width (mode 2)
    cand_in_blocks: int          # incoming candidate width (mode 3)
    query_start_loc: np.ndarray  # int32 [B+1]
    k_lens: np.ndarray           # int32 [B] compressed lengths
    seq_mod: np.ndarray | None   # int32 [B] raw length mod ratio (None at ratio 1)
    raw_lens: np.ndarray         # int64 [B] raw lengths (bookkeeping only)
    q: np.ndarray                # int8 [T, N, 128]
    q_scale: np.ndarray          # fp16 bits uint16 [T, N]
    weights: np.ndarray          # fp16 bits uint16 [T, N]
    block_table: np.ndarray      # int32 [B, bt_stride]
    k_pages: np.ndarray          # int8 [num_pages, R, 128]
    s_pages: np.ndarray          # fp16 bits uint16 [num_pages, R]
    cand_in: np.ndarray | None = None   # int32 [T, 1, cand_in_blocks]
    seed: int = 0
    meta: dict = field(default_factory=dict)

    @property
    def batch(self):
        return int(self.k_lens.shape[0])

    @property
    def num_tokens(self):
        return int(self.q.shape[0])

    @property
    def page_rows(self):
        return int(self.k_pages.shape[1])

    @property
    def num_pages(self):
        return int(self.k_pages.shape[0])

    @property
    def max_k_len(self):
        return int(self.k_lens.max()) if self.batch else 0

    def layout(self):
        return page_layout(self.ratio)


@dataclass
class Requests:
    """Per-request query counts n_b and raw lengths S_b, in TND order."""
    n: np.ndarray
    S: np.ndarray


def make_block_table(seed: int, raw_lens, extra_pages: int = 0, pages_needed=None):
    """Shuffled page ids: one page per 128 raw tokens of each request.

    Returns (block_table [B, bt_stride], num_pages, pages_per_request).
    Unassigned table entries are -1.
    """
    raw_lens = np.asarray(raw_lens, dtype=np.int64)
    if pages_needed is None:
        pages_needed = -(-raw_lens // RAW_TOKENS_PER_PAGE)
    pages_needed = np.asarray(pages_needed, dtype=np.int64)
    total = int(pages_needed.sum())
    num_pages = max(total + extra_pages, 1)
    perm = _rng(seed, _TID_BT).permutation(num_pages).astype(np.int32)
    bt_stride = max(int(pages_needed.max()) if len(pages_needed) else 1, 1)
    bt = np.full((len(raw_lens), bt_stride), -1, dtype=np.int32)
    off = 0
    for b, p in enumerate(pages_needed):
        bt[b, :p] = perm[off:off + p]
        off += int(p)
    return bt, num_pages, pages_needed


def fill_pages(seed: int, layer: int, ratio: int, k_lens, block_table, num_pages):
    """Random K rows / scales for each request's compressed positions,
    scattered into a poisoned compact pool through the block table."""
    R = page_layout(ratio)[0]
    k_pages = np.full((num_pages, R, HEAD_DIM), POISON_K, dtype=np.int8)
    s_pages = np.full((num_pages, R), POISON_S, dtype=np.uint16)
    for b, L in enumerate(np.asarray(k_lens)):
        L = int(L)
        if L == 0:
            continue
        rk = _rng(seed, _TID_K, layer, b)
        rs = _rng(seed, _TID_KS, layer, b)
        npg = -(-L // R)
        pages = block_table[b, :npg]
        k = _int8_uniform(rk, (npg * R, HEAD_DIM))
        s = _f16_uniform(rs, (npg * R,))
        k[L:] = POISON_K
        s[L:] = POISON_S
        k_pages[pages] = k.reshape(npg, R, HEAD_DIM)
        s_pages[pages] = s.reshape(npg, R)
    return k_pages, s_pages


def make_queries(seed: int, layer: int, T: int, N: int):
    q = _int8_uniform(_rng(seed, _TID_Q, layer), (T, N, HEAD_DIM))
    qs = _f16_uniform(_rng(seed, _TID_QS, layer), (T, N))
    w = _f16_normal(_rng(seed, _TID_W, layer), (T, N))
    return q, qs, w


def visible_counts(req: Requests, ratio: int):
    """Per token visible compressed count under the causal reading:
    the n_b queries are the last raw positions of the request, a compressed
    entry j covers raw [j*r, (j+1)*r) and is visible once complete.

    Used only to draw candidate ids that include the last visible block
    (input construction, not scoring).
    """
    out = []
    for n, S in zip(req.n, req.S):
        for i in range(int(n)):
            p = int(S) - int(n) + i
            out.append((p + 1) // ratio)
    return np.asarray(out, dtype=np.int64)


def make_candidates(seed: int, layer: int, vis, cb_in: int, p_invalid: float = 1 / 16,
                    messy: bool = False):
    """Incoming candidate block ids [T, 1, cb_in] for a consumer layer.

    Per token: the last visible block at a random slot, plus distinct
    random earlier blocks, each independently replaced by -1 with
    probability ``p_invalid``.  With ``messy`` the list also carries
    duplicates, ids past the visible range and large ids.
    """
    rng = _rng(seed, _TID_CAND, layer)
    T = len(vis)
    out = np.full((T, 1, cb_in), -1, dtype=np.int32)
    for t, V in enumerate(vis):
        nb = -(-int(V) // BLOCK_POSITIONS)
        if nb == 0:
            if messy:
                out[t, 0, : min(4, cb_in)] = rng.integers(0, 50, size=min(4, cb_in))
            continue
        last = nb - 1
        others = min(cb_in - 1, last)
        ids = rng.choice(last, size=others, replace=False).astype(np.int32) if others else \
            np.zeros(0, np.int32)
        row = np.concatenate([ids, np.asarray([last], np.int32)])
        if p_invalid > 0:
            drop = rng.random(len(row)) < p_invalid
            drop[-1] = False  # keep the last visible block
            row[drop] = -1
        if messy and cb_in - len(row) > 0:
            room = cb_in - len(row)
            extra = []
            extra += list(rng.choice(row, size=min(room, 8)))          # duplicates
            extra += [nb + 3, nb, 10**9, -7][: max(0, room - len(extra))]  # invisible / junk
            row = np.concatenate([row, np.asarray(extra[:room], np.int32)])
        rng.shuffle(row)
        out[t, 0, : len(row)] = row
    return out


def build_problem(name: str, seed: int, req: Requests, ratio: int, num_heads: int,
                  mode: int, topk: int, cand_blocks: int = 0, cand_in_blocks: int = 0,
                  layer: int = 0, block_table=None, num_pages=None, extra_pages: int = 8,
                  cand_policy: str = "random", p_invalid: float = 1 / 16) -> Problem:
    n = np.asarray(req.n, dtype=np.int64)
    S = np.asarray(req.S, dtype=np.int64)
    assert np.all(n <= S) and np.all(n >= 0)
    L = (S // ratio).astype(np.int32)
    seq_mod = None if ratio == 1 else (S % ratio).astype(np.int32)
    qsl = np.zeros(len(n) + 1, dtype=np.int32)
    qsl[1:] = np.cumsum(n)
    T = int(qsl[-1])
    if block_table is None:
        R = page_layout(ratio)[0]
        block_table, num_pages, _ = make_block_table(
            seed, S, extra_pages=extra_pages, pages_needed=-(-L.astype(np.int64) // R))
    k_pages, s_pages = fill_pages(seed, layer, ratio, L, block_table, num_pages)
    q, qs, w = make_queries(seed, layer, T, num_heads)
    cand = None
    if mode == 3 and cand_policy != "external":
        vis = visible_counts(req, ratio)
        cand = make_candidates(seed, layer, vis, cand_in_blocks, p_invalid=p_invalid,
                               messy=(cand_policy == "messy"))
    return Problem(name=name, ratio=ratio, num_heads=num_heads, mode=mode, topk=topk,
                   cand_blocks=cand_blocks, cand_in_blocks=cand_in_blocks,
                   query_start_loc=qsl, k_lens=L, seq_mod=seq_mod, raw_lens=S,
                   q=q, q_scale=qs, weights=w, block_table=block_table,
                   k_pages=k_pages, s_pages=s_pages, cand_in=cand, seed=seed)


# ---------------------------------------------------------------------------
# The five named workloads
# ---------------------------------------------------------------------------

def tiny():
    """1 request, raw 256, ratio 2 (128 compressed positions, 16 blocks),
    32 heads, the last 4 raw positions as queries, topk 16, 64 candidate
    blocks, 64-row pages drawn from a shuffled pool of 8, seed 0."""
    req = Requests(n=np.array([4]), S=np.array([256]))
    return build_problem("tiny", 0, req, ratio=2, num_heads=32, mode=2, topk=16,
                         cand_blocks=64, extra_pages=6)


def decode_source():
    """64 requests x 1 query token, raw context 32768, ratio 1, 64 heads,
    128-row pages at 147712 B (256 per request, 16384-page shuffled pool),
    topk 2048, 512 candidate blocks, seed 1."""
    req = Requests(n=np.ones(64, np.int64), S=np.full(64, 32768))
    return build_problem("decode_source", 1, req, ratio=1, num_heads=64, mode=2,
                         topk=2048, cand_blocks=512, extra_pages=0)


def prefill_chunk():
    """1 request, 8192 query tokens at the end of a 20032-token raw
    sequence, ratio 2 (10016 compressed positions, 64-row pages at
    131072 B), 64 heads, topk 2048, 2048 candidate blocks, seed 2."""
    req = Requests(n=np.array([8192]), S=np.array([20032]))
    return build_problem("prefill_chunk", 2, req, ratio=2, num_heads=64, mode=2,
                         topk=2048, cand_blocks=2048, extra_pages=157)


def decode_consumer_1m():
    """32 requests x 1 token, raw context 1048576, ratio 2 (524288
    compressed positions), 64 heads, consumer: incoming [32,1,2048]
    candidate ids (last visible block + random others, 1/16 set to -1),
    position topk 2048 inside the candidate blocks, seed 3."""
    req = Requests(n=np.ones(32, np.int64), S=np.full(32, 1048576))
    return build_problem("decode_consumer_1m", 3, req, ratio=2, num_heads=64, mode=3,
                         topk=2048, cand_in_blocks=2048, extra_pages=0)


def mixed_requests(seed: int = 4):
    """48 requests: 40 decode tokens with raw lengths log-uniform on
    [1, 131072] (two forced to 1: an empty compressed context at ratio 2)
    and 8 prefill chunks of 512-4096 tokens with raw lengths log-uniform on
    [n, 131072]; TND order shuffled."""
    rng = _rng(seed, _TID_REQ)
    nd, npf = 40, 8
    Sd = np.exp(rng.uniform(0.0, math.log(131072), size=nd)).round().astype(np.int64)
    Sd = np.clip(Sd, 1, 131072)
    Sd[:2] = 1
    npre = rng.integers(512, 4097, size=npf)
    Sp = np.array([int(round(math.exp(rng.uniform(math.log(m), math.log(131072)))))
                   for m in npre], dtype=np.int64)
    Sp = np.maximum(Sp, npre)
    n = np.concatenate([np.ones(nd, np.int64), npre.astype(np.int64)])
    S = np.concatenate([Sd, Sp])
    odd = S % 2 == 1
    if odd.sum() < len(S) // 4:  # at least a quarter odd raw lengths
        fix = np.flatnonzero(~odd)[: len(S) // 4 - int(odd.sum())]
        S[fix] += 1
    order = rng.permutation(len(n))
    return Requests(n=n[order], S=S[order])


def mixed_calls(seed: int = 4):
    """The four layer calls of the mixed batch on one request set and one
    block table (128-token blocks serve both ratios): (ratio 1, source),
    (ratio 1, consumer of that source), (ratio 2, source), (ratio 2,
    consumer).  32 heads.  Per call topk ~ U[1, 2048] and candidate width
    64 * U{1..32}.  Consumer calls carry ``cand_in=None``: they are fed
    the source call's candidate output."""
    req = mixed_requests(seed)
    rng = _rng(seed, _TID_REQ, 1)
    bt, num_pages, _ = make_block_table(seed, req.S, extra_pages=16)
    calls = []
    for ratio in (1, 2):
        topk_s, topk_c = (int(x) for x in rng.integers(1, 2049, size=2))
        cb = 64 * int(rng.integers(1, 33))
        src = build_problem(f"mixed_r{ratio}_source", seed, req, ratio, 32, 2, topk_s,
                            cand_blocks=cb, layer=2 * ratio, block_table=bt,
                            num_pages=num_pages)
        con = build_problem(f"mixed_r{ratio}_consumer", seed, req, ratio, 32, 3, topk_c,
                            cand_in_blocks=cb, layer=2 * ratio + 1, block_table=bt,
                            num_pages=num_pages, cand_policy="external")
        calls += [src, con]
    return calls


WORKLOADS = {
    "tiny": tiny,
    "decode_source": decode_source,
    "prefill_chunk": prefill_chunk,
    "decode_consumer_1m": decode_consumer_1m,
}


# ---------------------------------------------------------------------------
# Un-quantized activations (inputs of query quantization and the K write)
# ---------------------------------------------------------------------------

def bf16_bits(x):
    """bfloat16 bit patterns (uint16) of float32 values, rounded to nearest
    even: the storage encoding of the activations, not indexer arithmetic."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    u = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return u.astype(np.uint16)


def bf16_to_f32(b):
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def make_activations(seed: int, layer: int, rows: int, dtype: str = "bf16", which: str = "q"):
    """Rows of 128 un-quantized values (query heads or new K positions).

    Each row is N(0, 1) times a per-row magnitude log-uniform on [0.05, 20]
    (heads and tokens differ in scale), with 1% of the values multiplied by
    8 (outlier channels).  Returns float32 [rows, 128] or bfloat16 bits
    (uint16) [rows, 128]."""
    rng = _rng(seed, _TID_XQ if which == "q" else _TID_XK, layer)
    mag = np.exp(rng.uniform(math.log(0.05), math.log(20.0), size=(rows, 1)))
    x = rng.normal(0.0, 1.0, size=(rows, HEAD_DIM)) * mag
    x = np.where(rng.random((rows, HEAD_DIM)) < 0.01, x * 8.0, x).astype(np.float32)
    return bf16_bits(x) if dtype == "bf16" else x


def make_head_weights(seed: int, layer: int, n: int, dtype: str = "bf16"):
    """Un-rounded head weights, N(0, 0.1): float32 [n] or bfloat16 bits."""
    w = _rng(seed, _TID_WF, layer).normal(0.0, 0.1, size=n).astype(np.float32)
    return bf16_bits(w) if dtype == "bf16" else w


def request_slots(block_table, k_lens, ratio: int, positions=None):
    """Flat cache slots (page * page_rows + row) of compressed positions.

    ``positions``: per request, an array of positions (default: all
    [0, k_lens[b])).  Input construction for the K write: where each new
    row of a request lands in the paged pool."""
    R = page_layout(ratio)[0]
    out = []
    for b, L in enumerate(np.asarray(k_lens)):
        j = np.arange(int(L), dtype=np.int64) if positions is None else \
            np.asarray(positions[b], dtype=np.int64)
        out.append(block_table[b, j // R].astype(np.int64) * R + j % R)
    return np.concatenate(out) if out else np.zeros(0, np.int64)
