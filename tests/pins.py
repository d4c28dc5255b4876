"""Pins of the CPU oracle against facts that do not come from the oracle.

Each ``pin_*`` function raises AssertionError when the oracle disagrees with
something fixed independently of it: IEEE binary16 as numpy implements it,
closed-form values that follow from the golden order of the QLI developer
guide (section "当前 A3 契约"), numpy integer matrix products, brute-force
rank counting, special cases whose answer has a closed form, and invariants
that the guide's "数据流" section states (causal visibility, 8-position
blocks, the pinned last visible block, chronological order, -1 padding at
the tail, empty contexts).

The functions are plain so that they can also run against a deliberately
broken copy of the oracle (see test_oracle_mutations.py).
"""
from __future__ import annotations

import json
import os

import numpy as np

import oracle
import qli_workloads as W

HERE = os.path.dirname(os.path.abspath(__file__))
GOLDEN = json.load(open(os.path.join(HERE, "golden", "closed_forms.json")))


# ---------------------------------------------------------------------------
# helpers (independent of the oracle's code)
# ---------------------------------------------------------------------------

def small_problem(seed, ratio=2, N=32, mode=2, topk=16, cb=64, cb_in=64,
                  requests=((4, 300), (1, 77), (3, 3), (2, 2048)), cand_policy="random"):
    req = W.Requests(n=np.array([r[0] for r in requests]), S=np.array([r[1] for r in requests]))
    return W.build_problem(f"small{seed}", seed, req, ratio, N, mode, topk,
                           cand_blocks=cb, cand_in_blocks=cb_in, cand_policy=cand_policy)


def dense_k(pb, b):
    """Logical K rows [L, 128] (int32) and k-scales [L] (float64) of request b,
    gathered with numpy through the block table."""
    L = int(pb.k_lens[b])
    R = pb.page_rows
    j = np.arange(L)
    pages = pb.block_table[b, j // R]
    rows = j % R
    k = pb.k_pages[pages, rows].astype(np.int32)
    ks = pb.s_pages[pages, rows].view(np.float16).astype(np.float64)
    return k, ks


def token_requests(pb):
    qsl = pb.query_start_loc
    return np.searchsorted(qsl, np.arange(pb.num_tokens), side="right") - 1


def visible(pb):
    """Visible counts from the causal reading, computed from the workload's
    raw lengths (not from the oracle's metadata path)."""
    out = []
    for b in range(pb.batch):
        n = int(pb.query_start_loc[b + 1] - pb.query_start_loc[b])
        S = int(pb.raw_lens[b])
        out += [(S - n + i + 1) // pb.ratio for i in range(n)]
    return np.asarray(out, np.int64)


def eligible_sets(pb, cand_in=None):
    vis = visible(pb)
    cand = cand_in if cand_in is not None else pb.cand_in
    sets = []
    for t, V in enumerate(vis):
        if pb.mode == 3:
            blocks = {int(c) for c in cand[t, 0] if 0 <= int(c) and 8 * int(c) < V}
            sets.append(sorted(j for c in blocks for j in range(8 * c, min(8 * c + 8, V))))
        else:
            sets.append(list(range(V)))
    return sets


def rank_select(keys, ids, k):
    """Brute force: an item is selected iff fewer than k items beat it
    (higher key, or equal key and lower id).  Returns ascending ids."""
    keys = [0.0 if x == 0 else float(x) for x in keys]
    sel = []
    for a in range(len(ids)):
        beat = 0
        for c in range(len(ids)):
            if keys[c] > keys[a] or (keys[c] == keys[a] and ids[c] < ids[a]):
                beat += 1
        if beat < k:
            sel.append(ids[a])
    return sorted(sel)


def padded(vals, width):
    out = np.full(width, -1, np.int32)
    out[: len(vals)] = vals
    return out


# ---------------------------------------------------------------------------
# pins
# ---------------------------------------------------------------------------

def pin_f16_conversion():
    """binary16 decode/encode agrees with numpy on every bit pattern, on
    every half-way point and on random doubles (ties to even, subnormals,
    overflow to infinity)."""
    bits = np.arange(65536, dtype=np.uint16)
    ref = bits.view(np.float16).astype(np.float64)
    got = oracle.f16_value(bits)
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], ref[~nan])
    assert np.array_equal(oracle.f16_round(ref[~nan]), bits[~nan])
    pos = np.sort(ref[(~nan) & (ref >= 0) & np.isfinite(ref)])
    mids = (pos[:-1] + pos[1:]) / 2.0
    probe = np.concatenate([mids, np.nextafter(mids, np.inf), np.nextafter(mids, -np.inf),
                            [65519.0, 65520.0, 65535.0, 1e6, 2.0 ** -25, 2.0 ** -26]])
    probe = np.concatenate([probe, -probe])
    with np.errstate(over="ignore"):
        ref_probe = probe.astype(np.float16).view(np.uint16)
    assert np.array_equal(oracle.f16_round(probe), ref_probe)
    rng = np.random.default_rng(11)
    r = np.exp2(rng.uniform(-30, 17, 200000)) * rng.choice([-1.0, 1.0], 200000)
    with np.errstate(over="ignore"):
        ref_r = r.astype(np.float16).view(np.uint16)
    assert np.array_equal(oracle.f16_round(r), ref_r)


def _constructed(q_rows, k_rows, w_bits, qs_bits, ks_bits=0x3C00):
    """One request, one query token seeing every constructed K row, heads
    given explicitly (q_rows [N,128], k_rows [L,128])."""
    q_rows = np.asarray(q_rows, np.int8)
    k_rows = np.asarray(k_rows, np.int8)
    N, L = q_rows.shape[0], k_rows.shape[0]
    pb = small_problem(5, ratio=1, N=N, mode=1, topk=max(L, 1), requests=((1, L),))
    k_pages = np.full_like(pb.k_pages, 127)
    s_pages = np.full_like(pb.s_pages, 0x7B53)
    R = pb.page_rows
    for j in range(L):
        k_pages[pb.block_table[0, j // R], j % R] = k_rows[j]
        s_pages[pb.block_table[0, j // R], j % R] = ks_bits
    pb.k_pages, pb.s_pages = k_pages, s_pages
    pb.q = q_rows[None].copy()
    pb.weights = np.full((1, N), w_bits, np.uint16)
    pb.q_scale = np.full((1, N), qs_bits, np.uint16)
    return pb


def _dot_pair(target):
    """int8 vectors (q, k) in [-127,127] with q.k == target (|target| <= 127*127*128)."""
    q, k = np.zeros(128, np.int64), np.zeros(128, np.int64)
    T, sgn = abs(target), (1 if target >= 0 else -1)
    # q = 127 on dims 0..126 with k summing to S there, plus one free pair (a, b)
    for a in range(0, 128):
        for b in range(0, 128):
            S, r = divmod(T - a * b, 127)
            if r == 0 and 0 <= S <= 127 * 127:
                q[:127] = 127
                full, part = divmod(S, 127)
                k[:full] = 127
                if full < 127:
                    k[full] = part
                q[127], k[127] = a, b
                assert int(q @ k) == T
                return q, sgn * k
    raise AssertionError(f"no int8 construction for {target}")


def pin_closed_forms():
    """qk -> fp16(qk/1024) -> ReLU values and fp16 products from the
    closed-form fixtures."""
    ks = 0x3C00
    for e in GOLDEN["qk_to_fp16"]:
        q, k = _dot_pair(e["qk"])
        pb = _constructed([q], [k], 0x3C00, 0x3C00, ks)
        tm = oracle.OracleProblem(pb).terms(0, 0)
        assert tm["qk"][0] == e["qk"], (tm["qk"][0], e)
        assert oracle.f16_value(tm["x"][:1])[0] == e["x"], (e, tm["x"])
    for e in GOLDEN["fp16_products"]:
        q, k = _dot_pair(e["qk"])
        pb = _constructed([q], [k], e["b_bits"], 0x3C00, ks)  # m = fp16(b * 1) = b
        tm = oracle.OracleProblem(pb).terms(0, 0)
        assert tm["x"][0] == e["a_bits"] and tm["m"][0] == e["b_bits"]
        assert tm["p"][0] == e["p_bits"], (hex(tm["p"][0]), e)


def pin_head_multipliers():
    """m = fp16(w * q_scale) agrees with numpy's binary16 product for every
    (token, head) of the tiny workload."""
    pb = W.tiny()
    o = oracle.OracleProblem(pb)
    ref = (pb.weights.view(np.float16) * pb.q_scale.view(np.float16)).view(np.uint16)
    for t in range(pb.num_tokens):
        assert np.array_equal(o.terms(t, 0)["m"], ref[t])


def pin_integer_dot():
    """INT32 Q.K equals a numpy integer matrix product through the block table."""
    for ratio in (1, 2):
        pb = small_problem(7 + ratio, ratio=ratio, N=32, requests=((3, 700), (2, 260)))
        o = oracle.OracleProblem(pb)
        treq = token_requests(pb)
        rng = np.random.default_rng(ratio)
        for t in range(pb.num_tokens):
            b = treq[t]
            k, _ = dense_k(pb, b)
            ref = pb.q[t].astype(np.int32) @ k.T  # [N, L]
            for j in rng.choice(len(k), size=6, replace=False):
                assert np.array_equal(o.terms(t, int(j))["qk"], ref[:, j])


def _identical_heads(pb, w_sign):
    """Every head of a token replicates head 0; one K scale everywhere."""
    pb.q = np.repeat(pb.q[:, :1], pb.num_heads, axis=1).copy()
    w = np.abs(pb.weights[:, :1].view(np.float16)) * np.float16(w_sign)
    pb.weights = np.repeat(w.view(np.uint16), pb.num_heads, axis=1).copy()
    pb.q_scale = np.repeat(pb.q_scale[:, :1], pb.num_heads, axis=1).copy()
    pb.s_pages = np.full_like(pb.s_pages, np.float16(0.005).view(np.uint16))
    return pb


def pin_identical_heads():
    """With all heads identical and one K scale, the head sum is N*p exactly,
    so score = fp32(N * p * ks) and the position top-k is a textbook
    maximum-inner-product top-k of ReLU'd integer dot products (w > 0), or a
    tie-heavy selection where every non-positive product scores zero (w < 0)."""
    for w_sign, mode in ((1.0, 2), (-1.0, 1)):
        pb = _identical_heads(small_problem(21, ratio=2, N=64, mode=mode, topk=24,
                                            requests=((3, 500), (1, 130))), w_sign)
        o = oracle.OracleProblem(pb)
        res = o.run(want_scores=True)
        vis, treq = visible(pb), token_requests(pb)
        for t in range(pb.num_tokens):
            k, ks = dense_k(pb, treq[t])
            V = int(vis[t])
            qk = (pb.q[t, 0].astype(np.int32) @ k[:V].T).astype(np.float64)
            x = (qk / 1024.0).astype(np.float16)
            x = np.where(x > 0, x, np.float16(0))
            m = pb.weights[t, 0].view(np.float16) * pb.q_scale[t, 0].view(np.float16)
            p = (x * m).astype(np.float64)
            score = (p * pb.num_heads * ks[:V]).astype(np.float32)
            got = res["scores"][t, :V]
            assert np.array_equal(got, score), t
            order = np.lexsort((np.arange(V), -score.astype(np.float64)))
            want = padded(np.sort(order[: pb.topk]), pb.topk)
            assert np.array_equal(res["topk"][t], want), t
            if w_sign > 0:  # ordering by score == ordering by qk up to fp16 ties
                assert np.all(np.diff(qk[order[: pb.topk]]) <= 0)


def pin_sum_bound():
    """FP32 head sum within the recursive-summation bound of the exact sum,
    and equal to an ascending-order float32 accumulation done by numpy."""
    pb = small_problem(31, ratio=1, N=64, requests=((2, 400),))
    o = oracle.OracleProblem(pb)
    rng = np.random.default_rng(3)
    u = 2.0 ** -24
    for t in range(pb.num_tokens):
        for j in rng.choice(int(visible(pb)[t]), size=12, replace=False):
            tm = o.terms(t, int(j))
            p = tm["p"].view(np.float16).astype(np.float64)
            exact = p.sum()
            assert tm["exact_sum_q24"] == int(round(exact * 2 ** 24))
            n = len(p)
            gamma = (n - 1) * u / (1 - (n - 1) * u)
            assert abs(float(tm["sum"]) - exact) <= gamma * np.abs(p).sum()
            acc = np.float32(0)
            for v in p.astype(np.float32):
                acc = np.float32(acc + v)
            assert acc == tm["sum"]


def _check_selection(pb, res, cand_in=None):
    sets = eligible_sets(pb, cand_in)
    vis = visible(pb)
    for t, E in enumerate(sets):
        sc = res["scores"][t]
        want = padded(rank_select([sc[j] for j in E], E, pb.topk), pb.topk)
        assert np.array_equal(res["topk"][t], want), (pb.name, t)
        if pb.mode == 2:
            V = int(vis[t])
            nb = -(-V // 8)
            if nb == 0:
                assert np.all(res["cand"][t] == -1)
                continue
            bs = [max(sc[j] for j in range(8 * c, min(8 * c + 8, V))) for c in range(nb - 1)]
            sel = rank_select(bs, list(range(nb - 1)), pb.cand_blocks - 1) + [nb - 1]
            assert np.array_equal(res["cand"][t], padded(sorted(sel), pb.cand_blocks)), t


def pin_selection_bruteforce():
    """Position top-k and candidate blocks equal a brute-force rank count on
    small inputs, in all three modes, including heavy ties."""
    cases = [
        small_problem(41, ratio=2, N=32, mode=2, topk=16, cb=64),
        small_problem(42, ratio=1, N=32, mode=2, topk=40, cb=64, requests=((2, 700), (1, 9))),
        small_problem(43, ratio=2, N=32, mode=1, topk=7),
        small_problem(44, ratio=2, N=32, mode=3, topk=30, cb_in=64, cand_policy="messy"),
        small_problem(45, ratio=1, N=64, mode=3, topk=2048, cb_in=64),
    ]
    ties = _identical_heads(small_problem(46, ratio=1, N=32, mode=2, topk=50, cb=64,
                                          requests=((2, 600),)), -1.0)
    cases.append(ties)
    for pb in cases:
        # a small candidate width so that block selection is not trivial
        if pb.mode == 2:
            pb.cand_blocks = 64 if pb.max_k_len > 8 * 64 else pb.cand_blocks
        res = oracle.OracleProblem(pb).run(want_scores=True)
        _check_selection(pb, res)


def pin_small_cand_width():
    """Block selection with fewer slots than visible blocks (the pin then
    displaces a block): cb = 64 against up to 256 visible blocks."""
    pb = small_problem(47, ratio=1, N=32, mode=2, topk=100, cb=64, requests=((3, 2048),))
    res = oracle.OracleProblem(pb).run(want_scores=True)
    _check_selection(pb, res)


def pin_invariants():
    """Stated invariants on random problems: indices inside the eligible
    set, ascending, -1 only at the tail, count = min(k, |E|); source:
    min(cb, blocks) candidates, last visible block present, no duplicates;
    consumer: positions inside incoming blocks; empty context: all -1."""
    cases = [small_problem(s, ratio=r, N=32, mode=m, topk=k, cb=64, cb_in=64,
                           requests=((5, 900), (1, 1), (2, 2), (1, 513), (3, 64)))
             for s, r, m, k in ((51, 2, 2, 33), (52, 1, 2, 2048), (53, 2, 3, 100), (54, 1, 1, 1))]
    for pb in cases:
        res = oracle.OracleProblem(pb).run()
        vis = visible(pb)
        for t, E in enumerate(eligible_sets(pb)):
            row = res["topk"][t]
            valid = row[row >= 0]
            nvalid = len(valid)
            assert np.all(row[nvalid:] == -1) and np.all(np.diff(valid) > 0)
            assert nvalid == min(pb.topk, len(E))
            assert set(valid.tolist()) <= set(E)
            if vis[t] == 0:
                assert nvalid == 0
            if pb.mode == 2:
                c = res["cand"][t]
                cv = c[c >= 0]
                nb = -(-int(vis[t]) // 8)
                assert np.all(c[len(cv):] == -1) and np.all(np.diff(cv) > 0)
                assert len(cv) == min(pb.cand_blocks, nb)
                if nb:
                    assert cv[-1] == nb - 1
            if pb.mode == 3:
                blocks = set(int(x) for x in pb.cand_in[t, 0] if x >= 0)
                assert all(j // 8 in blocks for j in valid)


def pin_cross_mode():
    """Mode 1 positions equal mode 2 positions; a consumer fed every visible
    block equals the source; a consumer fed the source's own candidates
    equals the source when the candidates cover the whole context."""
    pb = small_problem(61, ratio=2, N=32, mode=2, topk=20, cb=64, requests=((4, 1000), (2, 30)))
    src = oracle.OracleProblem(pb).run()
    pb.mode = 1
    plain = oracle.OracleProblem(pb).run()
    assert np.array_equal(src["topk"], plain["topk"])
    pb.mode = 3
    pb.cand_in_blocks = 64
    vis = visible(pb)
    allblocks = np.full((pb.num_tokens, 1, 64), -1, np.int32)
    for t, V in enumerate(vis):
        nb = -(-int(V) // 8)
        allblocks[t, 0, :nb] = np.arange(nb)[::-1]  # any order
    con = oracle.OracleProblem(pb, cand_in=allblocks).run()
    assert np.array_equal(con["topk"], src["topk"])
    con2 = oracle.OracleProblem(pb, cand_in=src["cand"][:, None, :]).run()
    assert np.array_equal(con2["topk"], src["topk"])


def pin_layout_invariance():
    """Renumbering the pages (block table and pool permuted together) leaves
    every output unchanged."""
    pb = small_problem(71, ratio=1, N=32, mode=2, topk=64, requests=((2, 600), (1, 200)))
    a = oracle.OracleProblem(pb).run()
    perm = np.random.default_rng(1).permutation(pb.num_pages).astype(np.int32)
    k2 = np.empty_like(pb.k_pages)
    s2 = np.empty_like(pb.s_pages)
    k2[perm] = pb.k_pages
    s2[perm] = pb.s_pages
    bt = np.where(pb.block_table >= 0, perm[np.maximum(pb.block_table, 0)], -1)
    pb.k_pages, pb.s_pages, pb.block_table = k2, s2, bt.astype(np.int32)
    b = oracle.OracleProblem(pb).run()
    assert np.array_equal(a["topk"], b["topk"]) and np.array_equal(a["cand"], b["cand"])


def pin_visibility():
    """Visible counts of the tiny workload match the closed-form fixture, and
    the last query of a request sees the whole compressed context."""
    pb = W.tiny()
    o = oracle.OracleProblem(pb)
    assert [o.token_view(t)[1] for t in range(4)] == GOLDEN["tiny_visible"]["V"]
    pb = small_problem(81, ratio=2, N=32, mode=1, topk=2048,
                       requests=((3, 301), (2, 2), (1, 1), (4, 900)))
    res = oracle.OracleProblem(pb).run()
    qsl = pb.query_start_loc
    for b in range(pb.batch):
        if qsl[b + 1] == qsl[b]:
            continue
        last = qsl[b + 1] - 1
        L = int(pb.k_lens[b])
        row = res["topk"][last]
        assert np.array_equal(row[:L], np.arange(L)) and np.all(row[L:] == -1)


ALL_PINS = [pin_f16_conversion, pin_closed_forms, pin_head_multipliers, pin_integer_dot,
            pin_identical_heads, pin_sum_bound, pin_selection_bruteforce,
            pin_small_cand_width, pin_invariants, pin_cross_mode, pin_layout_invariance,
            pin_visibility]


def run_all():
    """Run every pin; return the names of those that fail."""
    failed = []
    for f in ALL_PINS:
        try:
            f()
        except Exception as e:  # noqa: BLE001 - any failure counts
            failed.append(f"{f.__name__}: {type(e).__name__}")
    return failed
