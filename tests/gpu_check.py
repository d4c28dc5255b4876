"""Helpers of the GPU parity tests: run the HIP library on a generated
problem, compare with the oracle, check stated invariants."""
from __future__ import annotations

import sys

import numpy as np

import oracle
import qli_workloads as W


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def run_gpu(pb, cand_in=None, debug=False, layout=None, status=None, max_k_len=None):
    """One library call on cuda:0; numpy outputs (max_k_len: a looser bound
    than the problem's longest context)."""
    import torch

    import quantized_top_indexer_amd as Q
    from qli_workloads.device import call_kwargs, to_device
    dev = to_device(pb, "cuda", cand_in=cand_in, **(layout or {}))
    kw = call_kwargs(pb, dev)
    if max_k_len is not None:
        kw["max_k_len"] = max_k_len
    if pb.mode == 3 and kw["cand_in"] is None:
        raise ValueError("consumer call without candidates")
    idx, cand, dbg = Q.score_topk(**kw, debug_scores=debug, status_out=status)
    torch.cuda.synchronize()
    out = {"topk": idx[:, 0].cpu().numpy(),
           "cand": None if cand is None else cand[:, 0].cpu().numpy(),
           "scores": None if dbg is None else dbg.cpu().numpy()}
    del dev
    return out


def visible(pb):
    out = np.empty(pb.num_tokens, np.int64)
    for b in range(pb.batch):
        q0, q1 = int(pb.query_start_loc[b]), int(pb.query_start_loc[b + 1])
        n, S = q1 - q0, int(pb.raw_lens[b])
        out[q0:q1] = (S - n + np.arange(n) + 1) // pb.ratio
    return out


def eligible_count(pb, cand_in=None):
    vis = visible(pb)
    if pb.mode != 3:
        return vis
    cand = cand_in if cand_in is not None else pb.cand_in
    cnt = np.zeros(pb.num_tokens, np.int64)
    for t in range(pb.num_tokens):
        nb = -(-int(vis[t]) // 8)
        c = np.unique(cand[t, 0])
        c = c[(c >= 0) & (c < nb)]
        cnt[t] = np.minimum(8, vis[t] - 8 * c.astype(np.int64)).sum()
    return cnt


def check_invariants(pb, res, cand_in=None):
    """Ascending, -1 tail, count = min(k, |E|), indices visible (and inside
    incoming blocks for a consumer); source: min(cb, blocks) ascending
    candidates with the last visible block present."""
    vis = visible(pb)
    top = res["topk"]
    valid = top >= 0
    assert np.all(valid[:, 1:] <= valid[:, :-1]), "-1 not only at the tail"
    d = np.diff(top, axis=1)
    assert np.all((d > 0) | ~valid[:, 1:]), "indices not strictly ascending"
    assert np.all(np.where(valid, top, -1) < vis[:, None]), "index not visible"
    want = np.minimum(pb.topk, eligible_count(pb, cand_in))
    assert np.array_equal(valid.sum(1), want), "wrong number of indices"
    if pb.mode == 3:
        cand = cand_in if cand_in is not None else pb.cand_in
        for t in range(pb.num_tokens):
            row = top[t][top[t] >= 0]
            if len(row):
                assert np.all(np.isin(row // 8, cand[t, 0])), f"token {t} outside candidates"
    if pb.mode == 2:
        c = res["cand"]
        cv = c >= 0
        nb = -(-vis // 8)
        assert np.all(cv[:, 1:] <= cv[:, :-1])
        assert np.all((np.diff(c, axis=1) > 0) | ~cv[:, 1:])
        assert np.array_equal(cv.sum(1), np.minimum(pb.cand_blocks, nb))
        last = np.where(cv.any(1), c.max(1), -1)
        assert np.array_equal(last, nb - 1), "last visible block missing"


def compare(pb, gpu, orc, tokens=None, scores=True):
    """GPU outputs of the listed tokens (rows of ``orc``) equal the oracle's,
    bit for bit (indices, candidate ids and, when present, FP32 scores)."""
    rows = np.arange(pb.num_tokens) if tokens is None else np.asarray(tokens)
    g_top = gpu["topk"][rows]
    bad = np.flatnonzero(~np.all(g_top == orc["topk"], axis=1))
    assert len(bad) == 0, f"{pb.name}: topk differs at tokens {rows[bad][:10]}"
    if pb.mode == 2:
        g_c = gpu["cand"][rows]
        bad = np.flatnonzero(~np.all(g_c == orc["cand"], axis=1))
        assert len(bad) == 0, f"{pb.name}: candidates differ at tokens {rows[bad][:10]}"
    if scores and gpu.get("scores") is not None and orc.get("scores") is not None:
        g = gpu["scores"][rows][:, : orc["scores"].shape[1]]
        o = orc["scores"]
        same = (g == o) | (np.isnan(g) & np.isnan(o))
        if not np.all(same):
            t, j = np.argwhere(~same)[0]
            raise AssertionError(f"{pb.name}: score differs at token {rows[t]} pos {j}: "
                                 f"gpu {g[t, j]!r} oracle {o[t, j]!r}")


def oracle_rows(pb, tokens=None, scores=False, cand_in=None):
    return oracle.OracleProblem(pb, cand_in=cand_in).run(
        tokens=tokens, want_scores=scores, score_cols=max(pb.max_k_len, 1))


def sample_tokens(pb, n, seed=0, include=()):
    rng = np.random.default_rng(seed)
    T = pb.num_tokens
    pick = set(int(x) for x in include if 0 <= x < T)
    pick |= {0, T - 1}
    if T > len(pick):
        pick |= set(int(x) for x in rng.choice(T, size=min(n, T), replace=False))
    return np.array(sorted(pick), np.int32)


def small_problem(seed, ratio=2, N=32, mode=2, topk=16, cb=64, cb_in=64,
                  requests=((4, 300), (1, 77), (3, 3), (2, 2048)), cand_policy="random"):
    req = W.Requests(n=np.array([r[0] for r in requests]), S=np.array([r[1] for r in requests]))
    return W.build_problem(f"case{seed}_r{ratio}_n{N}_m{mode}", seed, req, ratio, N, mode, topk,
                           cand_blocks=cb, cand_in_blocks=cb_in, cand_policy=cand_policy)
