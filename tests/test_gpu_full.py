"""GPU parity at the full sizes of the five named workloads, in the launch
configuration the benchmark times (no debug outputs), plus a debug run for
FP32 scores.  The oracle computes sampled tokens one by one; invariants are
checked on every token."""
import gc

import numpy as np
import pytest

import qli_workloads as W
from gpu_check import (check_invariants, compare, oracle_rows, run_gpu, sample_tokens, say,
                       visible)

pytestmark = pytest.mark.gpu


def _free():
    import torch
    gc.collect()
    torch.cuda.empty_cache()


def _full_case(pb, nsample, include=(), cand_in=None):
    say(f"{pb.name}: T={pb.num_tokens} L={pb.max_k_len} mode={pb.mode}")
    prod = run_gpu(pb, cand_in=cand_in)
    check_invariants(pb, prod, cand_in)
    dbg = run_gpu(pb, cand_in=cand_in, debug=True)
    assert np.array_equal(prod["topk"], dbg["topk"])
    if pb.mode == 2:
        assert np.array_equal(prod["cand"], dbg["cand"])
    tok = sample_tokens(pb, nsample, seed=pb.seed, include=include)
    orc = oracle_rows(pb, tokens=tok, scores=True, cand_in=cand_in)
    compare(pb, prod, orc, tokens=tok, scores=False)
    compare(pb, dbg, orc, tokens=tok, scores=True)
    _free()
    return prod, tok, orc


def test_tiny():
    pb = W.tiny()
    _full_case(pb, 4)


def test_decode_source():
    """Every one of the 64 tokens against the oracle (32768-key rows: the
    sampled-bracket selection on uniform random keys)."""
    pb = W.decode_source()
    _full_case(pb, pb.num_tokens)


def test_prefill_chunk():
    pb = W.prefill_chunk()
    # first, last and tokens around tile boundaries of the visible length
    _full_case(pb, 10, include=(1, 127, 128, 4095, 8191 - 64))


def test_decode_consumer_1m():
    _full_case(W.decode_consumer_1m(), 6)


def test_mixed_source_then_consumer():
    """Mixed batch: for each ratio a source call, then a consumer fed the
    source's candidate ids (the GPU consumer gets the GPU source output; the
    oracle consumer gets the oracle source output for the sampled tokens,
    which the source comparison has just shown to be identical)."""
    import torch
    calls = W.mixed_calls()
    for src, con in (calls[:2], calls[2:]):
        vis = visible(src)
        empty = np.flatnonzero(vis == 0)[:3]
        longest = np.argsort(vis)[-3:]
        prod, tok, orc = _full_case(src, 24, include=np.concatenate([empty, longest]))
        gpu_cand = torch.from_numpy(prod["cand"][:, None, :].copy()).to("cuda")
        con.cand_in_blocks = src.cand_blocks
        say(f"{con.name}: T={con.num_tokens} L={con.max_k_len}")
        cres = run_gpu(con, cand_in=gpu_cand)
        check_invariants(con, cres, prod["cand"][:, None, :])
        ocand = np.full((con.num_tokens, 1, src.cand_blocks), -1, np.int32)
        ocand[tok, 0] = orc["cand"]
        corc = oracle_rows(con, tokens=tok, scores=False, cand_in=ocand)
        compare(con, cres, corc, tokens=tok, scores=False)
        del gpu_cand
        _free()


def test_longest_context_source():
    """One query at the longest supported context (2^24 compressed positions,
    ratio 2): the chunked selection over 512 chunks of keys.  Scores at
    sampled positions equal the oracle's, and the returned positions and
    blocks are exactly the best ones by the GPU's own scores (properties that
    hold at any size; the oracle's full row would take minutes)."""
    import torch

    import oracle
    import quantized_top_indexer_amd as Q
    L = 1 << 24
    assert L == 16777216  # QLI_MAX_K_LEN
    req = W.Requests(n=np.array([1]), S=np.array([2 * L]))
    pb = W.build_problem("longest", 9, req, ratio=2, num_heads=32, mode=2, topk=2048,
                         cand_blocks=2048, extra_pages=0)
    say(f"longest context: L={pb.max_k_len} pages={pb.num_pages}")
    res = run_gpu(pb, debug=True)
    sc = res["scores"][0]
    assert not np.any(np.isnan(sc))
    o = oracle.OracleProblem(pb)
    rng = np.random.default_rng(9)
    for j in np.concatenate([rng.integers(0, L, 150), [0, L - 1, 32767, 32768]]):
        assert sc[j] == o.terms(0, int(j))["score"], j
    # positions: the top 2048 by (score desc, position asc), ascending
    order = np.lexsort((np.arange(L), -sc.astype(np.float64)))
    assert np.array_equal(res["topk"][0], np.sort(order[:2048]))
    # blocks: the last block pinned plus the best 2047 others by (max desc, id asc)
    bm = sc.reshape(-1, 8).max(axis=1)
    nb = L // 8
    others = np.lexsort((np.arange(nb - 1), -bm[:-1].astype(np.float64)))[:2047]
    assert np.array_equal(res["cand"][0], np.sort(np.concatenate([others, [nb - 1]])))
    del res, sc
    _free()
