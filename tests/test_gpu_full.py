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
    _full_case(W.decode_source(), 8)


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
