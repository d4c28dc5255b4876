"""GPU parity at sizes the oracle finishes in seconds: every output of every
token compared with the oracle, bit for bit (indices, candidate ids, FP32
scores), across ratios, head counts, modes, several 256-slot tiles and
ragged tails, plus the edge cases of the method."""
import numpy as np
import pytest

from gpu_check import (check_invariants, compare, oracle_rows, run_gpu, sample_tokens, say,
                       small_problem, visible)

pytestmark = pytest.mark.gpu

MEDIUM = [
    # (ratio, heads, mode, topk, cb, requests)
    (2, 32, 2, 16, 64, ((4, 256),)),                                   # the tiny shape
    (1, 64, 2, 100, 64, ((3, 1500), (1, 777), (2, 130))),
    (2, 64, 2, 300, 128, ((5, 4001), (1, 999))),
    (1, 32, 1, 7, 64, ((6, 2500), (1, 1), (2, 65))),
    (2, 32, 1, 2048, 64, ((2, 3000), (1, 513))),
    (1, 64, 3, 64, 64, ((3, 3333), (2, 700))),
    (2, 32, 3, 500, 128, ((4, 5000), (1, 20))),
    (1, 32, 2, 2048, 2048, ((2, 2600),)),
    # rows of 4097..10240 and 10241..16384 keys: the two 512-thread
    # selections (20 and 32 keys per thread)
    (1, 32, 2, 2048, 512, ((3, 9000), (1, 5000))),
    (1, 64, 1, 1500, 64, ((2, 12000), (1, 10300))),
    # 32 heads: several groups of four tokens per request, plus leftover tokens
    (2, 32, 2, 300, 128, ((19, 4000), (8, 900), (3, 300))),
    (1, 32, 1, 1000, 64, ((16, 2600), (11, 1300), (1, 40))),
]


@pytest.mark.parametrize("case", range(len(MEDIUM)))
def test_medium_all_tokens(case):
    ratio, N, mode, topk, cb, req = MEDIUM[case]
    pb = small_problem(100 + case, ratio=ratio, N=N, mode=mode, topk=topk, cb=cb, cb_in=cb,
                       requests=req)
    say(f"case {pb.name}: T={pb.num_tokens} L={pb.max_k_len}")
    gpu = run_gpu(pb, debug=True)
    orc = oracle_rows(pb, scores=True)
    compare(pb, gpu, orc)
    check_invariants(pb, gpu)
    # the production launch (no debug scores) gives the same outputs
    prod = run_gpu(pb, debug=False)
    assert np.array_equal(prod["topk"], gpu["topk"])
    if mode == 2:
        assert np.array_equal(prod["cand"], gpu["cand"])


def test_tiny_workload():
    import qli_workloads as W
    pb = W.tiny()
    gpu = run_gpu(pb, debug=True)
    orc = oracle_rows(pb, scores=True)
    compare(pb, gpu, orc)
    check_invariants(pb, gpu)
    assert np.all(gpu["cand"][:, 16:] == -1) and np.all(gpu["cand"][:, :16] == np.arange(16))


EDGES = {
    # empty compressed contexts at ratio 2 (raw length 1), a request whose
    # queries cover its whole raw length (first query sees nothing), a
    # request with no queries, lengths off every tile boundary
    "empty_and_ragged": dict(ratio=2, N=32, mode=2, topk=33, cb=64,
                             requests=((1, 1), (3, 3), (0, 500), (2, 17), (1, 1), (4, 1027))),
    "ratio1_single_positions": dict(ratio=1, N=64, mode=2, topk=5, cb=64,
                                    requests=((1, 1), (2, 2), (1, 9), (1, 257))),
    "topk_exceeds_eligible": dict(ratio=2, N=32, mode=1, topk=2048, cb=64,
                                  requests=((3, 600), (1, 4095))),
    "cand_exceeds_blocks": dict(ratio=1, N=32, mode=2, topk=64, cb=2048,
                                requests=((2, 1000), (1, 8), (1, 9))),
    "topk_one": dict(ratio=2, N=64, mode=2, topk=1, cb=64, requests=((3, 2000),)),
    "consumer_messy": dict(ratio=2, N=32, mode=3, topk=100, cb_in=128,
                           requests=((3, 3000), (1, 1), (2, 15), (1, 4096)),
                           cand_policy="messy"),
    "consumer_ratio1_full": dict(ratio=1, N=64, mode=3, topk=2048, cb_in=64,
                                 requests=((2, 600), (1, 1))),
    # rows longer than one select chunk (32768 keys): the chunked selection
    "long_rows_chunked": dict(ratio=1, N=32, mode=2, topk=2048, cb=1024,
                              requests=((2, 45000), (1, 33000))),
}


@pytest.mark.parametrize("name", sorted(EDGES))
def test_edges(name):
    pb = small_problem(200 + sorted(EDGES).index(name), **EDGES[name])
    say(f"edge {name}: T={pb.num_tokens} L={pb.max_k_len}")
    gpu = run_gpu(pb, debug=True)
    orc = oracle_rows(pb, scores=True)
    compare(pb, gpu, orc)
    check_invariants(pb, gpu)


@pytest.mark.parametrize("mode,patterns", [(1, 3), (2, 3), (3, 3), (1, 200), (2, 200), (3, 200)])
def test_heavy_ties(mode, patterns):
    """K rows drawn from a few patterns with one scale: each token sees at
    most that many distinct scores, so the selection is decided by position
    among equal keys (score desc, position asc).  With 3 patterns whole
    histogram bins are ties; with 200 each value repeats ~15 times, so the
    boundary falls inside a small run of equal keys."""
    pb = small_problem(310 + mode, ratio=1, N=32, mode=mode, topk=300, cb=64, cb_in=128,
                       requests=((2, 3000), (1, 1200), (1, 40), (1, 36000) if mode != 3 else (1, 60)))
    rng = np.random.default_rng(310 + mode + patterns)
    pats = rng.integers(-128, 128, size=(patterns, 128), dtype=np.int64).astype(np.int8)
    P, R, _ = pb.k_pages.shape
    pb.k_pages = pats[rng.integers(0, patterns, size=P * R)].reshape(P, R, 128).copy()
    pb.s_pages = np.full((P, R), 0x3C00, dtype=np.uint16)
    gpu = run_gpu(pb, debug=True)
    orc = oracle_rows(pb, scores=True)
    compare(pb, gpu, orc)
    check_invariants(pb, gpu)


# Rows of 24576..32768 eligible keys in batches of at most 4 rows per CU: the
# single-chunk 1024-thread selection, which first brackets the threshold from
# a sample of the keys, gathers the keys inside the bracket (at most 4096) and
# refines among them alone; when the bracket misses the threshold or holds
# more keys it falls back to refining over the whole row.
SEL_BRACKET_REQ = ((4, 32768), (2, 30001), (1, 24577), (1, 28000))
SEL_GATHER_CAP = 4096   # keys the bracket may gather (an eighth of the chunk)


@pytest.mark.parametrize("mode,patterns", [(1, 0), (2, 0), (1, 3), (2, 3), (1, 200), (2, 200)])
def test_sampled_bracket_selection(mode, patterns):
    """Every token's row in the sampled-bracket range, every output compared
    with the oracle.  patterns = 0: random K (no ties, the bracket holds);
    3: K rows from three patterns with one scale, so a token sees at most
    three distinct scores and the value at the k-th rank repeats more than
    4096 times: any bracket that contains the threshold holds more keys than
    it may gather, so the fallback over the whole row runs (asserted below
    on the oracle's scores); 200: about 160 copies of each value, so the
    boundary falls inside a run of equal keys within the bracket."""
    pb = small_problem(360 + mode + patterns, ratio=1, N=32, mode=mode, topk=2048, cb=512,
                       requests=SEL_BRACKET_REQ)
    vis = visible(pb)
    assert vis.min() >= 24576 and pb.max_k_len <= 32768 and 2 * pb.num_tokens <= 4 * 256
    if patterns:
        rng = np.random.default_rng(361 + patterns)
        pats = rng.integers(-128, 128, size=(patterns, 128), dtype=np.int64).astype(np.int8)
        P, R, _ = pb.k_pages.shape
        pb.k_pages = pats[rng.integers(0, patterns, size=P * R)].reshape(P, R, 128).copy()
        pb.s_pages = np.full((P, R), 0x3C00, dtype=np.uint16)
    say(f"sampled bracket {pb.name} patterns={patterns}: T={pb.num_tokens} L={pb.max_k_len}")
    gpu = run_gpu(pb, debug=True)
    orc = oracle_rows(pb, scores=True)
    compare(pb, gpu, orc)
    check_invariants(pb, gpu)
    if patterns == 3:
        for t in range(pb.num_tokens):
            row = orc["scores"][t, : vis[t]].astype(np.float64)
            kth = np.sort(row)[::-1][pb.topk - 1]
            assert np.count_nonzero(row == kth) > SEL_GATHER_CAP, t


# More than four rows per CU with rows longer than 10240 keys: one selection
# launch per length class, rows above 16384 keys in the chunked 512-thread
# selection (a sample read of the row bounds a bracket, one sweep gathers it,
# the search runs on the gathered keys, or on the whole row when the bracket
# misses or overflows).  Lengths from 600 to 60000 keys.
CLASS_REQ = ((120, 60000), (120, 40000), (120, 24000), (120, 17000), (120, 12000), (60, 9000),
             (40, 3000), (20, 600))


def best_by_score(sc, n, k):
    """Ascending indices of the best min(k, n) of sc[:n] by (value desc, index asc)."""
    order = np.lexsort((np.arange(n), -sc[:n].astype(np.float64)))
    return np.sort(order[: min(k, n)])


@pytest.mark.parametrize("patterns", [0, 3, 200])
def test_length_class_selection(patterns):
    """Every token's positions and candidate blocks equal the exact best ones
    by the GPU's own scores (the order the selection must reproduce, at any
    size), and the scores equal the oracle's at sampled positions of sampled
    tokens.  patterns = 3 and 200: K rows from that many patterns with one
    scale (runs of thousands, or hundreds, of equal scores around the k-th
    rank, so the chunked bracket overflows its gather or holds the boundary
    inside a run of ties)."""
    import oracle
    pb = small_problem(380 + patterns, ratio=1, N=32, mode=2, topk=1500, cb=1024, requests=CLASS_REQ)
    vis = visible(pb)
    assert 2 * pb.num_tokens > 4 * 256 and vis.max() > 32768
    if patterns:
        rng = np.random.default_rng(381 + patterns)
        pats = rng.integers(-128, 128, size=(patterns, 128), dtype=np.int64).astype(np.int8)
        P, R, _ = pb.k_pages.shape
        pb.k_pages = pats[rng.integers(0, patterns, size=P * R)].reshape(P, R, 128).copy()
        pb.s_pages = np.full((P, R), 0x3C00, dtype=np.uint16)
    say(f"length classes {pb.name} patterns={patterns}: T={pb.num_tokens} L={pb.max_k_len}")
    gpu = run_gpu(pb, debug=True)
    check_invariants(pb, gpu)
    sc = gpu["scores"]
    for t in range(pb.num_tokens):
        V = int(vis[t])
        assert not np.any(np.isnan(sc[t, :V])), t
        want = best_by_score(sc[t], V, pb.topk)
        got = gpu["topk"][t]
        assert np.array_equal(got[: len(want)], want) and np.all(got[len(want):] == -1), t
        nb = -(-V // 8)
        bm = np.full(nb * 8, -np.inf)
        bm[:V] = sc[t, :V]
        bm = bm.reshape(nb, 8).max(axis=1)
        if nb <= pb.cand_blocks:
            cw = np.arange(nb)
        else:
            cw = np.sort(np.append(best_by_score(bm, nb - 1, pb.cand_blocks - 1), nb - 1))
        gc = gpu["cand"][t]
        assert np.array_equal(gc[: len(cw)], cw) and np.all(gc[len(cw):] == -1), t
        if patterns == 3 and V > 16384:  # the chunked bracket cannot gather the k-th value's run
            kth = np.sort(sc[t, :V])[::-1][pb.topk - 1]
            assert np.count_nonzero(sc[t, :V] == kth) > 2048, t
    o = oracle.OracleProblem(pb)
    rng = np.random.default_rng(382)
    for t in sample_tokens(pb, 4, seed=383):
        V = int(vis[t])
        for j in np.concatenate([rng.integers(0, V, 40), [0, V - 1]]):
            assert sc[t, j] == o.terms(int(t), int(j))["score"], (t, j)


@pytest.mark.parametrize("ratio,N,mode", [(2, 64, 2), (1, 32, 1), (2, 32, 3)])
def test_head_multiplier_ranges(ratio, N, mode):
    """Head multipliers m = fp16(w * q_scale) across the ranges the score
    kernel treats differently: |m| < 32 (m * 2^11 is a finite fp16, the
    scaled epilogue), exactly 32 and -1024 (the plain epilogue for that
    token), the largest fp16 below 32, and fp16-subnormal m.  Queries are
    small so that no product overflows.  Requests of 5-9 queries make
    groups of four tokens share K tiles, so tokens of one group take
    different epilogues."""
    pb = small_problem(330 + ratio + N + mode, ratio=ratio, N=N, mode=mode, topk=150, cb=64, cb_in=128,
                       requests=((9, 3000), (5, 1100), (2, 500), (1, 64)))
    rng = np.random.default_rng(331)
    T = pb.num_tokens
    pb.q = rng.integers(-3, 4, size=pb.q.shape).astype(np.int8)
    w = pb.weights.view(np.float16).astype(np.float32).copy()
    qs = pb.q_scale.view(np.float16).astype(np.float32).copy()
    for t in range(T):
        h = (7 * t) % N
        kind = t % 5
        if kind == 1:                      # m = 32 exactly: plain epilogue
            w[t, h], qs[t, h] = 64.0, 0.5
        elif kind == 2:                    # largest fp16 below 32: scaled
            w[t, h], qs[t, h] = 31.984375, 1.0
        elif kind == 3:                    # every m an fp16 subnormal
            w[t] = np.where(rng.random(N) < 0.5, -1.0, 1.0) * 1e-3
            qs[t] = rng.uniform(1e-3, 2e-2, N)
        elif kind == 4:                    # a large negative m: plain epilogue
            w[t, h], qs[t, h] = -1024.0, 1.0
    pb.weights = w.astype(np.float16).view(np.uint16)
    pb.q_scale = qs.astype(np.float16).view(np.uint16)
    m = (pb.weights.view(np.float16).astype(np.float32) * pb.q_scale.view(np.float16).astype(np.float32))
    assert np.any(np.abs(m) >= 32) and np.any((np.abs(m) < 2 ** -14) & (m != 0))
    say(f"multipliers {pb.name}: T={T} L={pb.max_k_len}")
    gpu = run_gpu(pb, debug=True)
    orc = oracle_rows(pb, scores=True)
    compare(pb, gpu, orc)
    check_invariants(pb, gpu)


@pytest.mark.parametrize("ratio,N,mode", [(2, 64, 2), (1, 64, 1), (2, 32, 3)])
def test_extreme_products(ratio, N, mode):
    """The largest and smallest q.k that int8 operands allow: q = k = -128
    everywhere gives +2^21, q = -128 against k = 127 gives -2080768, and
    q = 127 against k = -128 the same negative value, on tokens and rows
    mixed among ordinary ones.  The score kernels carry q.k in a seeded
    FP32 accumulator, which must hold exactly over this whole range."""
    pb = small_problem(340 + ratio + N + mode, ratio=ratio, N=N, mode=mode, topk=120, cb=64, cb_in=128,
                       requests=((6, 2100), (5, 700), (1, 90)))
    rng = np.random.default_rng(341)
    T = pb.num_tokens
    q = pb.q.copy()
    q[0::3] = -128            # every head of every third token
    q[1::3, : N // 2] = 127   # half the heads of the next ones
    pb.q = q
    P, R, _ = pb.k_pages.shape
    k = pb.k_pages.reshape(P * R, 128).copy()
    pick = rng.random(P * R)
    k[pick < 0.3] = -128
    k[(pick >= 0.3) & (pick < 0.5)] = 127
    pb.k_pages = k.reshape(P, R, 128)
    say(f"extreme products {pb.name}: T={T} L={pb.max_k_len}")
    gpu = run_gpu(pb, debug=True)
    orc = oracle_rows(pb, scores=True)
    compare(pb, gpu, orc)
    check_invariants(pb, gpu)


def test_consumer_long_context_bound():
    """A context bound above 2^21 positions takes the sorting candidate
    preparation instead of the bitmap one: same outputs, same as the oracle."""
    pb = small_problem(320, ratio=2, N=32, mode=3, topk=100, cb_in=128,
                       requests=((3, 3000), (1, 1), (2, 15)), cand_policy="messy")
    base = run_gpu(pb, debug=True)
    bound = (1 << 21) + 8
    R = pb.k_pages.shape[1]
    bt = np.zeros((pb.block_table.shape[0], -(-bound // R)), np.int32)
    bt[:, :pb.block_table.shape[1]] = pb.block_table
    pb.block_table = bt
    big = run_gpu(pb, debug=True, max_k_len=bound)
    assert np.array_equal(base["topk"], big["topk"])
    L = base["scores"].shape[1]
    assert np.array_equal(base["scores"], big["scores"][:, :L], equal_nan=True)
    compare(pb, big, oracle_rows(pb, scores=True))


def test_large_consumer_batch_sorting_preparation():
    """A consumer batch of more than 1024 tokens whose context bound exceeds
    2^21 positions takes the sorting preparation (the plan in its block 0)
    instead of the lean bitmap launch: the same indices as with the tight
    bound, which test_select_length_classes checks against the oracle."""
    req = ((1030, 40000), (20, 6000), (1, 1))
    pb = small_problem(352, ratio=2, N=32, mode=3, topk=900, cb_in=2048, requests=req,
                       cand_policy="messy")
    say(f"large consumer batch: T={pb.num_tokens} L={pb.max_k_len}")
    base = run_gpu(pb)
    bound = (1 << 21) + 8
    R = pb.k_pages.shape[1]
    bt = np.zeros((pb.block_table.shape[0], -(-bound // R)), np.int32)
    bt[:, :pb.block_table.shape[1]] = pb.block_table
    pb.block_table = bt
    big = run_gpu(pb, max_k_len=bound)
    assert np.array_equal(base["topk"], big["topk"])
    check_invariants(pb, big)


def test_layout_invariance():
    """A larger page stride with K and scales moved inside the page gives
    identical outputs (the kernels only follow the strides)."""
    pb = small_problem(300, ratio=2, N=64, mode=2, topk=200, cb=64, requests=((3, 3000), (1, 50)))
    a = run_gpu(pb, debug=True)
    b = run_gpu(pb, debug=True, layout=dict(page_stride=131072 + 4096, k_offset=1024,
                                            s_offset=1024 + 64 * 128 + 256))
    assert np.array_equal(a["topk"], b["topk"]) and np.array_equal(a["cand"], b["cand"])
    assert np.array_equal(a["scores"], b["scores"], equal_nan=True)


def test_batching_invariance():
    """A TND batch of requests equals one call per request."""
    reqs = ((3, 1200), (1, 1), (2, 333), (1, 2048))
    pb = small_problem(301, ratio=2, N=32, mode=2, topk=50, cb=64, requests=reqs)
    whole = run_gpu(pb)
    for b, r in enumerate(reqs):
        one = small_problem(301, ratio=2, N=32, mode=2, topk=50, cb=64, requests=(r,))
        # same request content: copy this request's queries and pages
        q0, q1 = pb.query_start_loc[b], pb.query_start_loc[b + 1]
        one.q, one.q_scale, one.weights = pb.q[q0:q1], pb.q_scale[q0:q1], pb.weights[q0:q1]
        one.k_pages, one.s_pages = pb.k_pages, pb.s_pages
        one.block_table = pb.block_table[b:b + 1]
        res = run_gpu(one)
        assert np.array_equal(res["topk"], whole["topk"][q0:q1])
        assert np.array_equal(res["cand"], whole["cand"][q0:q1])


def test_determinism():
    pb = small_problem(302, ratio=1, N=64, mode=2, topk=256, cb=128, requests=((4, 3000),))
    a, b = run_gpu(pb, debug=True), run_gpu(pb, debug=True)
    for k in ("topk", "cand"):
        assert np.array_equal(a[k], b[k])
    assert np.array_equal(a["scores"], b["scores"], equal_nan=True)


def test_device_status_flags():
    """Out-of-contract device metadata is flagged and never dereferenced: a
    block-table entry past the pool and a k_len above max_k_len."""
    import torch

    import quantized_top_indexer_amd as Q
    pb = small_problem(303, ratio=2, N=32, mode=2, topk=40, cb=64, requests=((2, 2000), (1, 900)))
    status = torch.zeros(1, dtype=torch.int32, device="cuda")
    pb.block_table = pb.block_table.copy()
    pb.block_table[0, 3] = pb.num_pages + 1000
    res = run_gpu(pb, status=status)
    assert int(status.item()) & Q.QLI_DEV_BAD_PAGE
    row = res["topk"][:2]
    assert not np.any((row >= 3 * 64) & (row < 4 * 64))  # nothing from the bad page
    status.zero_()
    pb2 = small_problem(304, ratio=2, N=32, mode=1, topk=40, requests=((1, 2000),))
    pb2.k_lens = pb2.k_lens.copy()
    pb2.k_lens[0] = pb2.max_k_len + 5  # call still declares the old bound
    from qli_workloads.device import call_kwargs, to_device
    dev = to_device(pb2, "cuda")
    kw = call_kwargs(pb2, dev)
    kw["max_k_len"] = 1000
    idx, _, _ = Q.score_topk(**kw, status_out=status)
    torch.cuda.synchronize()
    assert int(status.item()) & Q.QLI_DEV_BAD_LENGTH
    assert torch.all(idx == -1)


@pytest.mark.parametrize("N", [32, 64])
def test_bad_page_in_four_token_groups(N):
    """A block-table entry past the pool read by 4-token groups (the prefill
    paths: with 32 heads the group kernel of its own, with 64 the two-wave
    path): the status flag is raised, the page's positions and blocks are
    excluded for every token of the request, and every token still equals
    the oracle run on the same table with that page's positions removed."""
    import torch

    import quantized_top_indexer_amd as Q
    pb = small_problem(308 + N, ratio=2, N=N, mode=2, topk=300, cb=64,
                       requests=((8, 2000), (4, 900)))
    status = torch.zeros(1, dtype=torch.int32, device="cuda")
    clean = run_gpu(pb, debug=True)
    pb.block_table = pb.block_table.copy()
    pb.block_table[0, 2] = pb.num_pages + 5          # positions 128..191 of request 0
    res = run_gpu(pb, debug=True, status=status)
    assert int(status.item()) & Q.QLI_DEV_BAD_PAGE
    sc = res["scores"]
    assert np.all(np.isnan(sc[:8, 128:192]))          # never scored
    for t in range(8):
        row = res["topk"][t]
        assert not np.any((row >= 128) & (row < 192))
        assert not np.any((res["cand"][t] >= 16) & (res["cand"][t] < 24))
        # the other positions keep their scores; the selection is the best of them
        keep = ~np.isnan(sc[t])
        assert np.array_equal(sc[t][keep], clean["scores"][t][keep])
        order = np.lexsort((np.arange(sc.shape[1])[keep], -sc[t][keep].astype(np.float64)))
        want = np.sort(np.flatnonzero(keep)[order[:300]])
        assert np.array_equal(row[row >= 0], want)
    for t in range(8, 12):                            # request 1 is untouched
        assert np.array_equal(res["topk"][t], clean["topk"][t])
        assert np.array_equal(res["cand"][t], clean["cand"][t])


def test_bad_page_when_everything_fits():
    """When top-k and the candidate width cover every visible position and
    block, the selection is everything visible; a block-table entry past the
    pool must still take its positions and blocks out (the general path)."""
    import torch

    import quantized_top_indexer_amd as Q
    pb = small_problem(306, ratio=2, N=32, mode=2, topk=2048, cb=512, requests=((3, 1200), (2, 700)))
    status = torch.zeros(1, dtype=torch.int32, device="cuda")
    clean = run_gpu(pb)
    vis = visible(pb)
    for t, V in enumerate(vis):   # everything fits: all positions / blocks in order
        assert np.array_equal(clean["topk"][t, :V], np.arange(V))
        assert np.all(clean["topk"][t, V:] == -1)
        nb = -(-int(V) // 8)
        assert np.array_equal(clean["cand"][t, :nb], np.arange(nb))
    pb.block_table = pb.block_table.copy()
    pb.block_table[0, 1] = pb.num_pages + 7          # positions 64..127 of request 0
    res = run_gpu(pb, status=status)
    assert int(status.item()) & Q.QLI_DEV_BAD_PAGE
    for t in range(3):                                # request 0's tokens
        V = int(vis[t])
        want = np.array([j for j in range(V) if not 64 <= j < 128])
        assert np.array_equal(res["topk"][t, :len(want)], want)
        assert np.all(res["topk"][t, len(want):] == -1)
        nb = -(-V // 8)
        wb = np.array([c for c in range(nb) if not 8 <= c < 16])
        assert np.array_equal(res["cand"][t, :len(wb)], wb)
    for t in range(3, 5):                             # request 1 is untouched
        assert np.array_equal(res["topk"][t], clean["topk"][t])
        assert np.array_equal(res["cand"][t], clean["cand"][t])


def _expect_fits(pb, res, vis, bad=None):
    """Everything visible is selected, in order, except the positions 64..127
    and blocks 8..15 of request `bad` (a block-table entry past the pool)."""
    q = pb.query_start_loc
    for t, V in enumerate(vis):
        V = int(V)
        b = int(np.searchsorted(q, t, side="right")) - 1
        hit = bad is not None and b == bad
        want = np.array([j for j in range(V) if not (hit and 64 <= j < 128)], np.int64)
        assert np.array_equal(res["topk"][t, :len(want)], want), (t, bad)
        assert np.all(res["topk"][t, len(want):] == -1), (t, bad)
        nb = -(-V // 8)
        wb = np.array([c for c in range(nb) if not (hit and 8 <= c < 16)], np.int64)
        assert np.array_equal(res["cand"][t, :len(wb)], wb), (t, bad)
        assert np.all(res["cand"][t, len(wb):] == -1), (t, bad)


def test_bad_page_marks_across_calls_on_one_workspace():
    """Calls sharing one workspace, with an out-of-contract page and without
    it in turn: each call's marks are its own (a clean call after a bad one
    selects everything again; a bad call after clean ones takes the page's
    positions and blocks out), whether the plan runs in its own launch or in
    the score kernel (5 tokens, and 66 tokens with groups of four)."""
    import torch

    import quantized_top_indexer_amd as Q
    from qli_workloads.device import call_kwargs, to_device
    for requests in (((3, 1200), (2, 700)), ((30, 1400), (36, 1500))):
        pb = small_problem(306, ratio=2, N=32, mode=2, topk=2048, cb=512, requests=requests)
        vis = visible(pb)
        clean_bt = pb.block_table.copy()
        ws = torch.empty(256 << 20, dtype=torch.uint8, device="cuda")
        for bad in (0, None, 1, None, 0):
            pb.block_table = clean_bt.copy()
            if bad is not None:
                pb.block_table[bad, 1] = pb.num_pages + 7   # positions 64..127
            say(f"tokens {pb.num_tokens}, bad page in request {bad}")
            dev = to_device(pb, "cuda")
            status = torch.zeros(1, dtype=torch.int32, device="cuda")
            idx, cand, _ = Q.score_topk(**call_kwargs(pb, dev), status_out=status, workspace=ws)
            torch.cuda.synchronize()
            res = {"topk": idx[:, 0].cpu().numpy(), "cand": cand[:, 0].cpu().numpy()}
            assert bool(int(status.item()) & Q.QLI_DEV_BAD_PAGE) == (bad is not None)
            _expect_fits(pb, res, vis, bad)
            del dev


@pytest.mark.parametrize("shape", ["tokens64_requests64", "tokens65", "requests65"])
def test_plan_inside_score_kernel_limits(shape):
    """Batches of at most 64 tokens and 64 requests plan inside the score
    kernel, larger ones in a launch of their own: batches just inside and
    just outside both limits equal the oracle on every token and score."""
    single = tuple((1, 300 + 37 * i) for i in range(63))
    requests = {"tokens64_requests64": single + ((1, 2700),),
                "tokens65": single + ((2, 2700),),
                "requests65": single + ((1, 2700), (0, 40))}[shape]
    pb = small_problem(331, ratio=1, N=64, mode=2, topk=128, cb=64, requests=requests)
    say(f"{shape}: {pb.num_tokens} tokens, {pb.batch} requests")
    res = run_gpu(pb, debug=True)
    orc = oracle_rows(pb, scores=True)
    compare(pb, res, orc)


def test_consumer_mostly_invalid_candidates():
    """Consumer tokens whose incoming lists are mostly -1: the plan bounds the
    work by the list width, the prepared eligible count is far smaller, and
    the items past it must load nothing and score as not eligible."""
    import qli_workloads as W
    req = W.Requests(n=np.array([2, 1, 3]), S=np.array([9000, 300, 20000]))
    pb = W.build_problem("consumer_sparse_in", 320, req, ratio=2, num_heads=64, mode=3, topk=500,
                         cand_in_blocks=512, p_invalid=0.9)
    say(f"consumer sparse: T={pb.num_tokens} valid ids per token "
        f"{[int((pb.cand_in[t, 0] >= 0).sum()) for t in range(pb.num_tokens)]}")
    gpu = run_gpu(pb, debug=True)
    orc = oracle_rows(pb, scores=True)
    compare(pb, gpu, orc)
    check_invariants(pb, gpu)


@pytest.mark.parametrize("mode,ratio,N", [(2, 2, 64), (1, 1, 32), (3, 2, 64)])
def test_debug_qk_matches_oracle(mode, ratio, N):
    """The debug output of the exact INT32 q.k (both score paths: a request
    with 8 queries forms 4-token groups, the others are single tokens) at
    sampled (token, position) pairs, every head; positions that are not
    eligible keep the caller's fill."""
    import torch

    import oracle
    import quantized_top_indexer_amd as Q
    from qli_workloads.device import call_kwargs, to_device
    pb = small_problem(330 + mode, ratio=ratio, N=N, mode=mode, topk=64, cb=64, cb_in=64,
                       requests=((8, 1500), (1, 700), (2, 300)))
    dev = to_device(pb, "cuda")
    kw = call_kwargs(pb, dev)
    L = pb.max_k_len
    fill = -(2 ** 31) + 7
    dq = torch.full((pb.num_tokens, N, L), fill, dtype=torch.int32, device="cuda")
    _, _, dbg = Q.score_topk(**kw, debug_scores=True, dbg_qk=dq)
    torch.cuda.synchronize()
    got = dq.cpu().numpy()
    scores = dbg.cpu().numpy()
    o = oracle.OracleProblem(pb)
    rng = np.random.default_rng(5)
    checked = 0
    for t in range(pb.num_tokens):
        elig = np.flatnonzero(~np.isnan(scores[t]))
        assert np.all(got[t][:, np.isnan(scores[t])] == fill)  # nothing written elsewhere
        for j in rng.choice(elig, size=min(12, len(elig)), replace=False) if len(elig) else []:
            want = o.terms(t, int(j))["qk"]
            assert np.array_equal(got[t, :, j], want), (t, j)
            checked += 1
    assert checked > 50


def test_zero_tokens():
    import torch

    import quantized_top_indexer_amd as Q
    pb = small_problem(305, ratio=1, N=32, mode=2, topk=8, requests=((0, 100),))
    from qli_workloads.device import call_kwargs, to_device
    dev = to_device(pb, "cuda")
    idx, cand, _ = Q.score_topk(**call_kwargs(pb, dev))
    torch.cuda.synchronize()
    assert idx.shape == (0, 1, 8) and cand.shape == (0, 1, 64)


@pytest.mark.parametrize("mode,policy", [(2, None), (3, "random"), (3, "messy")])
def test_select_length_classes(mode, policy):
    """More than four rows per CU and rows of widely different lengths: the
    selection runs one launch per row-length class, each taking its own
    rows.  Source: position rows in every class (up to 10240, up to 16384,
    up to 32768, longer) and short block rows; consumer: rows up to 10240
    and up to 16384 eligible slots, prepared by the lean per-token launch
    that batches of 1024 tokens and more take (messy: duplicated, negative
    and invisible incoming ids).  The first and last token of every request
    and a random sample against the oracle; invariants on every token."""
    if mode == 2:
        req = ((520, 12000), (3, 40000), (2, 20000), (3, 3000), (1, 9))
        pb = small_problem(350, ratio=1, N=32, mode=2, topk=700, cb=256, requests=req)
    else:
        req = ((1030, 40000), (20, 6000), (1, 1))
        pb = small_problem(351 if policy == "random" else 352, ratio=2, N=32, mode=3, topk=900,
                           cb_in=2048, requests=req, cand_policy=policy)
    starts = np.concatenate([[0], np.cumsum([r[0] for r in req])])
    include = np.concatenate([starts[:-1], starts[1:] - 1])
    say(f"length classes {pb.name}: T={pb.num_tokens} L={pb.max_k_len}")
    gpu = run_gpu(pb)
    check_invariants(pb, gpu)
    tok = sample_tokens(pb, 12, seed=pb.seed, include=include)
    orc = oracle_rows(pb, tokens=tok, scores=False)
    compare(pb, gpu, orc, tokens=tok, scores=False)


@pytest.mark.parametrize("mode,ratio,N,slice_tokens,shape", [(2, 2, 32, 3, "mixed"), (1, 1, 64, 5, "mixed"),
                                                             (3, 2, 32, 2, "mixed"), (2, 1, 64, 7, "mixed"),
                                                             (2, 1, 64, 7, "one_token_each"),
                                                             (1, 2, 32, 6, "one_token_each")])
def test_sliced_workspace(mode, ratio, N, slice_tokens, shape):
    """A workspace that holds a slice of only a few tokens: the call runs
    slice by slice (4-token groups cut by a slice boundary are scored as
    single tokens; with one token per request, every slice after the first
    plans for requests that start past its first token) and gives the
    oracle's outputs and scores bit for bit, the same as the unsliced call."""
    import torch

    import quantized_top_indexer_amd as Q
    from qli_workloads.device import call_kwargs, to_device
    requests = (((9, 3000), (5, 1100), (1, 1), (6, 2049), (2, 40)) if shape == "mixed"
                else tuple((1, 300 + 97 * i) for i in range(20)))
    pb = small_problem(370 + mode + ratio + N, ratio=ratio, N=N, mode=mode, topk=120, cb=64, cb_in=128,
                       requests=requests)
    say(f"sliced {pb.name}: T={pb.num_tokens} L={pb.max_k_len} slice={slice_tokens}")
    whole = run_gpu(pb, debug=True)
    dev = to_device(pb, "cuda")
    kw = call_kwargs(pb, dev)
    T = pb.num_tokens
    shp_i, shp_c = Q.output_shapes(T, pb.topk, pb.cand_blocks, pb.mode)
    topk = torch.full(shp_i, -7, dtype=torch.int32, device="cuda")
    cand = torch.full(shp_c, -7, dtype=torch.int32, device="cuda") if shp_c else None
    dbg = torch.full((T, pb.max_k_len), float("nan"), dtype=torch.float32, device="cuda")
    args = {k: v for k, v in kw.items() if k != "cand_blocks"}
    p = Q.make_params(**args, cand_blocks=pb.cand_blocks, topk_out=topk, cand_out=cand, dbg_scores=dbg)
    p.num_tokens = slice_tokens
    small = Q.qli_workspace_bytes(p)          # the layout of a slice of that many tokens
    p.num_tokens = T
    assert small < Q.qli_workspace_bytes(p)
    ws = torch.empty(small, dtype=torch.uint8, device="cuda")
    p.workspace, p.workspace_bytes = ws.data_ptr(), small
    rc = Q.qli_score_topk(p)
    assert rc == Q.QLI_OK, Q.qli_status_string(rc)
    torch.cuda.synchronize()
    got = {"topk": topk[:, 0].cpu().numpy(), "cand": None if cand is None else cand[:, 0].cpu().numpy(),
           "scores": dbg.cpu().numpy()}
    assert np.array_equal(got["topk"], whole["topk"])
    if mode == 2:
        assert np.array_equal(got["cand"], whole["cand"])
    assert np.array_equal(got["scores"], whole["scores"], equal_nan=True)
    compare(pb, got, oracle_rows(pb, scores=True))
    check_invariants(pb, got)
