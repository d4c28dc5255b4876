"""GPU parity of the sparse-attention consumer of the indexer's positions
(qli_sparse_attention) against the oracle (qli_attn_oracle.c), through the
C ABI.  Heads in multiples of 64 run the split kernel (a token's entries
over up to four workgroups whose states a merge launch combines from the
workspace, or one workgroup per token without a workspace); other head
counts run the head-group kernel.

Tolerance, from the kernel's arithmetic: the logits are exact products
summed in FP32 (relative error far below 1e-5 of the logit range); the
weights of the value sum are rounded to BF16 (relative 2^-9 each) and the
normalizer sums the same rounded weights, so the output is a convex
combination whose weights differ from the exact ones by at most about
2^-8 relative: |out - exact| <= 2^-8 * max_j |v_j|; the BF16 output adds
2^-9 |out|; FP32 sums over a few thousand terms add less than 2^-12
max |v|.  The test allows |out - oracle| <= 2^-7 max_j |v_j| + 2^-8 |oracle|
per token, and 4e-3 on the log-sum-exp."""
import dataclasses

import numpy as np
import pytest

import oracle
from gpu_check import say
from qli_workloads import attn as A
from qli_workloads import bf16_to_f32

pytestmark = pytest.mark.gpu

QLI_DEV_BAD_PAGE, QLI_DEV_BAD_LENGTH, QLI_DEV_BAD_METADATA, QLI_DEV_BAD_INDEX = 1, 2, 4, 8


def run_attn(ap, indices=None, lse=True, status=False, workspace="auto"):
    import torch

    import quantized_top_indexer_amd as Q
    idx = ap.indices if indices is None else indices

    def dev(a, dt=None):
        a = np.ascontiguousarray(a if dt is None else a.astype(dt))
        return torch.from_numpy(a).cuda()

    q = dev(ap.q.view(np.int16)).view(torch.bfloat16)
    c_cache = dev(ap.c_pages)
    r_cache = dev(ap.r_pages)
    st = torch.zeros(1, dtype=torch.int32, device="cuda") if status else None
    lse_t = torch.full((ap.num_tokens, ap.num_heads), 7.0, dtype=torch.float32, device="cuda") if lse else None
    out, _ = Q.sparse_attention(
        q, c_cache, dev(ap.c_bt, np.int32), dev(ap.c_lens, np.int32), dev(ap.query_start_loc, np.int32),
        indices=dev(idx, np.int32) if idx.shape[1] > 0 else None,
        r_cache=r_cache if ap.window > 0 else None,
        r_block_table=dev(ap.r_bt, np.int32) if ap.window > 0 else None,
        r_lens=dev(ap.r_lens, np.int32) if ap.window > 0 else None,
        window=ap.window, sinks=None if ap.sinks is None else dev(ap.sinks, np.float32), scale=ap.scale,
        c_page_rows=ap.c_page_rows, c_page_stride=ap.c_page_stride, c_num_pages=ap.c_pages.shape[0],
        r_page_rows=ap.r_page_rows, r_page_stride=ap.r_page_stride, r_num_pages=ap.r_pages.shape[0],
        lse=lse_t, status_out=st, workspace=workspace)
    torch.cuda.synchronize()
    o = bf16_to_f32(out.view(torch.int16).cpu().numpy().view(np.uint16)).astype(np.float64)
    return o, (lse_t.cpu().numpy() if lse else None), (int(st.item()) if status else None)


def value_bound(ap, t, idx):
    """max |v| over the entries token t reads (gathered on the host)."""
    qsl = ap.query_start_loc
    b = int(np.searchsorted(qsl, t, side="right") - 1)
    vals = []
    for c in idx[t]:
        if 0 <= c < ap.c_lens[b]:
            page = ap.c_bt[b, c // ap.c_page_rows]
            vals.append(np.abs(bf16_to_f32(ap.c_pages[page].view(np.uint16)[
                (c % ap.c_page_rows) * 512:(c % ap.c_page_rows + 1) * 512])).max())
    if ap.window > 0:
        p = int(ap.r_lens[b]) - (qsl[b + 1] - qsl[b]) + (t - qsl[b])
        for s in range(max(0, p - ap.window + 1), p + 1):
            page = ap.r_bt[b, s // ap.r_page_rows]
            vals.append(np.abs(bf16_to_f32(ap.r_pages[page].view(np.uint16)[
                (s % ap.r_page_rows) * 512:(s % ap.r_page_rows + 1) * 512])).max())
    return max(vals) if vals else 0.0


def check(ap, indices=None, tokens=None, workspace="auto"):
    idx = ap.indices if indices is None else indices
    say(f"attn {ap.name}: T={ap.num_tokens} H={ap.num_heads} topk={idx.shape[1]} window={ap.window} "
        f"sinks={ap.sinks is not None} workspace={'auto' if isinstance(workspace, str) else workspace is not None}")
    o, lse, _ = run_attn(ap, indices=idx, workspace=workspace)
    tok = np.arange(ap.num_tokens) if tokens is None else np.asarray(tokens)
    ref, rlse = oracle.sparse_attn(ap, tokens=tok, indices=idx)
    worst = 0.0
    for i, t in enumerate(tok):
        vb = value_bound(ap, int(t), idx)
        err = np.abs(o[t] - ref[i])
        lim = 2.0 ** -7 * vb + 2.0 ** -8 * np.abs(ref[i])
        assert np.all(err <= lim), f"{ap.name} token {t}: max excess {np.max(err - lim)} (bound {vb})"
        # the bound above is loose for outputs averaged over many entries; the
        # rounding errors are independent, so the whole token's output is
        # also held to 2^-8 of its norm (a wrong weight or row fails it)
        nrm = np.linalg.norm(ref[i])
        if nrm > 0:
            rel = np.linalg.norm(o[t] - ref[i]) / nrm
            worst = max(worst, rel)
            assert rel <= 2.0 ** -8, f"{ap.name} token {t}: relative error {rel}"
        fin = np.isfinite(rlse[i])
        assert np.array_equal(fin, np.isfinite(lse[t])), f"{ap.name} token {t}: lse finiteness"
        assert np.all(np.abs(lse[t][fin] - rlse[i][fin]) <= 4e-3), f"{ap.name} token {t}: lse"
        assert np.all(lse[t][~fin] == -np.inf)
    say(f"  worst relative error {worst:.2e}")
    return o, lse


def test_small_mixed():
    check(A.attn_small())


def test_no_sinks_no_window():
    ap = A.build_attn_problem("nosink", 21, [2, 3], [300, 77], [600, 154], 2, 64, 128, 0, sinks=False,
                              pad_frac=0.5)
    check(ap)


def test_window_only_and_128_heads():
    ap = A.build_attn_problem("window_only", 22, [4, 1], [50, 10], [100, 3], 1, 128, 0, 64)
    check(ap, indices=np.zeros((5, 0), np.int32))


def test_ragged_tiles_and_empty_rows():
    # rows of 1, 15, 16, 17, 31, 33 entries and an all-padding row (no window):
    # partial tiles, one pair with nothing to score, sinks only
    idx = np.full((7, 40), -1, np.int32)
    rng = np.random.default_rng(3)
    for t, n in enumerate([1, 15, 16, 17, 31, 33, 0]):
        idx[t, :n] = np.sort(rng.choice(400, n, replace=False))
    ap = A.build_attn_problem("ragged", 23, [7], [400], [800], 2, 64, 40, 0, sinks=True, indices=idx)
    check(ap)
    ap2 = dataclasses.replace(ap, sinks=None)
    o, lse = check(ap2)
    assert np.all(o[6] == 0) and np.all(lse[6] == -np.inf)


def test_full_decode_shape_sampled():
    ap = A.attn_decode()
    check(ap, tokens=[0, 17, 40, 63])


def test_out_of_contract_entries_flagged_and_skipped():
    ap = A.build_attn_problem("bad", 24, [2, 1], [90, 30], [180, 60], 2, 64, 32, 8)
    idx = ap.indices.copy()
    idx[0, 3] = 90          # at the compressed length
    idx[2, 0] = 10 ** 6     # far beyond
    o, lse, st = run_attn(ap, indices=idx, status=True)
    assert st & QLI_DEV_BAD_INDEX
    ref, rlse = oracle.sparse_attn(ap, indices=idx)
    keep = idx.copy()
    keep[0, 3] = -1
    keep[2, 0] = -1
    ref2, _ = oracle.sparse_attn(ap, indices=keep)
    assert np.max(np.abs(ref - ref2)) == 0.0
    check(ap, indices=keep)
    # a block-table entry past the pool: that entry is dropped and flagged
    bt = ap.c_bt.copy()
    page_of = idx[1, 0] // ap.c_page_rows
    bt[0, page_of] = ap.c_pages.shape[0] + 5
    ap3 = dataclasses.replace(ap, c_bt=bt)
    _, _, st3 = run_attn(ap3, indices=keep, status=True)
    assert st3 & QLI_DEV_BAD_PAGE


def test_head_group_kernel_32_and_48_heads():
    # heads not a multiple of 64: the head-group kernel
    check(A.build_attn_problem("heads32", 25, [3, 2], [200, 90], [400, 180], 2, 32, 64, 24, pad_frac=0.3))
    check(A.build_attn_problem("heads48", 26, [2, 1], [300, 50], [600, 100], 1, 48, 96, 40))


def test_split_kernel_without_workspace():
    # one workgroup per (token, 64 heads): no partial states
    check(A.attn_small(), workspace=None)
    ap = A.build_attn_problem("ragged_nows", 27, [7], [400], [800], 2, 128, 40, 8, pad_frac=0.5)
    check(ap, workspace=None)


def test_split_kernel_many_tokens():
    # 260 tokens x 64 heads fill the GPU without splitting; a ragged last
    # group of 8 tokens
    ap = A.build_attn_problem("many", 28, [100, 1, 159], [500, 20, 300], [1000, 40, 600], 2, 64, 32, 16,
                              pad_frac=0.2)
    check(ap)


def test_split_workspace_reused_without_initialisation():
    # three calls in a row on one workspace filled with garbage first (the
    # last call smaller, with fewer splits): each equals the oracle
    import ctypes

    import torch

    import quantized_top_indexer_amd as Q
    calls = [A.attn_small(),
             A.build_attn_problem("ws2", 29, [5, 4], [900, 700], [1800, 1400], 1, 128, 256, 64),
             A.build_attn_problem("ws3", 30, [2], [60], [120], 2, 64, 40, 8)]
    need = []
    for ap in calls:
        p = Q.qli_attn_params()
        p.num_tokens, p.num_heads, p.topk, p.window = ap.num_tokens, ap.num_heads, ap.indices.shape[1], ap.window
        need.append(Q.load_library().qli_attn_workspace_bytes(ctypes.byref(p)))
    assert min(need) > 0
    ws = torch.full((max(need),), 0xFF, dtype=torch.uint8, device="cuda")  # NaN bit patterns
    for ap in calls:
        check(ap, workspace=ws)


def test_maximum_entries_and_heads():
    # topk 2048 and a 512-position window: 2560 entries per token, the most a
    # workgroup's entry list holds; 128 heads (two head blocks); sampled tokens
    B = 3
    ap = A.build_attn_problem("max_entries", 31, [1, 2, 1], [4096, 3000, 2100], [9000, 600, 513], 1, 128,
                              2048, 512)
    assert ap.num_tokens == 4 and B == len(ap.c_lens)
    check(ap, tokens=[0, 1, 2, 3])
    # the same entries through the head-group kernel (48 heads)
    ap48 = A.build_attn_problem("max_entries48", 33, [1, 2, 1], [4096, 3000, 2100], [9000, 600, 513], 1, 48,
                                2048, 512)
    check(ap48, tokens=[0, 2, 3])


def test_three_splits():
    # 100 tokens x 64 heads: three workgroups per token (72 entries: three
    # 32-entry steps, one per split)
    import ctypes

    import quantized_top_indexer_amd as Q
    ap = A.build_attn_problem("three_splits", 32, [60, 40], [500, 90], [1000, 180], 2, 64, 64, 8, pad_frac=0.2)
    p = Q.qli_attn_params()
    p.num_tokens, p.num_heads, p.topk, p.window = ap.num_tokens, ap.num_heads, 64, 8
    assert Q.load_library().qli_attn_workspace_bytes(ctypes.byref(p)) == 100 * 3 * 64 * (2 + 512) * 4
    check(ap)


def test_prefill_shape_without_split_sampled():
    # 300 query tokens of one request (enough to fill the GPU without a
    # split: one workgroup per token) with full 2048-position rows and a
    # 128-position window; sampled tokens against the oracle
    ap = A.build_attn_problem("prefill_like", 34, [300], [4096], [8192], 2, 64, 2048, 128)
    check(ap, tokens=[0, 1, 149, 150, 298, 299])
