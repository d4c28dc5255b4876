"""Pins of the sparse-attention oracle (qli_attn_oracle.c) to results fixed
by the mathematics, not by the oracle itself:

  - one entry and no sink: the output is that entry's row, exactly, and the
    log-sum-exp is its logit;
  - every position of a request selected: a dense softmax attention,
    recomputed with numpy matrix products over the rows gathered in Python;
  - the window stage alone, and both stages together: the same dense
    computation over the position sets written out by brute force;
  - a sink equal to the only logit (scale 1, a one-hot query, so the logit
    is a BF16 value held exactly by the FP32 sink): output half the row,
    log-sum-exp the logit plus log 2;
  - shuffled index rows with padding and out-of-contract entries inserted:
    the same output.

Each pin returns a list of failure strings; run_all() collects them.  The
mutation tests load a planted-mistake build of the oracle through the
QLI_ORACLE_LIB environment variable and expect run_all() to fail.
"""
from __future__ import annotations

import numpy as np

import oracle
from qli_workloads import attn as A
from qli_workloads import bf16_to_f32


def _rows(ap, b, which, positions):
    """float64 [n, D] rows of request b at the given positions (gathered
    here, independently of the oracle's addressing)."""
    D = ap.head_dim
    if which == "c":
        pages, bt, R = ap.c_pages, ap.c_bt, ap.c_page_rows
    else:
        pages, bt, R = ap.r_pages, ap.r_bt, ap.r_page_rows
    out = np.zeros((len(positions), D))
    for i, p in enumerate(positions):
        page = int(bt[b, p // R])
        raw = pages[page].view(np.uint16)[(p % R) * D:(p % R + 1) * D]
        out[i] = bf16_to_f32(raw).astype(np.float64)
    return out


def _dense(q, K, scale, sink=None):
    """softmax(scale q K^T (+ sink column)) K for one query row q [D]."""
    z = scale * (K @ q)
    m = z.max() if len(z) else -np.inf
    if sink is not None:
        m = max(m, sink)
    w = np.exp(z - m)
    den = w.sum() + (np.exp(sink - m) if sink is not None else 0.0)
    return (w @ K) / den, m + np.log(den)


def _qrow(ap, t, h):
    return bf16_to_f32(ap.q[t, h]).astype(np.float64)


def pin_single_entry():
    fails = []
    ap = A.build_attn_problem("pin1", 101, [2], [40], [80], 2, 64, 6, 0, sinks=False)
    idx = np.full((2, 6), -1, np.int32)
    idx[0, 3] = 17
    idx[1, 0] = 39
    out, lse = oracle.sparse_attn(ap, indices=idx)
    for t, p in ((0, 17), (1, 39)):
        row = _rows(ap, 0, "c", [p])[0]
        for h in (0, 31, 63):
            if not np.array_equal(out[t, h], row):
                fails.append(f"single entry: token {t} head {h} output is not the row")
            z = ap.scale * float(_qrow(ap, t, h) @ row)
            if abs(lse[t, h] - z) > 1e-12 * max(1.0, abs(z)):
                fails.append(f"single entry: lse {lse[t, h]} != logit {z}")
    return fails


def pin_dense():
    fails = []
    L = 50
    ap = A.build_attn_problem("pin2", 102, [1, 2], [L, 33], [L * 2, 70], 2, 64, L, 0, sinks=False, fill_all=True)
    idx = np.full((3, L), -1, np.int32)
    idx[0, :L] = np.arange(L)
    idx[1, :33] = np.arange(33)
    idx[2, :33] = np.arange(33)[::-1]
    out, lse = oracle.sparse_attn(ap, indices=idx)
    for t, b, n in ((0, 0, L), (1, 1, 33), (2, 1, 33)):
        K = _rows(ap, b, "c", list(range(n)))
        for h in range(0, 64, 9):
            ref, rl = _dense(_qrow(ap, t, h), K, ap.scale)
            if np.max(np.abs(out[t, h] - ref)) > 1e-12 * max(1.0, np.max(np.abs(ref))):
                fails.append(f"dense: token {t} head {h} differs by {np.max(np.abs(out[t, h] - ref))}")
            if abs(lse[t, h] - rl) > 1e-12 * max(1.0, abs(rl)):
                fails.append(f"dense: token {t} head {h} lse {lse[t, h]} != {rl}")
    return fails


def pin_window_and_union():
    fails = []
    W = 7
    # request 0: 3 tokens, raw length 20 (positions 17, 18, 19); request 1: one
    # token at raw position 4 (the window is cut at 0)
    ap = A.build_attn_problem("pin3", 103, [3, 1], [9, 2], [20, 5], 2, 64, 5, W, sinks=True, fill_all=True)
    idx = np.full((4, 5), -1, np.int32)
    idx[1, :3] = [2, 5, 8]
    idx[3, :2] = [0, 1]
    out, lse = oracle.sparse_attn(ap, indices=idx)
    cases = [(0, 0, 17, []), (1, 0, 18, [2, 5, 8]), (2, 0, 19, []), (3, 1, 4, [0, 1])]
    for t, b, p, csa in cases:
        win = [s for s in range(p - W + 1, p + 1) if s >= 0]
        K = np.concatenate([_rows(ap, b, "c", csa), _rows(ap, b, "r", win)]) if csa else _rows(ap, b, "r", win)
        for h in (0, 13, 63):
            ref, rl = _dense(_qrow(ap, t, h), K, ap.scale, float(ap.sinks[h]))
            if np.max(np.abs(out[t, h] - ref)) > 1e-12 * max(1.0, np.max(np.abs(ref))):
                fails.append(f"window: token {t} head {h} differs by {np.max(np.abs(out[t, h] - ref))}")
            if abs(lse[t, h] - rl) > 1e-12 * max(1.0, abs(rl)):
                fails.append(f"window: token {t} head {h} lse {lse[t, h]} != {rl}")
    return fails


def pin_sink_half():
    fails = []
    ap = A.build_attn_problem("pin4", 104, [1], [12], [24], 2, 64, 4, 0, sinks=True, fill_all=True)
    ap.scale = 1.0
    ap.q[:] = 0
    d0 = 5
    ap.q[0, :, d0] = np.uint16(0x3F80)  # one-hot 1.0: the logit is k[d0]
    idx = np.array([[-1, 7, -1, -1]], np.int32)
    row = _rows(ap, 0, "c", [7])[0]
    ap.sinks = np.full(64, np.float32(row[d0]), np.float32)
    out, lse = oracle.sparse_attn(ap, indices=idx)
    for h in (0, 40, 63):
        if np.max(np.abs(out[0, h] - row / 2)) > 1e-15 * max(1.0, np.max(np.abs(row))):
            fails.append(f"sink: head {h} output is not half the row")
        if abs(lse[0, h] - (row[d0] + np.log(2.0))) > 1e-12:
            fails.append(f"sink: head {h} lse {lse[0, h]} != {row[d0] + np.log(2.0)}")
    return fails


def pin_order_padding():
    fails = []
    ap = A.build_attn_problem("pin5", 105, [4], [300], [600], 2, 64, 40, 16, sinks=True)
    base_out, base_lse = oracle.sparse_attn(ap)
    rng = np.random.default_rng(5)
    idx = np.full((4, 64), -1, np.int32)
    for t in range(4):
        row = ap.indices[t]
        row = row[row >= 0]
        junk = np.array([-1, -7, 300, 10 ** 6], np.int32)[: rng.integers(1, 5)]
        mixed = np.concatenate([row, junk])
        rng.shuffle(mixed)
        idx[t, : len(mixed)] = mixed
    out, lse = oracle.sparse_attn(ap, indices=idx)
    d = np.max(np.abs(out - base_out))
    if d > 1e-12:
        fails.append(f"order/padding: outputs differ by {d}")
    if np.max(np.abs(lse - base_lse)) > 1e-12:
        fails.append("order/padding: lse differs")
    return fails


PINS = [pin_single_entry, pin_dense, pin_window_and_union, pin_sink_half, pin_order_padding]


def run_all():
    fails = []
    for p in PINS:
        try:
            fails += p()
        except Exception as e:  # a broken oracle may fail loudly instead
            fails.append(f"{p.__name__} raised {type(e).__name__}: {e}")
    return fails
