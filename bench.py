#!/usr/bin/env python3
"""Benchmark of the quantized lightning indexer on one MI355X.

One step = one full indexer call (every kernel of the op) on the decode
candidate-source workload: 64 requests x 1 query token, 32768 compressed
positions each (ratio 1, 128-row pages at a 147712-byte stride, shuffled
block table), 64 index heads, position top-k 2048, 512 candidate blocks.
Inputs are resident in HBM before timing starts; four copies of the paged
cache are rotated so that no step re-reads the previous step's K from the
256 MB last-level cache.

Prints one JSON line: compressed keys scored per second, the dominant
kernel against its roofline (algorithmic bytes per launch over its average
duration, measured with HIP events on the launch stream), and the oracle
timed on the host cores on a bounded sample.  Secondary workloads (the
8192-token prefill chunk against the INT8 MFMA peak, the 1M-context
consumer against HBM) are reported under "other_workloads", and the two
producers of the indexer's inputs (query quantization, index-K cache
write) at decode and prefill shapes under "producers".
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, published
INT8_PEAK_TOPS = 5000.0        # MI355X dense INT8 MFMA, published (5.0 POP/s)
BF16_PEAK_TFLOPS = 2500.0      # MI355X dense BF16 MFMA, published (2.5 PFLOP/s)
KEY_BYTES = 130                # one 128-byte index-K row + its 2-byte FP16 scale
# what roofline.achieved divides by (roofline.kernel_ms)
DURATION_SOURCE = ("duration per call of roofline.kernel (its launches in one call summed), from HIP "
                   "events the library records around each launch on the launch stream, averaged "
                   "over `steps` calls run after the timed region (same process, same inputs)")


def log(msg):
    print(msg, file=sys.stderr, flush=True)


# kernels the library's timing facility reports under one name
KERNEL_GROUPS = {"score_kernel": ("score_kernel", "score_multi_kernel"),
                 "sparse_attn_split_kernel": ("sparse_attn_split_kernel", "sparse_attn_merge_kernel")}


def recorded_traffic(workload, kernel, source="qli_kernels.hip"):
    """HBM bytes per call of `kernel` (all its launches in one call; the
    score kernel's name covers both score kernels) from the committed
    rocprofv3 counter summary (profiles/traffic.json), or None when the
    kernel source changed since the counters were taken."""
    import hashlib
    path = os.path.join(ROOT, "profiles", "traffic.json")
    src = os.path.join(ROOT, "quantized_top_indexer_amd", "csrc", source)
    if not os.path.exists(path):
        return None, None
    h = hashlib.sha256(open(src, "rb").read()).hexdigest()[:16]
    entry = json.load(open(path)).get(workload)
    if not entry or entry.get("source_hash") != h:
        return None, None
    per = entry.get("hbm_bytes_per_call") or entry.get("hbm_bytes_per_launch", {})
    names = KERNEL_GROUPS.get(kernel, (kernel,))
    hits = [v for k, v in per.items() if k.split("<")[0] in names]
    return (sum(hits), entry.get("summary")) if hits else (None, None)


def algorithmic(pb, cand_in=None):
    """Keys scored, algorithmic HBM bytes and INT8 ops of one call:
    each request's eligible K rows (+scale) once, queries/scales/weights,
    block-table entries needed, metadata, incoming candidates and outputs;
    ops = eligible (token, position) pairs x heads x 2 x 128."""
    import numpy as np
    cand = cand_in if cand_in is not None else pb.cand_in
    T, N = pb.num_tokens, pb.num_heads
    keys = 0
    rows = 0
    pages = 0
    qsl = pb.query_start_loc
    for b in range(pb.batch):
        q0, q1 = int(qsl[b]), int(qsl[b + 1])
        if q1 == q0:
            continue
        n, S = q1 - q0, int(pb.raw_lens[b])
        vis = (S - n + np.arange(n) + 1) // pb.ratio
        if pb.mode == 3:
            union = set()
            for i, t in enumerate(range(q0, q1)):
                nb = -(-int(vis[i]) // 8)
                c = np.unique(cand[t, 0])
                c = c[(c >= 0) & (c < nb)].astype(np.int64)
                e = np.minimum(8, vis[i] - 8 * c)
                keys += int(e.sum())
                union |= set(c.tolist())
            touched = sorted(union)
            rows += sum(min(8, int(vis.max()) - 8 * c) for c in touched)
            pages += len({(8 * c) // pb.page_rows for c in touched})
        else:
            keys += int(vis.sum())
            rows += int(vis.max())
            pages += -(-int(vis.max()) // pb.page_rows)
    nbytes = rows * KEY_BYTES + T * N * (128 + 2 + 2) + pages * 4 + (pb.batch * 3 + 1) * 4
    nbytes += T * pb.topk * 4
    if pb.mode == 2:
        nbytes += T * pb.cand_blocks * 4
    if pb.mode == 3:
        nbytes += T * pb.cand_in_blocks * 4
    ops = keys * N * 256
    return keys, nbytes, ops


class Runner:
    """Device inputs (several rotated copies), outputs and workspace of one
    workload, plus prepared qli_params per copy."""

    def __init__(self, pb, copies=1, cand_sets=None):
        import torch

        import quantized_top_indexer_amd as Q
        from qli_workloads.device import to_device
        self.pb = pb
        self.Q = Q
        dev0 = to_device(pb, "cuda", cand_in=cand_sets[0] if cand_sets else None)
        self.devs = [dev0]
        for c in range(1, copies):
            d = dict(dev0)
            if cand_sets:
                d["cand_in"] = torch.from_numpy(cand_sets[c]).to("cuda")
            else:
                from qli_workloads.device import device_pool
                d["pool"], d["k_cache"], d["k_scale"] = device_pool(pb, "cuda")
            self.devs.append(d)
        T = pb.num_tokens
        shp_i, shp_c = Q.output_shapes(T, pb.topk, pb.cand_blocks, pb.mode)
        self.topk_out = torch.empty(shp_i, dtype=torch.int32, device="cuda")
        self.cand_out = torch.empty(shp_c, dtype=torch.int32, device="cuda") if shp_c else None
        self.params = []
        for d in self.devs:
            p = Q.make_params(q=d["q"], q_scale=d["q_scale"], weights=d["weights"],
                              k_cache=d["k_cache"], k_scale=d["k_scale"],
                              block_table=d["block_table"], query_start_loc=d["query_start_loc"],
                              k_lens=d["k_lens"], seq_mod=d["seq_mod"], cand_in=d["cand_in"],
                              ratio=pb.ratio, mode=pb.mode, topk=pb.topk,
                              cand_blocks=pb.cand_blocks, max_k_len=pb.max_k_len,
                              topk_out=self.topk_out, cand_out=self.cand_out)
            self.params.append(p)
        need = Q.qli_workspace_bytes(self.params[0])
        self.ws = torch.empty(max(need, 256), dtype=torch.uint8, device="cuda")
        for p in self.params:
            p.workspace, p.workspace_bytes = self.ws.data_ptr(), self.ws.numel()
        self.stream = torch.cuda.current_stream().cuda_stream

    def step(self, i):
        rc = self.Q.qli_score_topk(self.params[i % len(self.params)], self.stream)
        if rc != self.Q.QLI_OK:
            raise RuntimeError(self.Q.qli_status_string(rc))

    def timed(self, steps, warmup):
        import torch
        for i in range(warmup):
            self.step(i)
        torch.cuda.synchronize()
        start = torch.cuda.Event(enable_timing=True)
        stop = torch.cuda.Event(enable_timing=True)
        t0 = time.perf_counter()
        start.record()
        for i in range(steps):
            self.step(i)
        stop.record()
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
        return start.elapsed_time(stop) / steps, wall

    def kernel_ms(self, steps):
        """Duration per call of each kernel (HIP events recorded by the
        library around each launch, on the launch stream): the sum over the
        call's launches of that kernel (one, except for slices and the
        select's row-length classes), averaged over ``steps`` calls."""
        Q = self.Q
        Q.qli_timing_read(reset=True)
        Q.qli_timing_enable(True)
        try:
            for i in range(steps):
                self.step(i)
            ms, cnt = Q.qli_timing_read(reset=True)
        finally:
            Q.qli_timing_enable(False)
        self.launches = {Q.KERNEL_NAMES[k]: cnt[k] / steps for k in range(len(ms)) if cnt[k]}
        return {Q.KERNEL_NAMES[k]: ms[k] / steps for k in range(len(ms)) if cnt[k]}


def measure(pb, steps, warmup, copies=1, cand_sets=None, bound="hbm", run=None):
    """Time `steps` calls after `warmup` untimed ones, then the per-kernel
    durations; `run` is a Runner built beforehand (else one is built here)."""
    if run is None:
        run = Runner(pb, copies=copies, cand_sets=cand_sets)
    ms, wall = run.timed(steps, warmup)
    kms = run.kernel_ms(steps)
    keys, nbytes, ops = algorithmic(pb, cand_sets[0] if cand_sets else None)
    kern = max(kms, key=kms.get)
    kt = kms[kern] * 1e-3
    traffic, summary = recorded_traffic(pb.name, kern)
    if bound == "hbm":
        achieved = nbytes / kt / 1e9
        roof = {"bound": "hbm", "kernel": kern, "achieved": round(achieved, 1),
                "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                "traffic": traffic, "traffic_summary": summary, "alg_bytes_per_launch": nbytes,
                "kernel_ms": round(kms[kern], 5), "duration_source": DURATION_SOURCE}
    else:
        achieved = ops / kt / 1e12
        roof = {"bound": "mfma", "kernel": kern, "achieved": round(achieved, 1),
                "peak": INT8_PEAK_TOPS, "unit": "TOP/s",
                "frac": round(achieved / INT8_PEAK_TOPS, 4), "traffic": traffic,
                "traffic_summary": summary,
                "alg_ops_per_launch": ops, "kernel_ms": round(kms[kern], 5),
                "duration_source": DURATION_SOURCE}
    launches = run.launches
    roof["launches_per_call"] = launches.get(kern, 1.0)
    del run
    import torch
    torch.cuda.empty_cache()
    return {"keys": keys, "ms_per_step": ms, "wall_s": wall, "kernels_ms": kms, "roofline": roof,
            "keys_per_s": keys / (ms * 1e-3), "launches_per_call": launches}


def source_candidates(pb):
    """Candidate-block output of one GPU call of a source-mode problem
    (numpy [T, 1, cb]): the incoming candidates of the consumer call that
    follows it in the mixed batch."""
    import torch
    run = Runner(pb)
    run.step(0)
    torch.cuda.synchronize()
    cand = run.cand_out.cpu().numpy()
    del run
    torch.cuda.empty_cache()
    return cand


def measure_mixed(steps, warmup):
    """The mixed batch's four layer calls on one request set and block table
    (ratio 1 source, its consumer, ratio 2 source, its consumer), each timed
    on its own; every consumer is fed the candidates its source produced on
    the GPU.  The roofline of a call is the one its arithmetic intensity
    selects (INT8 ops per algorithmic byte against the ridge point)."""
    import qli_workloads as W
    ridge = INT8_PEAK_TOPS * 1e12 / (HBM_PEAK_GBS * 1e9)
    out, cand = {}, None
    tot_keys, tot_ms = 0, 0.0
    for pb in W.mixed_calls():
        sets = [cand] if pb.mode == 3 else None
        _, nbytes, ops = algorithmic(pb, cand if pb.mode == 3 else None)
        bound = "mfma" if ops > ridge * nbytes else "hbm"
        m = measure(pb, steps, warmup, cand_sets=sets, bound=bound)
        out[pb.name] = {"tokens": pb.num_tokens, "mode": {2: "source", 3: "consumer"}[pb.mode],
                        "ratio": pb.ratio, "topk": pb.topk,
                        "cand_blocks": pb.cand_blocks or pb.cand_in_blocks,
                        "keys": m["keys"], "keys_per_s": round(m["keys_per_s"], 1),
                        "ms_per_call": round(m["ms_per_step"], 5), "kernels_ms": m["kernels_ms"],
                        "roofline": m["roofline"]}
        tot_keys += m["keys"]
        tot_ms += m["ms_per_step"]
        log(f"{pb.name}: {m['ms_per_step']:.4f} ms/call kernels {m['kernels_ms']}")
        cand = source_candidates(pb) if pb.mode == 2 else None
    return {"keys_per_s": round(tot_keys / (tot_ms * 1e-3), 1), "ms_per_four_calls": round(tot_ms, 5),
            "calls": out}


def measure_producers(steps, warmup, copies=2):
    """Query quantization and the index-K write at the shapes of the decode
    and prefill workloads: each launch timed with HIP events on its stream
    (the library's timing facility), against HBM.  Algorithmic bytes: per
    row, its 128 values in + 128 INT8 codes + one FP16 scale out; per head
    weight, its value in + 2 bytes out; per K row also its 8-byte slot.
    ``copies`` rotated input/output sets keep the previous launch's data out
    of the last-level cache."""
    import numpy as np
    import torch

    import quantized_top_indexer_amd as Q
    import qli_workloads as W
    Q.load_library()
    out = {}

    def timed(launch, kernel_id):
        for i in range(warmup):
            launch(i)
        torch.cuda.synchronize()
        Q.qli_timing_read(reset=True)
        Q.qli_timing_enable(True)
        try:
            for i in range(steps):
                launch(i)
            ms, cnt = Q.qli_timing_read(reset=True)
        finally:
            Q.qli_timing_enable(False)
        return ms[kernel_id] / cnt[kernel_id]

    # query quantization: T tokens x N heads of bfloat16, bfloat16 weights
    for name, T, N in (("quantize_query_prefill", 8192, 64), ("quantize_query_decode", 64, 64)):
        rows = T * N
        x = W.make_activations(7, 0, rows, "bf16").view(np.int16)
        w = W.make_head_weights(7, 0, rows, "bf16").view(np.int16)
        sets = []
        for c in range(copies):
            xt = torch.from_numpy(x).cuda().view(torch.bfloat16).view(T, N, 128)
            wt = torch.from_numpy(w).cuda().view(torch.bfloat16).view(T, N)
            sets.append((xt, wt, torch.empty((T, N, 128), dtype=torch.int8, device="cuda"),
                         torch.empty((T, N), dtype=torch.float16, device="cuda"),
                         torch.empty((T, N), dtype=torch.float16, device="cuda")))

        def launch(i, sets=sets):
            xt, wt, q, qs, wo = sets[i % len(sets)]
            Q.quantize_query(xt, wt, q=q, q_scale=qs, w_out=wo)
        kms = timed(launch, Q.QLI_KERNEL_QUANTIZE)
        nbytes = rows * (256 + 128 + 2) + rows * (2 + 2)
        out[name] = _producer_line(name, "quantize_kernel", kms, nbytes, rows,
                                   {"tokens": T, "heads": N, "x": "bf16", "weights": "bf16"})
        del sets
        torch.cuda.empty_cache()

    # index-K write: the compressed K rows of one prefill chunk (8192 raw
    # tokens at ratio 2 -> 4096 rows, 64-row pages at 131072 B) and of one
    # decode step (64 requests x 1 row, 128-row pages at 147712 B)
    for name, ratio, rows, pages in (("write_k_prefill", 2, 4096, 157 * 4),
                                     ("write_k_decode", 1, 64, 16384)):
        R, stride, koff, soff = W.page_layout(ratio)
        pool = torch.empty((pages, stride), dtype=torch.uint8, device="cuda")
        kv = pool[:, koff:koff + R * 128].view(torch.int8).view(pages, R, 128)
        sv = pool[:, soff:soff + R * 2].view(torch.int16)
        rng = np.random.default_rng(9)
        if rows == 64:   # one new row per request, each in its own page
            slot = rng.permutation(pages)[:rows].astype(np.int64) * R + rng.integers(0, R, rows)
        else:            # consecutive positions of one request over shuffled pages
            pg = rng.permutation(pages)[:rows // R].astype(np.int64)
            slot = (pg[:, None] * R + np.arange(R)[None, :]).reshape(-1)
        x = W.make_activations(8, ratio, rows, "bf16", which="k").view(np.int16)
        sets = [(torch.from_numpy(x).cuda().view(torch.bfloat16),
                 torch.from_numpy(slot).cuda()) for _ in range(copies)]

        def launch(i, sets=sets, kv=kv, sv=sv):
            xt, st = sets[i % len(sets)]
            Q.write_index_k(xt, st, kv, sv)
        kms = timed(launch, Q.QLI_KERNEL_WRITE_K)
        nbytes = rows * (256 + 8 + 128 + 2)
        out[name] = _producer_line(name, "write_k_kernel", kms, nbytes, rows,
                                   {"rows": rows, "ratio": ratio, "page_rows": R,
                                    "page_stride_bytes": stride, "x": "bf16"})
        del sets, pool, kv, sv
        torch.cuda.empty_cache()
    return out


def measure_attention(steps, warmup, index_sets=4, prepared=None):
    """The sparse-attention consumer of the indices at the decode shape
    (attn_decode: 64 tokens x 2048 selected positions + a 128-position window,
    64 heads, D = 512), each launch timed with HIP events on its stream,
    against HBM.  Algorithmic bytes: every entry's 1024-byte row once per
    token (the head groups of a token share it through their XCD's L2), the
    queries and outputs (64 x 1 KB each per token), the index row and the
    log-sum-exp.  ``index_sets`` rotated index sets (rows drawn for all of
    them) keep the previous launch's rows out of the last-level cache.  The
    matrix work (S^T and O^T, 4 * H * D flops per entry) is reported beside
    it against the dense BF16 peak."""
    import numpy as np
    import torch

    import quantized_top_indexer_amd as Q
    from qli_workloads import attn as A
    if prepared is None:
        log("attn_decode: generating")
        ap, sets = A.attn_decode(index_sets=index_sets)
    else:
        ap, sets = prepared
    dev = lambda a, dt=None: torch.from_numpy(np.ascontiguousarray(a if dt is None else a.astype(dt))).cuda()
    q = dev(ap.q.view(np.int16)).view(torch.bfloat16)
    c_cache, r_cache = dev(ap.c_pages), dev(ap.r_pages)
    c_bt, r_bt = dev(ap.c_bt, np.int32), dev(ap.r_bt, np.int32)
    c_lens, r_lens = dev(ap.c_lens, np.int32), dev(ap.r_lens, np.int32)
    qsl, sinks = dev(ap.query_start_loc, np.int32), dev(ap.sinks, np.float32)
    idx = [dev(x, np.int32) for x in sets]
    out = torch.empty((ap.num_tokens, ap.num_heads, ap.head_dim), dtype=torch.bfloat16, device="cuda")
    lse = torch.empty((ap.num_tokens, ap.num_heads), dtype=torch.float32, device="cuda")

    def launch(i):
        Q.sparse_attention(q, c_cache, c_bt, c_lens, qsl, indices=idx[i % len(idx)], r_cache=r_cache,
                           r_block_table=r_bt, r_lens=r_lens, window=ap.window, sinks=sinks, scale=ap.scale,
                           c_page_rows=ap.c_page_rows, c_page_stride=ap.c_page_stride,
                           c_num_pages=ap.c_pages.shape[0], r_page_rows=ap.r_page_rows,
                           r_page_stride=ap.r_page_stride, r_num_pages=ap.r_pages.shape[0], out=out, lse=lse)
    for i in range(warmup):
        launch(i)
    torch.cuda.synchronize()
    Q.qli_timing_read(reset=True)
    Q.qli_timing_enable(True)
    t0 = time.perf_counter()
    try:
        for i in range(steps):
            launch(i)
        torch.cuda.synchronize()
        wall = (time.perf_counter() - t0) / steps
        ms, cnt = Q.qli_timing_read(reset=True)
    finally:
        Q.qli_timing_enable(False)
    # the split kernel (and its merge launch) when the heads are a multiple of
    # 64, else the head-group kernel; the roofline takes the call's launches
    # together
    kid = Q.QLI_KERNEL_ATTN_SPLIT if cnt[Q.QLI_KERNEL_ATTN_SPLIT] else Q.QLI_KERNEL_ATTN
    kname = Q.KERNEL_NAMES[kid]
    main_ms = ms[kid] / steps
    merge_ms = ms[Q.QLI_KERNEL_ATTN_MERGE] / steps
    kms = main_ms + merge_ms
    entries = int((sets[0] >= 0).sum()) + ap.num_tokens * ap.window
    T, H, D = ap.num_tokens, ap.num_heads, ap.head_dim
    nbytes = entries * D * 2 + T * H * D * 2 * 2 + T * ap.topk * 4 + T * H * 4
    flops = 4 * H * D * entries
    achieved = nbytes / (kms * 1e-3) / 1e9
    traffic, summary = recorded_traffic("attn_decode", kname, source="qli_attn.hip")
    log(f"attn_decode: {kms:.5f} ms {achieved:.1f} GB/s")
    del c_cache, r_cache, idx
    torch.cuda.empty_cache()
    return {"attn_decode": {
        "config": {"tokens": T, "heads": H, "head_dim": D, "topk": ap.topk, "window": ap.window,
                   "compressed_len": int(ap.c_lens[0]), "page_rows": ap.c_page_rows,
                   "page_stride_bytes": ap.c_page_stride, "sinks": True, "index_sets": len(sets)},
        "kernel_ms": round(kms, 5), "main_kernel_ms": round(main_ms, 5), "merge_kernel_ms": round(merge_ms, 5),
        "ms_per_call": round(wall * 1e3, 5),
        "entries_per_s": round(entries / (kms * 1e-3), 1),
        "roofline": {"bound": "hbm", "kernel": kname, "achieved": round(achieved, 1),
                     "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "traffic": traffic, "traffic_summary": summary, "alg_bytes_per_launch": nbytes,
                     "duration_source": "HIP events the library records around each launch; the "
                                        "call's launches (attention kernel and merge) summed"},
        "bf16_mfma": {"flops_per_launch": flops, "achieved_TFLOPs": round(flops / (kms * 1e-3) / 1e12, 1),
                      "peak_TFLOPs": BF16_PEAK_TFLOPS,
                      "frac": round(flops / (kms * 1e-3) / 1e12 / BF16_PEAK_TFLOPS, 4)},
    }}


def measure_ceilings():
    """What this GPU sustains: a 2 GiB streaming read with 16-byte
    non-temporal loads (GB/s) and back-to-back independent INT8 MFMAs on
    every SIMD (TOP/s), each the best of 10 timed launches after 3 warm-ups
    (include/qli_probe.h)."""
    import torch

    import quantized_top_indexer_amd as Q
    sink = torch.zeros(65536, dtype=torch.int32, device="cuda")
    buf = torch.empty(2 << 30, dtype=torch.uint8, device="cuda")
    buf.fill_(1)

    def best(launch):
        for _ in range(3):
            launch()
        t = []
        for _ in range(10):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            launch()
            e1.record()
            torch.cuda.synchronize()
            t.append(e0.elapsed_time(e1) * 1e-3)
        return min(t)

    def read():
        rc = Q.qli_probe_hbm_read(buf.data_ptr(), buf.numel(), 4096, sink.data_ptr())
        assert rc == Q.QLI_OK, Q.qli_status_string(rc)

    grid, iters = 2048, 20000

    def mfma():
        rc = Q.qli_probe_int8_mfma(grid, iters, sink.data_ptr())
        assert rc == Q.QLI_OK, Q.qli_status_string(rc)
    tops = Q.qli_probe_int8_mfma_ops(grid, iters) / best(mfma) / 1e12
    hbm = buf.numel() / best(read) / 1e9  # last: the memory clocks are up afterwards
    del buf
    torch.cuda.empty_cache()
    return {"hbm_read_GBps": round(hbm, 1), "int8_mfma_TOPs": round(tops, 1)}


def with_measured(roof, ceilings):
    """Add the measured ceiling of the roofline's unit and the fraction of it."""
    if not ceilings:
        return roof
    peak = ceilings["hbm_read_GBps"] if roof["unit"] == "GB/s" else ceilings["int8_mfma_TOPs"]
    roof["measured_peak"] = peak
    roof["frac_of_measured"] = round(roof["achieved"] / peak, 4)
    return roof


def _producer_line(name, kernel, kms, nbytes, rows, config):
    achieved = nbytes / (kms * 1e-3) / 1e9
    traffic, summary = recorded_traffic(name, kernel, source="qli_quant.hip")
    return {"config": config, "kernel_ms": round(kms, 5), "rows_per_s": round(rows / (kms * 1e-3), 1),
            "roofline": {"bound": "hbm", "kernel": kernel, "achieved": round(achieved, 1),
                         "peak": HBM_PEAK_GBS, "unit": "GB/s",
                         "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": traffic,
                         "traffic_summary": summary, "alg_bytes_per_launch": nbytes}}


def cpu_model():
    """The host CPU's model name (Linux /proc/cpuinfo), or None."""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def host_threads():
    """Threads the all-core oracle run uses: the CPUs this process may run
    on, capped by OMP_NUM_THREADS when that is set (the host's CPU share of
    one GPU)."""
    try:
        n = len(os.sched_getaffinity(0))
    except (AttributeError, OSError):
        n = os.cpu_count() or 1
    cap = os.environ.get("OMP_NUM_THREADS", "")
    if cap.isdigit() and int(cap) > 0:
        n = min(n, int(cap))
    return max(1, n)


def cpu_baseline(pb, single_tokens=16):
    """The oracle as it stands, timed on the host: once on one thread over
    the first ``single_tokens`` query tokens, once on every thread of the
    host's share over all of the workload's tokens (threads take tokens)."""
    import numpy as np

    import oracle
    assert pb.mode != 3, "the CPU baseline runs on a source or plain workload"
    vis = []
    for b in range(pb.batch):
        n = int(pb.query_start_loc[b + 1] - pb.query_start_loc[b])
        vis += [(int(pb.raw_lens[b]) - n + i + 1) // pb.ratio for i in range(n)]
    o = oracle.OracleProblem(pb)

    def timed(toks, nthreads):
        t0 = time.perf_counter()
        o.run(tokens=toks, nthreads=nthreads)
        dt = time.perf_counter() - t0
        keys = int(sum(vis[int(t)] for t in toks))
        return keys, dt

    one = np.arange(min(single_tokens, pb.num_tokens))
    k1, d1 = timed(one, 1)
    nthreads = host_threads()
    allt = np.arange(pb.num_tokens)
    kn, dn = timed(allt, nthreads)
    return {"value": round(kn / dn, 1), "unit": "keys/s", "cores": nthreads, "kind": "oracle",
            "sample": f"all {len(allt)} query tokens of {pb.name} ({kn} keys, {dn:.2f} s wall "
                      f"on {nthreads} threads, one token per thread at a time)",
            "single_thread": {"value": round(k1 / d1, 1), "unit": "keys/s", "cores": 1,
                              "sample": f"first {len(one)} of {pb.num_tokens} query tokens "
                                        f"({k1} keys, {d1:.2f} s wall)"},
            "host_cpus": os.cpu_count(), "cpu_model": cpu_model()}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=300,
                    help="untimed steps first: the GPU reaches its sustained clocks only after "
                         "some milliseconds of continuous work")
    ap.add_argument("--copies", type=int, default=4)
    ap.add_argument("--workload", default="decode_source",
                    help="main workload (decode_source is the headline configuration)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--others", default="prefill_chunk,decode_consumer_1m,mixed",
                    help="comma list of secondary workloads ('' for none; 'mixed' = the four "
                         "layer calls of the mixed batch)")
    ap.add_argument("--no-producers", action="store_true",
                    help="skip the query-quantization and index-K write measurements")
    ap.add_argument("--no-attention", action="store_true",
                    help="skip the sparse-attention consumer of the indices")
    ap.add_argument("--attention-only", action="store_true",
                    help="only measure the sparse-attention consumer (one JSON object, for profiling runs)")
    ap.add_argument("--no-ceilings", action="store_true",
                    help="skip the measured HBM-read and INT8-MFMA ceilings")
    ap.add_argument("--producers-only", action="store_true",
                    help="only measure the producers (one JSON object, for profiling runs)")
    ap.add_argument("--copy-calibration", type=float, default=0.0, metavar="MIB",
                    help="only run a plain device copy kernel of this many MiB (5 launches), "
                         "to scale HBM byte counters")
    args = ap.parse_args()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU: the indexer library has no multi-GPU path "
              "(requests or positions would shard with no exchange / one top-k merge; "
              "see the design notes). Run with --gpus 1.", file=sys.stderr)
        sys.exit(2)

    import torch
    import qli_workloads as W
    assert torch.cuda.is_available(), "bench.py needs a GPU"
    if args.copy_calibration:
        n = int(args.copy_calibration * (1 << 20)) // 4
        src = torch.ones(n, dtype=torch.int32, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(5):
            torch.mul(src, 1, out=dst)  # one elementwise kernel: reads n*4 B, writes n*4 B
        torch.cuda.synchronize()
        print(json.dumps({"copy_kernel_bytes_read": n * 4, "copy_kernel_bytes_written": n * 4,
                          "launches": 5}), flush=True)
        return
    import quantized_top_indexer_amd as Q
    Q.load_library()
    if args.producers_only:
        print(json.dumps({"producers": measure_producers(args.steps, args.warmup)}), flush=True)
        return
    if args.attention_only:
        print(json.dumps({"consumer_attention": measure_attention(args.steps, args.warmup)}), flush=True)
        return

    def prepare_workload(name, copies):
        """Inputs of a named single-call workload on the GPU: (problem,
        Runner, candidate sets, bound)."""
        log(f"{name}: generating")
        wpb = W.WORKLOADS[name]()
        sets, bound = None, "hbm"
        if name == "decode_consumer_1m":
            import numpy as np
            from qli_workloads import make_candidates, visible_counts, Requests
            vis = visible_counts(Requests(n=np.ones(wpb.batch, np.int64), S=wpb.raw_lens),
                                 wpb.ratio)
            # eight candidate sets: the touched K rows of successive calls differ
            sets = [wpb.cand_in] + [make_candidates(wpb.seed + 100 * c, 1, vis, 2048)
                                    for c in range(1, 8)]
            copies = 8
        elif name == "prefill_chunk":
            copies, bound = 1, "mfma"
        return wpb, Runner(wpb, copies=copies, cand_sets=sets), sets, bound

    def run_workload(name, steps, copies):
        if name.startswith("mixed_r"):
            # one of the mixed batch's four layer calls on its own (for
            # profiling); a consumer is fed its source's GPU candidates
            log(f"{name}: generating")
            calls = {c.name: c for c in W.mixed_calls()}
            wpb = calls[name]
            _, nbytes, ops = algorithmic(wpb, None) if wpb.mode == 2 else (None, None, None)
            sets = None
            if wpb.mode == 3:
                src = calls[name.replace("consumer", "source")]
                sets = [source_candidates(src)]
                wpb.cand_in_blocks = src.cand_blocks
                _, nbytes, ops = algorithmic(wpb, sets[0])
            ridge = INT8_PEAK_TOPS * 1e12 / (HBM_PEAK_GBS * 1e9)
            m = measure(wpb, steps, args.warmup, cand_sets=sets,
                        bound="mfma" if ops > ridge * nbytes else "hbm")
        else:
            wpb, run, sets, bound = prepare_workload(name, copies)
            m = measure(wpb, steps, args.warmup, cand_sets=sets, bound=bound, run=run)
            del run
        log(f"{name}: {m['ms_per_step']:.4f} ms/call kernels {m['kernels_ms']}")
        return wpb, m

    # The headline's inputs go to the GPU first and the headline is timed last,
    # right after the other workloads and the ceiling probes (a 2 GiB
    # streaming read among them): from an idle GPU its memory clocks take
    # tens of milliseconds of traffic to come up, and a call timed after only
    # a few warm-up calls would measure that ramp (decode_source: 73 us from
    # idle with 5 warm-up calls, 70.5 us right after the probes, 68.7 us at
    # steady state, on one box).
    main_prep = None
    if args.workload in W.WORKLOADS:
        main_prep = prepare_workload(args.workload, args.copies)
    else:
        pb, main_m = run_workload(args.workload, args.steps, args.copies)
    others = {}
    for name in [s for s in args.others.split(",") if s and s != args.workload]:
        if name == "mixed":
            log("mixed: generating the four layer calls")
            others["mixed"] = measure_mixed(max(10, args.steps // 5), args.warmup)
            continue
        opb, m = run_workload(name, max(10, args.steps // 5) if name == "prefill_chunk"
                              else args.steps, args.copies)
        others[name] = {"keys_per_s": round(m["keys_per_s"], 1),
                        "ms_per_call": round(m["ms_per_step"], 5), "kernels_ms": m["kernels_ms"],
                        "roofline": m["roofline"]}
        del opb
    producers = {}
    if not args.no_producers:
        log("producers: query quantization and index-K write")
        producers = measure_producers(args.steps, args.warmup)
        for k, v in producers.items():
            log(f"{k}: {v['kernel_ms']:.5f} ms {v['roofline']['achieved']} GB/s")

    attention = {}
    if not args.no_attention:
        log("consumer attention: sparse attention over the decode indices")
        attention = measure_attention(args.steps, args.warmup)

    ceilings = None
    if not args.no_ceilings:
        log("ceilings: streaming read and INT8 MFMA probes")
        ceilings = measure_ceilings()
        log(f"ceilings: {ceilings}")

    if main_prep is not None:
        pb, run, sets, bound = main_prep
        del main_prep
        main_m = measure(pb, args.steps, args.warmup, cand_sets=sets, bound=bound, run=run)
        del run
        log(f"{args.workload}: {main_m['ms_per_step']:.4f} ms/call kernels {main_m['kernels_ms']}")

    if ceilings is not None:
        with_measured(main_m["roofline"], ceilings)
        for v in list(others.values()) + list(producers.values()) + list(attention.values()):
            for r in ([c["roofline"] for c in v["calls"].values()] if "calls" in v
                      else [v["roofline"]]):
                with_measured(r, ceilings)

    cpu = None
    if not args.no_cpu_baseline and pb.mode != 3:
        log("cpu baseline: oracle on the host")
        cpu = cpu_baseline(pb)

    line = {
        # keys/s is the value; the decode HBM rate is roofline.achieved and the
        # prefill INT8 MFMA fraction other_workloads.prefill_chunk.roofline.frac
        "metric": "compressed keys scored/s; decode HBM GB/s & prefill INT8 MFMA %peak",
        "value": round(main_m["keys_per_s"], 1),
        "unit": "keys/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(main_m["ms_per_step"], 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "i8",
        "data": "synthetic",
        "config": {"workload": pb.name, "requests": pb.batch, "query_tokens": pb.num_tokens,
                   "compressed_len": pb.max_k_len, "ratio": pb.ratio, "heads": pb.num_heads,
                   "head_dim": 128, "mode": {1: "plain", 2: "source", 3: "consumer"}[pb.mode],
                   "topk": pb.topk, "cand_blocks": pb.cand_blocks or pb.cand_in_blocks,
                   "page_rows": pb.page_rows, "page_stride_bytes": pb.layout()[1],
                   "rotated_cache_copies": args.copies if pb.mode != 3 else 8,
                   "parallelism": "single GPU"},
        "roofline": main_m["roofline"],
        "cpu_baseline": cpu,
        "kernels_ms": main_m["kernels_ms"],
        "other_workloads": others,
        "producers": producers,
        "consumer_attention": attention,
        "measured_ceilings": ceilings,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
