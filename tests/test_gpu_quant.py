"""GPU parity of the two producers of the indexer's inputs: query
quantization (INT8 heads, FP16 scales, FP16 weights) and the index-K cache
write (INT8 rows and FP16 scales scattered into the paged pool), bit for
bit against the oracle, plus the chain quantize -> write K -> score/top-k
against the same chain run by the oracle."""
import dataclasses

import numpy as np
import pytest

import oracle
import qli_workloads as W
from gpu_check import compare, oracle_rows, run_gpu, say

pytestmark = pytest.mark.gpu


def torch_in(a, dtype_name):
    import torch
    if dtype_name == "bf16":
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).cuda().view(torch.bfloat16)
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).cuda()


def gpu_quantize(x, w=None, dtype="bf16", wdtype="bf16"):
    import torch

    import quantized_top_indexer_amd as Q
    xt = torch_in(x, dtype)
    wt = None if w is None else torch_in(w, wdtype)
    q, qs, wo = Q.quantize_query(xt, wt)
    torch.cuda.synchronize()
    return (q.cpu().numpy(), qs.view(torch.int16).cpu().numpy().view(np.uint16),
            None if wo is None else wo.view(torch.int16).cpu().numpy().view(np.uint16))


def special_rows():
    """Rows that reach every branch of the quantizer: exact ties at a
    power-of-two scale, a zero row, rows whose scale underflows to FP16
    subnormals or to zero, rows whose scale saturates, negative maxima,
    FP32 subnormal values, a single non-zero value."""
    rows = []
    r = np.zeros(128, np.float32)
    rows.append(r.copy())                                        # all zero
    for k in (-6, 0, 3):                                         # s = 2^k, ties k + 1/2
        r = (np.arange(128, dtype=np.float32) - 63.5) * np.float32(2.0 ** k)
        r[0] = np.float32(-127 * 2.0 ** k)
        rows.append(r)
    r = np.zeros(128, np.float32)
    r[7] = -5.0                                                  # negative maximum
    r[8] = 2.5
    rows.append(r)
    for t in (1.2, 1.45, 2.45, 0.4, 0.6):                        # subnormal / zero scale
        r = np.linspace(-1, 1, 128).astype(np.float32) * np.float32(127 * t * 2.0 ** -24)
        rows.append(r)
    for big in (127 * 70000.0, 3.0e38, 1.0e30):                  # saturated scale
        r = np.linspace(-1, 1, 128).astype(np.float32) * np.float32(big)
        rows.append(r)
    r = np.full(128, np.float32(1e-41))                          # FP32 subnormal inputs
    r[3] = np.float32(-3e-39)
    rows.append(r)
    r = np.zeros(128, np.float32)
    r[127] = 0.1                                                 # one non-zero value
    rows.append(r)
    rows.append(np.full(128, np.float32(-7.25)))                 # all equal
    x = np.stack(rows).astype(np.float32)
    # the scale 1 - 2^-13 rounds to 1.0 in FP16, so 2.5 is a tie only after
    # rounding the scale (the unrounded quotient would be 2.5003)
    r = np.zeros(128, np.float32)
    r[0] = np.float32(127 * (1 - 2.0 ** -13))
    r[1:9] = [2.5, -3.5, 0.5, -0.5, 126.5, 1.5, 64.5, -64.5]
    return np.concatenate([x, r[None]])


@pytest.mark.parametrize("dtype,wdtype,rows,nw", [
    ("bf16", "bf16", 3001, 5000),     # one pass per workgroup, ragged; more weights than rows
    ("f32", "f32", 3001, 5000),
    ("bf16", "f32", 40007, 40007),    # four passes per workgroup, ragged last workgroup
    ("f32", "bf16", 40007, 1000),     # fewer weights than rows
])
def test_quantize_parity(dtype, wdtype, rows, nw):
    say(f"quantize {dtype}/{wdtype} rows={rows} weights={nw}")
    x = W.make_activations(11, 0, rows, dtype)
    w = W.make_head_weights(11, 0, nw, wdtype)
    q, s, wo = gpu_quantize(x, w, dtype, wdtype)
    oq, osc = oracle.quantize_rows(x)
    assert np.array_equal(s, osc)
    assert np.array_equal(q, oq)
    assert np.array_equal(wo, oracle.round_weights(w))


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_quantize_special_rows(dtype):
    x = special_rows()
    if dtype == "bf16":
        x = W.bf16_bits(x)
    say(f"quantize special rows {dtype}: {x.shape[0]}")
    q, s, _ = gpu_quantize(x, None, dtype)
    oq, osc = oracle.quantize_rows(x)
    assert np.array_equal(s, osc)
    assert np.array_equal(q, oq)
    if dtype == "f32":
        assert s[0] == 0 and np.all(q[0] == 0)
        assert np.any(osc == 0x7BFF)          # the saturated scale was reached


def near_tie_rows(rows, seed):
    """Rows whose quotients x / s sit on or within a few FP32 ulp of
    half-integers, for scales s with full FP16 mantissas (so 1 / s is not
    exact and the shortcut through the reciprocal must defer to the
    correctly rounded quotient)."""
    rng = np.random.default_rng(seed)
    mant = 1.0 + rng.integers(1, 1024, size=(rows, 1)) / 1024.0
    s = mant * 2.0 ** rng.integers(-8, 8, size=(rows, 1))     # exact FP16 values
    k = rng.integers(-127, 127, size=(rows, 128)) + 0.5
    d = rng.integers(-6, 7, size=(rows, 128)) * 2.0 ** -19
    x = ((k + d) * s).astype(np.float32)
    x[:, 0] = (127 * s[:, 0]).astype(np.float32)
    return x


def test_quantize_near_ties_dense():
    x = near_tie_rows(2048, 5)
    q, s, _ = gpu_quantize(x, None, "f32")
    oq, osc = oracle.quantize_rows(x)
    assert np.array_equal(s, osc) and np.array_equal(q, oq)


def test_quantize_empty_and_weights_only():
    import torch

    import quantized_top_indexer_amd as Q
    x = torch.zeros((0, 128), dtype=torch.bfloat16, device="cuda")
    w = torch_in(W.make_head_weights(3, 0, 777, "f32"), "f32")
    q, qs, wo = Q.quantize_query(x, w)
    torch.cuda.synchronize()
    assert q.shape == (0, 128) and qs.shape == (0,)
    got = wo.view(torch.int16).cpu().numpy().view(np.uint16)
    assert np.array_equal(got, oracle.round_weights(W.make_head_weights(3, 0, 777, "f32")))


def test_quantize_prefill_chunk_size():
    """Full size of the prefill chunk's queries: 8192 tokens x 64 heads of
    bfloat16, every row compared."""
    T, N = 8192, 64
    say(f"quantize full prefill size rows={T * N}")
    x = W.make_activations(2, 0, T * N, "bf16").reshape(T, N, 128)
    w = W.make_head_weights(2, 0, T * N, "bf16").reshape(T, N)
    q, s, wo = gpu_quantize(x, w)
    oq, osc = oracle.quantize_rows(x)
    assert np.array_equal(s, osc)
    assert np.array_equal(q, oq)
    assert np.array_equal(wo, oracle.round_weights(w))


def pool_for(ratio, num_pages, seed):
    """A poisoned device pool with random K already in place (the state of a
    cache before new rows are written) and its host copy."""
    import torch

    from qli_workloads.device import device_pool
    R = W.page_layout(ratio)[0]
    rng = np.random.default_rng(seed)
    kp = rng.integers(-127, 128, size=(num_pages, R, 128), dtype=np.int8)
    sp = rng.integers(0x1000, 0x2000, size=(num_pages, R)).astype(np.uint16)
    fake = dataclasses.make_dataclass("P", ["ratio", "num_pages", "k_pages", "s_pages"])
    pool, kv, sv = device_pool(fake(ratio, num_pages, kp, sp))
    torch.cuda.synchronize()
    return pool, kv, sv, kp, sp


def read_pool(kv, sv):
    import torch
    torch.cuda.synchronize()
    return kv.cpu().numpy(), sv.cpu().numpy().view(np.uint16)


@pytest.mark.parametrize("ratio,dtype", [(2, "bf16"), (1, "f32"), (2, "f32"), (1, "bf16")])
def test_write_k_parity(ratio, dtype):
    import torch

    import quantized_top_indexer_amd as Q
    P = 37
    R = W.page_layout(ratio)[0]
    pool, kv, sv, kp, sp = pool_for(ratio, P, 21 + ratio)
    before = pool.cpu().numpy()
    rng = np.random.default_rng(31 + ratio)
    rows = 1001
    slot = rng.permutation(P * R)[:rows].astype(np.int64)
    slot[rng.random(rows) < 0.05] = -1
    slot[[5, 77, 500]] = [P * R, P * R + 9999, 1 << 40]       # beyond the pool: flagged
    x = W.make_activations(41, ratio, rows, dtype, which="k")
    status = torch.zeros(1, dtype=torch.int32, device="cuda")
    say(f"write_k ratio={ratio} {dtype} rows={rows} pool={P}x{R}")
    Q.write_index_k(torch_in(x, dtype), torch.from_numpy(slot).cuda(), kv, sv, status_out=status)
    gk, gs = read_pool(kv, sv)
    ok, os_ = oracle.write_k(x, slot, kp, sp)
    assert np.array_equal(gs, os_)
    assert np.array_equal(gk, ok)
    assert int(status.item()) == Q.QLI_DEV_BAD_PAGE
    # nothing outside the K rows and scales of the pool moved
    after = pool.cpu().numpy()
    _, _, koff, soff = W.page_layout(ratio)
    mask = np.ones(before.shape, bool)
    mask[:, koff:koff + R * 128] = False
    mask[:, soff:soff + R * 2] = False
    assert np.array_equal(after[mask], before[mask])


def test_write_k_in_range_sets_no_status():
    import torch

    import quantized_top_indexer_amd as Q
    pool, kv, sv, kp, sp = pool_for(2, 4, 3)
    slot = np.array([0, 255, 64, -1, 130], np.int64)
    x = W.make_activations(5, 0, len(slot), "bf16", which="k")
    status = torch.zeros(1, dtype=torch.int32, device="cuda")
    Q.write_index_k(torch_in(x, "bf16"), torch.from_numpy(slot).cuda(), kv, sv, status_out=status)
    gk, gs = read_pool(kv, sv)
    ok, os_ = oracle.write_k(x, slot, kp, sp)
    assert np.array_equal(gk, ok) and np.array_equal(gs, os_)
    assert int(status.item()) == 0


@pytest.mark.parametrize("ratio,mode", [(2, 2), (1, 2), (2, 1)])
def test_chain_quantize_write_score(ratio, mode):
    """Un-quantized queries, weights and K rows go through the two producers
    and then the indexer on the GPU; the oracle runs the same chain on the
    CPU; indices, candidates and scores must agree bit for bit."""
    import torch

    import quantized_top_indexer_amd as Q
    from qli_workloads.device import call_kwargs, to_device
    req = W.Requests(n=np.array([3, 1, 40]), S=np.array([700, 2049, 1500]))
    pb = W.build_problem(f"chain_r{ratio}_m{mode}", 60 + ratio, req, ratio=ratio, num_heads=64,
                         mode=mode, topk=100, cand_blocks=64)
    T, N = pb.q.shape[:2]
    xq = W.make_activations(61, ratio, T * N, "bf16").reshape(T, N, 128)
    wf = W.make_head_weights(61, ratio, T * N, "bf16").reshape(T, N)
    slot = W.request_slots(pb.block_table, pb.k_lens, ratio)
    xk = W.make_activations(62, ratio, len(slot), "bf16", which="k")
    say(f"chain ratio={ratio} mode={mode} T={T} K rows={len(slot)}")

    # oracle chain
    q, qs = oracle.quantize_rows(xq)
    w16 = oracle.round_weights(wf)
    kp, sp = oracle.write_k(xk, slot, pb.k_pages, pb.s_pages)
    opb = dataclasses.replace(pb, q=q, q_scale=qs, weights=w16, k_pages=kp, s_pages=sp)
    orc = oracle_rows(opb, scores=True)

    # GPU chain: the pool starts with the problem's (poisoned, random) pages
    dev = to_device(pb, "cuda")
    gq, gqs, gw = Q.quantize_query(torch_in(xq, "bf16"), torch_in(wf, "bf16"))
    Q.write_index_k(torch_in(xk, "bf16"), torch.from_numpy(slot).cuda(), dev["k_cache"],
                    dev["k_scale"])
    kw = call_kwargs(pb, dev)
    kw.update(q=gq, q_scale=gqs, weights=gw)
    idx, cand, dbg = Q.score_topk(**kw, debug_scores=True)
    torch.cuda.synchronize()
    gpu = {"topk": idx[:, 0].cpu().numpy(),
           "cand": None if cand is None else cand[:, 0].cpu().numpy(),
           "scores": dbg.cpu().numpy()}
    compare(opb, gpu, orc)
    # the same problem through run_gpu (inputs quantized by the oracle) agrees too
    ref = run_gpu(opb, debug=False)
    assert np.array_equal(ref["topk"], gpu["topk"])
