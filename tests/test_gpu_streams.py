"""Stream semantics of the C ABI on the GPU: calls are stateless and
re-entrant with distinct workspaces (two streams in flight at once give the
sequential results), and a call captured in a HIP graph replays correctly,
on the live buffers, with other work between the replays."""
import numpy as np
import pytest

import qli_workloads as W
from gpu_check import say, small_problem

pytestmark = pytest.mark.gpu


def prepared(pb):
    """Device inputs, preallocated outputs and workspace, and qli_params."""
    import torch

    import quantized_top_indexer_amd as Q
    from qli_workloads.device import call_kwargs, to_device
    dev = to_device(pb, "cuda")
    kw = call_kwargs(pb, dev)
    shp_i, shp_c = Q.output_shapes(pb.num_tokens, pb.topk, pb.cand_blocks, pb.mode)
    topk_out = torch.full(shp_i, -7, dtype=torch.int32, device="cuda")
    cand_out = torch.full(shp_c, -7, dtype=torch.int32, device="cuda") if shp_c else None
    p = Q.make_params(**kw, topk_out=topk_out, cand_out=cand_out)
    ws = torch.empty(max(Q.qli_workspace_bytes(p), 256), dtype=torch.uint8, device="cuda")
    p.workspace, p.workspace_bytes = ws.data_ptr(), ws.numel()
    return {"dev": dev, "p": p, "ws": ws, "topk": topk_out, "cand": cand_out}


def launch(st, stream):
    import quantized_top_indexer_amd as Q
    rc = Q.qli_score_topk(st["p"], stream)
    assert rc == Q.QLI_OK, Q.qli_status_string(rc)


def outputs(st):
    return (st["topk"].cpu().numpy().copy(),
            None if st["cand"] is None else st["cand"].cpu().numpy().copy())


def test_two_streams_in_flight():
    import torch
    a = small_problem(400, ratio=1, N=64, mode=2, topk=300, cb=64, requests=((4, 5000), (1, 3000)))
    b = small_problem(401, ratio=2, N=32, mode=1, topk=100, requests=((2, 9000), (3, 700)))
    sa, sb = prepared(a), prepared(b)
    cur = torch.cuda.current_stream()
    launch(sa, cur.cuda_stream)
    launch(sb, cur.cuda_stream)
    torch.cuda.synchronize()
    ref_a, ref_b = outputs(sa), outputs(sb)
    s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()  # default priority
    for rep in range(3):
        say(f"two streams, round {rep}")
        sa["topk"].fill_(-7)
        sb["topk"].fill_(-7)
        torch.cuda.synchronize()
        for _ in range(4):  # both streams busy at the same time
            launch(sa, s1.cuda_stream)
            launch(sb, s2.cuda_stream)
        torch.cuda.synchronize()
        ga, gb = outputs(sa), outputs(sb)
        assert np.array_equal(ga[0], ref_a[0]) and np.array_equal(ga[1], ref_a[1])
        assert np.array_equal(gb[0], ref_b[0])


def test_graph_capture_and_replay():
    import torch
    pb = small_problem(402, ratio=1, N=64, mode=2, topk=200, cb=64,
                       requests=((1, 4000), (1, 2500), (1, 6100), (1, 300)))
    st = prepared(pb)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):  # warm up off the default stream, as torch graphs expect
        launch(st, side.cuda_stream)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    ref = outputs(st)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        launch(st, torch.cuda.current_stream().cuda_stream)
    # other queries, same caches: the eager result for them
    q2 = torch.flip(st["dev"]["q"], dims=[1]).contiguous()
    for rep in range(3):
        say(f"graph replay {rep}")
        st["topk"].fill_(-7)
        st["cand"].fill_(-7)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        got = outputs(st)
        assert np.array_equal(got[0], ref[0]) and np.array_equal(got[1], ref[1])
        # eager work between replays: another library call on other outputs
        other = prepared(small_problem(403 + rep, ratio=2, N=32, mode=1, topk=50,
                                       requests=((2, 800),)))
        launch(other, torch.cuda.current_stream().cuda_stream)
        torch.cuda.synchronize()
    # the graph reads the live input buffers: new queries in place change the result
    orig = st["dev"]["q"].clone()
    st["dev"]["q"].copy_(q2)
    torch.cuda.synchronize()
    g.replay()
    torch.cuda.synchronize()
    via_graph = outputs(st)
    launch(st, torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    eager = outputs(st)
    assert np.array_equal(via_graph[0], eager[0]) and np.array_equal(via_graph[1], eager[1])
    assert not np.array_equal(via_graph[0], ref[0])
    st["dev"]["q"].copy_(orig)
    del g
