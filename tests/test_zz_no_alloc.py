"""The entry point that allocates nothing (qli_score_topk_noalloc): its
outputs equal those of qli_score_topk with a caller workspace, bit for bit,
on two calls in a row through the C ABI, the second on a smaller input (the
static scratch keeps the first call's contents), in source and in consumer
mode, and on a call larger than the static array (run in slices)."""
import numpy as np
import pytest

from gpu_check import say, small_problem

pytestmark = pytest.mark.gpu


def _both(pb, cand_in=None):
    """(regular, no-alloc) outputs of one problem, each through the C ABI."""
    import torch

    import quantized_top_indexer_amd as Q
    from qli_workloads.device import call_kwargs, to_device
    dev = to_device(pb, "cuda", cand_in=cand_in)
    kw = call_kwargs(pb, dev)
    outs = []
    for noalloc in (False, True):
        T = pb.num_tokens
        shp_i, shp_c = Q.output_shapes(T, pb.topk, pb.cand_blocks, pb.mode)
        topk = torch.full(shp_i, -7, dtype=torch.int32, device="cuda")
        cand = torch.full(shp_c, -7, dtype=torch.int32, device="cuda") if shp_c else None
        args = {k: v for k, v in kw.items() if k not in ("cand_blocks",)}
        p = Q.make_params(**args, cand_blocks=pb.cand_blocks, topk_out=topk, cand_out=cand)
        if noalloc:
            rc = Q.qli_score_topk_noalloc(p)
            ws = None
        else:
            ws = torch.empty(max(Q.qli_workspace_bytes(p), 256), dtype=torch.uint8, device="cuda")
            p.workspace, p.workspace_bytes = ws.data_ptr(), ws.numel()
            rc = Q.qli_score_topk(p)
        assert rc == Q.QLI_OK, Q.qli_status_string(rc)
        torch.cuda.synchronize()
        outs.append((topk.cpu().numpy(), None if cand is None else cand.cpu().numpy()))
        del ws
    return outs


@pytest.mark.parametrize("mode", [2, 3])
def test_noalloc_matches_workspace_call(mode):
    # first call: 44 decode-like tokens over up to 32768 positions (ratio 1, 64
    # heads); second: fewer tokens and shorter contexts (ratio 2, 32 heads)
    big = small_problem(900 + mode, ratio=1, N=64, mode=mode, topk=2048, cb=512, cb_in=512,
                        requests=tuple((1, 32768 - 97 * i) for i in range(40)) + ((4, 20000),))
    small = small_problem(910 + mode, ratio=2, N=32, mode=mode, topk=100, cb=64, cb_in=128,
                          requests=((3, 3000), (1, 1), (2, 900)))
    for pb in (big, small):
        say(f"no-alloc {pb.name}: T={pb.num_tokens} L={pb.max_k_len} mode={mode}")
        (ti, ci), (tn, cn) = _both(pb)
        assert np.array_equal(ti, tn), pb.name
        assert np.all(tn != -7)
        if mode == 2:
            assert np.array_equal(ci, cn), pb.name


def test_noalloc_slices_a_call_beyond_its_array():
    """A call whose workspace exceeds the 32 MiB static array runs in token
    slices that fit it (4-token groups cut at slice boundaries are scored as
    single tokens): the same outputs as the workspace call."""
    import quantized_top_indexer_amd as Q
    # 1500 tokens of two long requests: 1500 x 6400 key slots x 4 B > 32 MiB
    pb = small_problem(920, ratio=2, N=32, mode=2, topk=300, cb=128,
                       requests=((1000, 12800), (499, 9000), (1, 300)))
    from qli_workloads.device import call_kwargs, to_device
    p = Q.make_params(**{k: v for k, v in call_kwargs(pb, to_device(pb, "cuda")).items()
                         if k != "cand_blocks"}, cand_blocks=pb.cand_blocks)
    assert Q.qli_workspace_bytes(p) > Q.QLI_STATIC_SCRATCH_BYTES
    say(f"no-alloc sliced {pb.name}: T={pb.num_tokens} L={pb.max_k_len}")
    (ti, ci), (tn, cn) = _both(pb)
    assert np.array_equal(ti, tn)
    assert np.array_equal(ci, cn)

