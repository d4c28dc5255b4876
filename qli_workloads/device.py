"""Upload a generated problem to the GPU in the cache layout the indexer reads.

The device pool is one uint8 tensor [num_pages, page_stride_bytes] per layer
call.  It is first poisoned (K byte 127, scale 60000.0 = 0x7B53, KV region
0x7F) and the index K and scale rows are then copied into their regions of
each page, giving strided int8 / fp16 views whose leading (page) stride is
the real page size.  No indexer arithmetic happens here.
"""
from __future__ import annotations

import numpy as np
import torch

from . import page_layout


def device_pool(pb, device="cuda", page_stride=None, k_offset=None, s_offset=None):
    """(pool, k_view [P, R, 128] int8, s_view [P, R] int16) on ``device``.

    The stride and offsets default to the ratio's real layout; other values
    (e.g. a larger stride) describe the same cache at another placement.
    """
    R, stride, koff, soff = page_layout(pb.ratio)
    stride = page_stride or stride
    koff = koff if k_offset is None else k_offset
    soff = soff if s_offset is None else s_offset
    P = pb.num_pages
    pool = torch.full((P, stride), 0x7F, dtype=torch.uint8, device=device)
    kview = pool[:, koff:koff + R * 128].view(torch.int8).view(P, R, 128)
    sview = pool[:, soff:soff + R * 2].view(torch.int16)
    kview.copy_(torch.from_numpy(pb.k_pages))
    sview.copy_(torch.from_numpy(pb.s_pages.view(np.int16)))
    return pool, kview, sview


def to_device(pb, device="cuda", cand_in=None, **layout):
    """Every tensor of one call, on ``device``."""
    def t(a, dt):
        return None if a is None else torch.from_numpy(np.ascontiguousarray(a)).to(
            device=device, dtype=dt)

    pool, kview, sview = device_pool(pb, device, **layout)
    cand = cand_in if cand_in is not None else pb.cand_in
    return {
        "pool": pool,
        "k_cache": kview,
        "k_scale": sview,
        "q": t(pb.q, torch.int8),
        "q_scale": t(pb.q_scale.view(np.int16), torch.int16),
        "weights": t(pb.weights.view(np.int16), torch.int16),
        "block_table": t(pb.block_table, torch.int32),
        "query_start_loc": t(pb.query_start_loc, torch.int32),
        "k_lens": t(pb.k_lens, torch.int32),
        "seq_mod": t(pb.seq_mod, torch.int32),
        "cand_in": cand if isinstance(cand, torch.Tensor) else t(cand, torch.int32),
    }


def call_kwargs(pb, dev):
    """Keyword arguments of quantized_top_indexer_amd.score_topk for one call."""
    keys = ("q", "q_scale", "weights", "k_cache", "k_scale", "block_table", "query_start_loc",
            "k_lens", "seq_mod", "cand_in")
    kw = {k: dev[k] for k in keys}
    kw.update(ratio=pb.ratio, mode=pb.mode, topk=pb.topk, cand_blocks=pb.cand_blocks,
              max_k_len=pb.max_k_len)
    return kw
