"""Python binding of the MI355X quantized lightning indexer (QLI) library.

Thin ctypes layer over ``libqli.so`` (C ABI in ``include/qli.h``): it only
marshals torch tensors into ``qli_params`` and calls the library; every step
of the indexer runs in the HIP kernels.  There is no fallback: if the
library is not built, importing the entry points raises.

Entry points (same names as the C ABI): ``qli_score_topk``,
``qli_score_topk_noalloc``, ``qli_workspace_bytes``, ``qli_validate``, ``qli_status_string``,
``qli_abi_version``, ``qli_quantize_query``, ``qli_write_index_k``,
``qli_sparse_attention`` (``qli_attn_workspace_bytes`` through the loaded
library); plus ``score_topk``, ``quantize_query``, ``write_index_k`` and
``sparse_attention``, convenience wrappers that allocate the outputs (and
the workspace) with torch and run one call on the current stream, and
``output_shapes`` (shapes of a call's outputs).
"""
from __future__ import annotations

import ctypes as C
import math
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libqli.so")

QLI_OK, QLI_ERR_INVALID_ARG, QLI_ERR_UNSUPPORTED, QLI_ERR_NO_SOURCE, QLI_ERR_WORKSPACE, \
    QLI_ERR_HIP, QLI_ERR_SCRATCH_LIMIT = range(7)
QLI_STATIC_SCRATCH_BYTES = 32 << 20
QLI_MODE_PLAIN, QLI_MODE_SOURCE, QLI_MODE_CONSUMER = 1, 2, 3
QLI_QUANT_INT8 = 2
QLI_DEV_BAD_PAGE, QLI_DEV_BAD_LENGTH, QLI_DEV_BAD_METADATA = 1, 2, 4


class qli_params(C.Structure):
    """Mirror of ``struct qli_params`` in include/qli.h."""
    _fields_ = [
        ("struct_size", C.c_uint32), ("mode", C.c_int32), ("ratio", C.c_int32),
        ("num_heads", C.c_int32), ("head_dim", C.c_int32), ("quant_mode", C.c_int32),
        ("batch", C.c_int32), ("num_tokens", C.c_int32), ("topk", C.c_int32),
        ("cand_blocks", C.c_int32), ("cand_in_blocks", C.c_int32), ("page_rows", C.c_int32),
        ("bt_stride", C.c_int32), ("num_pages", C.c_int32), ("max_k_len", C.c_int32),
        ("reserved0", C.c_int32),
        ("k_page_stride", C.c_int64), ("s_page_stride", C.c_int64),
        ("q", C.c_void_p), ("q_scale", C.c_void_p), ("weights", C.c_void_p),
        ("k_cache", C.c_void_p), ("k_scale", C.c_void_p), ("block_table", C.c_void_p),
        ("query_start_loc", C.c_void_p), ("k_lens", C.c_void_p), ("seq_mod", C.c_void_p),
        ("cand_in", C.c_void_p),
        ("topk_out", C.c_void_p), ("cand_out", C.c_void_p), ("dbg_scores", C.c_void_p),
        ("dbg_qk", C.c_void_p), ("status_out", C.c_void_p),
        ("workspace", C.c_void_p), ("workspace_bytes", C.c_size_t),
    ]


QLI_DTYPE_F32, QLI_DTYPE_BF16 = 0, 1


class qli_quant_params(C.Structure):
    """Mirror of ``struct qli_quant_params`` in include/qli.h."""
    _fields_ = [
        ("struct_size", C.c_int32), ("num_rows", C.c_int32), ("head_dim", C.c_int32),
        ("x_dtype", C.c_int32), ("num_weights", C.c_int32), ("w_dtype", C.c_int32),
        ("x", C.c_void_p), ("q", C.c_void_p), ("q_scale", C.c_void_p),
        ("w", C.c_void_p), ("w_out", C.c_void_p),
    ]


class qli_kwrite_params(C.Structure):
    """Mirror of ``struct qli_kwrite_params`` in include/qli.h."""
    _fields_ = [
        ("struct_size", C.c_int32), ("num_rows", C.c_int32), ("head_dim", C.c_int32),
        ("x_dtype", C.c_int32), ("page_rows", C.c_int32), ("reserved0", C.c_int32),
        ("num_pages", C.c_int64), ("k_page_stride", C.c_int64), ("s_page_stride", C.c_int64),
        ("x", C.c_void_p), ("slot", C.c_void_p), ("k_cache", C.c_void_p),
        ("k_scale", C.c_void_p), ("status_out", C.c_void_p),
    ]


class qli_attn_params(C.Structure):
    """Mirror of ``struct qli_attn_params`` in include/qli.h."""
    _fields_ = [
        ("struct_size", C.c_int32), ("num_heads", C.c_int32), ("head_dim", C.c_int32),
        ("batch", C.c_int32), ("num_tokens", C.c_int32), ("topk", C.c_int32),
        ("window", C.c_int32), ("c_page_rows", C.c_int32), ("c_bt_stride", C.c_int32),
        ("r_page_rows", C.c_int32), ("r_bt_stride", C.c_int32), ("reserved0", C.c_int32),
        ("c_num_pages", C.c_int64), ("r_num_pages", C.c_int64),
        ("c_page_stride", C.c_int64), ("r_page_stride", C.c_int64),
        ("scale", C.c_float), ("reserved1", C.c_int32),
        ("q", C.c_void_p), ("c_cache", C.c_void_p), ("c_block_table", C.c_void_p),
        ("c_lens", C.c_void_p), ("r_cache", C.c_void_p), ("r_block_table", C.c_void_p),
        ("r_lens", C.c_void_p), ("query_start_loc", C.c_void_p), ("indices", C.c_void_p),
        ("sinks", C.c_void_p), ("out", C.c_void_p), ("lse", C.c_void_p),
        ("status_out", C.c_void_p), ("workspace", C.c_void_p), ("workspace_bytes", C.c_int64),
    ]


EXPORTS = ("qli_abi_version", "qli_validate", "qli_workspace_bytes", "qli_score_topk",
           "qli_score_topk_noalloc", "qli_status_string", "qli_timing_enable", "qli_timing_read",
           "qli_quantize_query", "qli_write_index_k", "qli_sparse_attention",
           "qli_attn_workspace_bytes")
# the ceiling probes (include/qli_probe.h): a library of their own, for
# measurement only
PROBE_LIB_PATH = os.path.join(_HERE, "libqli_probe.so")
PROBE_EXPORTS = ("qli_probe_hbm_read", "qli_probe_int8_mfma", "qli_probe_int8_mfma_ops")
QLI_KERNEL_CONSUMER_PREP, QLI_KERNEL_PLAN, QLI_KERNEL_SCORE, QLI_KERNEL_SELECT, \
    QLI_KERNEL_QUANTIZE, QLI_KERNEL_WRITE_K, QLI_KERNEL_ATTN, QLI_KERNEL_ATTN_SPLIT, \
    QLI_KERNEL_ATTN_MERGE, QLI_NUM_KERNELS = range(10)
KERNEL_NAMES = ("consumer_prep_kernel", "plan_kernel", "score_kernel", "select_kernel",
                "quantize_kernel", "write_k_kernel", "sparse_attn_kernel", "sparse_attn_split_kernel",
                "sparse_attn_merge_kernel")
QLI_ABI_VERSION = 6

_lib = None


def load_library(path: str = LIB_PATH):
    """Load libqli.so (raises if it has not been built)."""
    global _lib
    if _lib is not None and path == LIB_PATH:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(f"QLI HIP library not built ({path}); run __graft_entry__.build()")
    # torch bundles its own HIP runtime, whose file name differs from the
    # soname this library asks for: if this library were loaded first, the
    # process would end up with two runtimes, and torch's streams and device
    # memory would be foreign to ours.  Loading torch first makes the dynamic
    # linker resolve our dependency to torch's (already loaded) runtime.
    import torch  # noqa: F401
    L = C.CDLL(path)
    L.qli_abi_version.restype = C.c_int
    L.qli_validate.restype = C.c_int
    L.qli_validate.argtypes = [C.POINTER(qli_params)]
    L.qli_workspace_bytes.restype = C.c_size_t
    L.qli_workspace_bytes.argtypes = [C.POINTER(qli_params)]
    L.qli_score_topk.restype = C.c_int
    L.qli_score_topk.argtypes = [C.POINTER(qli_params), C.c_void_p]
    L.qli_score_topk_noalloc.restype = C.c_int
    L.qli_score_topk_noalloc.argtypes = [C.POINTER(qli_params), C.c_void_p]
    L.qli_status_string.restype = C.c_char_p
    L.qli_status_string.argtypes = [C.c_int]
    L.qli_timing_enable.restype = C.c_int
    L.qli_timing_enable.argtypes = [C.c_int]
    L.qli_timing_read.restype = C.c_int
    L.qli_timing_read.argtypes = [C.c_void_p, C.c_void_p, C.c_int]
    L.qli_quantize_query.restype = C.c_int
    L.qli_quantize_query.argtypes = [C.POINTER(qli_quant_params), C.c_void_p]
    L.qli_write_index_k.restype = C.c_int
    L.qli_write_index_k.argtypes = [C.POINTER(qli_kwrite_params), C.c_void_p]
    L.qli_sparse_attention.restype = C.c_int
    L.qli_sparse_attention.argtypes = [C.POINTER(qli_attn_params), C.c_void_p]
    L.qli_attn_workspace_bytes.restype = C.c_int64
    L.qli_attn_workspace_bytes.argtypes = [C.POINTER(qli_attn_params)]
    if path == LIB_PATH:
        _lib = L
    return L


_probe_lib = None


def load_probe_library():
    """Load libqli_probe.so, the measured-ceiling probes (raises if not built)."""
    global _probe_lib
    if _probe_lib is None:
        if not os.path.exists(PROBE_LIB_PATH):
            raise RuntimeError(f"probe library not built ({PROBE_LIB_PATH}); run __graft_entry__.build()")
        import torch  # noqa: F401  (one HIP runtime: torch's)
        L = C.CDLL(PROBE_LIB_PATH)
        L.qli_probe_hbm_read.restype = C.c_int
        L.qli_probe_hbm_read.argtypes = [C.c_void_p, C.c_size_t, C.c_int, C.c_void_p, C.c_void_p]
        L.qli_probe_int8_mfma.restype = C.c_int
        L.qli_probe_int8_mfma.argtypes = [C.c_int, C.c_int, C.c_void_p, C.c_void_p]
        L.qli_probe_int8_mfma_ops.restype = C.c_double
        L.qli_probe_int8_mfma_ops.argtypes = [C.c_int, C.c_int]
        _probe_lib = L
    return _probe_lib


def qli_abi_version() -> int:
    return load_library().qli_abi_version()


def qli_validate(p: qli_params) -> int:
    return load_library().qli_validate(C.byref(p))


def qli_workspace_bytes(p: qli_params) -> int:
    return load_library().qli_workspace_bytes(C.byref(p))


def qli_score_topk(p: qli_params, stream=None) -> int:
    """Enqueue one call on ``stream`` (a raw hipStream_t handle as int, or
    None for torch's current stream)."""
    if stream is None:
        import torch
        stream = torch.cuda.current_stream().cuda_stream
    return load_library().qli_score_topk(C.byref(p), C.c_void_p(stream))


def qli_score_topk_noalloc(p: qli_params, stream=None) -> int:
    """Enqueue one call with the library's static scratch instead of a
    workspace (p.workspace is ignored); see include/qli.h."""
    return load_library().qli_score_topk_noalloc(C.byref(p), _stream(stream))


def _stream(stream):
    if stream is None:
        import torch
        stream = torch.cuda.current_stream().cuda_stream
    return C.c_void_p(stream)


def qli_quantize_query(p: qli_quant_params, stream=None) -> int:
    """Enqueue query quantization + weight rounding on ``stream``."""
    return load_library().qli_quantize_query(C.byref(p), _stream(stream))


def qli_write_index_k(p: qli_kwrite_params, stream=None) -> int:
    """Enqueue the quantization and paged scatter of new index-K rows."""
    return load_library().qli_write_index_k(C.byref(p), _stream(stream))


def qli_probe_hbm_read(buf, nbytes: int, grid: int, sink, stream=None) -> int:
    """Enqueue the streaming-read ceiling probe (include/qli_probe.h)."""
    return load_probe_library().qli_probe_hbm_read(C.c_void_p(buf), C.c_size_t(nbytes), grid,
                                             C.c_void_p(sink), _stream(stream))


def qli_probe_int8_mfma(grid: int, iterations: int, sink, stream=None) -> int:
    """Enqueue the INT8 MFMA ceiling probe (include/qli_probe.h)."""
    return load_probe_library().qli_probe_int8_mfma(grid, iterations, C.c_void_p(sink),
                                                    _stream(stream))


def qli_probe_int8_mfma_ops(grid: int, iterations: int) -> float:
    return load_probe_library().qli_probe_int8_mfma_ops(grid, iterations)


def _dtype_code(t):
    import torch
    if t.dtype == torch.float32:
        return QLI_DTYPE_F32
    if t.dtype == torch.bfloat16:
        return QLI_DTYPE_BF16
    raise ValueError(f"unsupported dtype {t.dtype} (float32 or bfloat16)")


def quantize_query(x, weights=None, *, q=None, q_scale=None, w_out=None, stream=None):
    """Quantize query heads x [..., 128] (float32 or bfloat16, contiguous) to
    INT8 with one FP16 scale per head, and round ``weights`` to FP16.

    Returns ``(q int8 [..., 128], q_scale fp16 [...], weights fp16 or None)``;
    outputs are allocated with torch unless given.
    """
    import torch
    if x.shape[-1] != 128 or not x.is_contiguous():
        raise ValueError("x must be contiguous with a last dimension of 128")
    lead = x.shape[:-1]
    rows = x.numel() // 128
    if q is None:
        q = torch.empty(x.shape, dtype=torch.int8, device=x.device)
    if q_scale is None:
        q_scale = torch.empty(lead, dtype=torch.float16, device=x.device)
    p = qli_quant_params()
    p.struct_size = C.sizeof(qli_quant_params)
    p.num_rows, p.head_dim, p.x_dtype = rows, 128, _dtype_code(x)
    p.x, p.q, p.q_scale = x.data_ptr(), q.data_ptr(), q_scale.data_ptr()
    p.w_dtype = QLI_DTYPE_F32
    if weights is not None:
        if not weights.is_contiguous():
            raise ValueError("weights must be contiguous")
        if w_out is None:
            w_out = torch.empty(weights.shape, dtype=torch.float16, device=weights.device)
        p.num_weights, p.w_dtype = weights.numel(), _dtype_code(weights)
        p.w, p.w_out = weights.data_ptr(), w_out.data_ptr()
    rc = qli_quantize_query(p, stream)
    if rc != QLI_OK:
        raise RuntimeError(qli_status_string(rc))
    return q, q_scale, w_out


def write_index_k(x, slot, k_cache, k_scale, *, status_out=None, stream=None):
    """Quantize new index-K rows x [rows, 128] (float32 or bfloat16) and
    scatter them into the paged cache: k_cache is an int8 view
    [num_pages, page_rows, 128] (rows of 128 contiguous bytes, any page
    stride), k_scale an fp16 view [num_pages, page_rows] (any page stride);
    slot int64 [rows] holds page * page_rows + row, negative to skip."""
    if x.shape[-1] != 128 or x.dim() != 2 or not x.is_contiguous():
        raise ValueError("x must be a contiguous [rows, 128] tensor")
    if k_cache.stride(1) != 128 or k_cache.stride(2) != 1 or k_scale.stride(1) != 1:
        raise ValueError("k_cache rows must be 128 contiguous bytes, k_scale rows 2 bytes")
    p = qli_kwrite_params()
    p.struct_size = C.sizeof(qli_kwrite_params)
    p.num_rows, p.head_dim, p.x_dtype = x.shape[0], 128, _dtype_code(x)
    p.page_rows, p.num_pages = k_cache.shape[1], k_cache.shape[0]
    p.k_page_stride = k_cache.stride(0) * k_cache.element_size()
    p.s_page_stride = k_scale.stride(0) * k_scale.element_size()
    p.x, p.slot = x.data_ptr(), slot.data_ptr()
    p.k_cache, p.k_scale = k_cache.data_ptr(), k_scale.data_ptr()
    p.status_out = _ptr(status_out)
    rc = qli_write_index_k(p, stream)
    if rc != QLI_OK:
        raise RuntimeError(qli_status_string(rc))


def qli_sparse_attention(p: qli_attn_params, stream=None) -> int:
    """Raw C-ABI call (see include/qli.h)."""
    return load_library().qli_sparse_attention(C.byref(p), _stream(stream))


_attn_ws = {}


def attention_workspace(nbytes: int, device):
    """The cached attention workspace of `device` with at least nbytes (None
    for nbytes == 0).  Calls that use it must be ordered on one stream."""
    import torch
    if nbytes <= 0:
        return None
    key = str(device)
    ws = _attn_ws.get(key)
    if ws is None or ws.numel() < nbytes:
        ws = torch.empty(nbytes, dtype=torch.uint8, device=device)
        _attn_ws[key] = ws
    return ws


def sparse_attention(q, c_cache, c_block_table, c_lens, query_start_loc, *, indices=None,
                     r_cache=None, r_block_table=None, r_lens=None, window=0, sinks=None,
                     scale=None, c_page_rows, c_page_stride, r_page_rows=0, r_page_stride=0,
                     c_num_pages, r_num_pages=0, out=None, lse=None, status_out=None, stream=None,
                     workspace="auto"):
    """Sparse attention over the indexer's positions (argument marshalling
    for qli_sparse_attention): q bfloat16 [T, H, 512]; c_cache / r_cache
    device buffers of BF16 rows paged as described in include/qli.h (any
    tensor, passed by address with the page geometry given explicitly);
    block tables int32 [B, stride]; lengths int32 [B]; query_start_loc
    int32 [B + 1]; indices int32 [T, topk] or None; sinks float32 [H] or
    None.  workspace: a uint8 device tensor (any contents), None for no
    split, or "auto" for one cached per device, grown as calls need it;
    calls sharing a workspace must be ordered on one stream.  Returns
    (out bfloat16 [T, H, 512], lse float32 [T, H] or None)."""
    import torch
    T, H, D = q.shape
    if out is None:
        out = torch.empty((T, H, D), dtype=torch.bfloat16, device=q.device)
    p = qli_attn_params()
    p.struct_size = C.sizeof(qli_attn_params)
    p.num_heads, p.head_dim, p.batch, p.num_tokens = H, D, c_lens.shape[0], T
    p.topk = 0 if indices is None else indices.shape[1]
    p.window = window
    p.c_page_rows, p.c_bt_stride = c_page_rows, c_block_table.shape[1]
    p.c_num_pages, p.c_page_stride = c_num_pages, c_page_stride
    if window > 0:
        p.r_page_rows, p.r_bt_stride = r_page_rows, r_block_table.shape[1]
        p.r_num_pages, p.r_page_stride = r_num_pages, r_page_stride
    p.scale = float(1.0 / math.sqrt(D) if scale is None else scale)
    p.q, p.c_cache, p.c_block_table = q.data_ptr(), c_cache.data_ptr(), c_block_table.data_ptr()
    p.c_lens, p.query_start_loc = c_lens.data_ptr(), query_start_loc.data_ptr()
    p.r_cache, p.r_block_table, p.r_lens = _ptr(r_cache), _ptr(r_block_table), _ptr(r_lens)
    p.indices, p.sinks = _ptr(indices), _ptr(sinks)
    p.out, p.lse, p.status_out = out.data_ptr(), _ptr(lse), _ptr(status_out)
    if isinstance(workspace, str) and workspace == "auto":
        workspace = attention_workspace(load_library().qli_attn_workspace_bytes(C.byref(p)), q.device)
    if workspace is not None:
        p.workspace, p.workspace_bytes = workspace.data_ptr(), workspace.numel() * workspace.element_size()
    rc = qli_sparse_attention(p, stream)
    if rc != QLI_OK:
        raise RuntimeError(qli_status_string(rc))
    return out, lse


def qli_status_string(code: int) -> str:
    return load_library().qli_status_string(code).decode()


def qli_timing_enable(on: bool) -> int:
    return load_library().qli_timing_enable(1 if on else 0)


def qli_timing_read(reset: bool = True):
    """(ms per kernel, launches per kernel) accumulated by the timing facility."""
    ms = (C.c_double * QLI_NUM_KERNELS)()
    cnt = (C.c_int64 * QLI_NUM_KERNELS)()
    rc = load_library().qli_timing_read(ms, cnt, 1 if reset else 0)
    if rc != QLI_OK:
        raise RuntimeError(qli_status_string(rc))
    return list(ms), list(cnt)


def new_params() -> qli_params:
    p = qli_params()
    p.struct_size = C.sizeof(qli_params)
    p.head_dim = 128
    p.quant_mode = QLI_QUANT_INT8
    return p


def output_shapes(num_tokens: int, topk: int, cand_blocks: int, mode: int):
    """Shapes of (indices, candidates) for a call; candidates only in source mode."""
    return (num_tokens, 1, topk), ((num_tokens, 1, cand_blocks) if mode == QLI_MODE_SOURCE
                                   else None)


def _ptr(t):
    return None if t is None else t.data_ptr()


def make_params(*, q, q_scale, weights, k_cache, k_scale, block_table, query_start_loc, k_lens,
                seq_mod=None, cand_in=None, ratio, mode, topk, cand_blocks=0, max_k_len,
                topk_out=None, cand_out=None, dbg_scores=None, dbg_qk=None, status_out=None,
                workspace=None):
    """Fill qli_params from torch tensors.

    k_cache: int8 view [num_pages, page_rows, 128] of the paged index K (row
    stride 128 bytes, any page stride); k_scale: fp16/int16 view
    [num_pages, page_rows] (row stride 2 bytes, any page stride).  The page
    strides are taken from the views, as given.
    """
    p = new_params()
    T, N, D = q.shape
    p.mode, p.ratio, p.num_heads, p.head_dim = mode, ratio, N, D
    p.batch = k_lens.shape[0]
    p.num_tokens = T
    p.topk = topk
    p.cand_blocks = cand_blocks
    p.cand_in_blocks = cand_in.shape[-1] if cand_in is not None else 0
    p.page_rows = k_cache.shape[1]
    p.bt_stride = block_table.shape[1]
    p.num_pages = k_cache.shape[0]
    p.max_k_len = max_k_len
    if k_cache.stride(1) != 128 or k_cache.stride(2) != 1 or k_scale.stride(1) != 1:
        raise ValueError("k_cache rows must be 128 contiguous bytes, k_scale rows 2 bytes")
    p.k_page_stride = k_cache.stride(0) * k_cache.element_size()
    p.s_page_stride = k_scale.stride(0) * k_scale.element_size()
    p.q, p.q_scale, p.weights = _ptr(q), _ptr(q_scale), _ptr(weights)
    p.k_cache, p.k_scale = _ptr(k_cache), _ptr(k_scale)
    p.block_table, p.query_start_loc, p.k_lens = _ptr(block_table), _ptr(query_start_loc), \
        _ptr(k_lens)
    p.seq_mod, p.cand_in = _ptr(seq_mod), _ptr(cand_in)
    p.topk_out, p.cand_out = _ptr(topk_out), _ptr(cand_out)
    p.dbg_scores, p.dbg_qk, p.status_out = _ptr(dbg_scores), _ptr(dbg_qk), _ptr(status_out)
    if workspace is not None:
        p.workspace, p.workspace_bytes = _ptr(workspace), workspace.numel()
    return p


def score_topk(*, q, q_scale, weights, k_cache, k_scale, block_table, query_start_loc, k_lens,
               seq_mod=None, cand_in=None, ratio, mode, topk, cand_blocks=0, max_k_len,
               debug_scores=False, dbg_qk=None, status_out=None, workspace=None, stream=None):
    """One indexer call on torch device tensors.

    Returns ``(indices [T,1,topk] int32, candidates [T,1,cb] int32 or None,
    dbg_scores [T, max_k_len] float32 or None)``.  ``dbg_qk`` (optional, with
    ``debug_scores``): an int32 tensor [T, N, max_k_len] that receives the
    exact q.k of every eligible (token, head, position).  Raises RuntimeError
    with the library's status string on a rejected call.
    """
    import torch
    dev = q.device
    T = q.shape[0]
    shp_i, shp_c = output_shapes(T, topk, cand_blocks, mode)
    topk_out = torch.empty(shp_i, dtype=torch.int32, device=dev)
    cand_out = torch.empty(shp_c, dtype=torch.int32, device=dev) if shp_c else None
    dbg = None
    if debug_scores:
        dbg = torch.full((T, max(max_k_len, 1)), float("nan"), dtype=torch.float32, device=dev)
    p = make_params(q=q, q_scale=q_scale, weights=weights, k_cache=k_cache, k_scale=k_scale,
                    block_table=block_table, query_start_loc=query_start_loc, k_lens=k_lens,
                    seq_mod=seq_mod, cand_in=cand_in, ratio=ratio, mode=mode, topk=topk,
                    cand_blocks=cand_blocks, max_k_len=max_k_len, topk_out=topk_out,
                    cand_out=cand_out, dbg_scores=dbg, dbg_qk=dbg_qk, status_out=status_out)
    need = qli_workspace_bytes(p)
    if workspace is None or workspace.numel() < need:
        workspace = torch.empty(max(need, 256), dtype=torch.uint8, device=dev)
    p.workspace, p.workspace_bytes = workspace.data_ptr(), workspace.numel()
    rc = qli_score_topk(p, stream)
    if rc != QLI_OK:
        raise RuntimeError(qli_status_string(rc))
    return topk_out, cand_out, dbg
