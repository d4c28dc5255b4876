"""ctypes front end of the CPU oracle (``qli_oracle.c``).

TEST INFRASTRUCTURE ONLY: imported by the tests, by the smoke check and by
the CPU-baseline leg of the benchmark.  The GPU library never loads it.
"""
from __future__ import annotations

import ctypes as C
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "qli_oracle.c")
_SRC_QUANT = os.path.join(_HERE, "qli_quant_oracle.c")
_SRC_ATTN = os.path.join(_HERE, "qli_attn_oracle.c")
_LIB = os.path.join(_HERE, "libqli_oracle.so")
# an alternative build (used by the tests that plant mistakes in a copy)
_LOAD = os.environ.get("QLI_ORACLE_LIB", _LIB)
CFLAGS = ["-O2", "-std=c11", "-D_GNU_SOURCE", "-ffp-contract=off", "-fno-fast-math",
          "-fexcess-precision=standard", "-fPIC", "-shared", "-pthread"]


def build(force: bool = True) -> str:
    """Compile the oracle with gcc (no GPU toolchain involved)."""
    if force or not os.path.exists(_LIB):
        tmp = _LIB + ".tmp"
        subprocess.run(["gcc", *CFLAGS, _SRC, _SRC_QUANT, _SRC_ATTN, "-o", tmp, "-lm"], check=True)
        os.replace(tmp, _LIB)
    return _LIB


class _Problem(C.Structure):
    _fields_ = [
        ("mode", C.c_int32), ("ratio", C.c_int32), ("num_heads", C.c_int32),
        ("batch", C.c_int32), ("num_tokens", C.c_int32), ("topk", C.c_int32),
        ("cand_blocks", C.c_int32), ("cand_in_blocks", C.c_int32),
        ("page_rows", C.c_int32), ("bt_stride", C.c_int32), ("num_pages", C.c_int32),
        ("pad0", C.c_int32),
        ("k_page_stride", C.c_int64), ("s_page_stride", C.c_int64),
        ("q", C.c_void_p), ("q_scale", C.c_void_p), ("weights", C.c_void_p),
        ("k_base", C.c_void_p), ("s_base", C.c_void_p),
        ("block_table", C.c_void_p), ("query_start_loc", C.c_void_p),
        ("k_lens", C.c_void_p), ("seq_mod", C.c_void_p), ("cand_in", C.c_void_p),
    ]


class _Terms(C.Structure):
    _fields_ = [("qk", C.c_int32 * 256), ("x", C.c_uint16 * 256), ("m", C.c_uint16 * 256),
                ("p", C.c_uint16 * 256), ("score", C.c_float), ("sum", C.c_float),
                ("exact_sum_q24", C.c_int64), ("abs_sum", C.c_double)]


_lib = None


def lib():
    global _lib
    if _lib is None:
        if _LOAD == _LIB and not os.path.exists(_LIB):
            build()
        L = C.CDLL(_LOAD)
        L.oracle_f16_round.restype = C.c_uint16
        L.oracle_f16_round.argtypes = [C.c_double]
        L.oracle_f16_value.restype = C.c_double
        L.oracle_f16_value.argtypes = [C.c_uint16]
        L.oracle_f16_round_array.argtypes = [C.c_void_p, C.c_void_p, C.c_int64]
        L.oracle_f16_value_array.argtypes = [C.c_void_p, C.c_void_p, C.c_int64]
        L.oracle_token_view.argtypes = [C.POINTER(_Problem), C.c_int, C.POINTER(C.c_int),
                                        C.POINTER(C.c_int)]
        L.oracle_score_terms.argtypes = [C.POINTER(_Problem), C.c_int, C.c_int,
                                         C.POINTER(_Terms)]
        L.oracle_run.argtypes = [C.POINTER(_Problem), C.c_void_p, C.c_int, C.c_void_p,
                                 C.c_void_p, C.c_void_p, C.c_int, C.c_int]
        _lib = L
    return _lib


def _ptr(a):
    return None if a is None else a.ctypes.data


class OracleProblem:
    """Holds contiguous host copies and the C struct for one problem."""

    def __init__(self, pb, cand_in=None):
        self.pb = pb
        self._keep = []

        def keep(a, dt):
            if a is None:
                return None
            a = np.ascontiguousarray(a, dtype=dt)
            self._keep.append(a)
            return a

        R = pb.page_rows
        cand = cand_in if cand_in is not None else pb.cand_in
        cand = keep(cand, np.int32)
        s = _Problem()
        s.mode, s.ratio, s.num_heads = pb.mode, pb.ratio, pb.num_heads
        s.batch, s.num_tokens, s.topk = pb.batch, pb.num_tokens, pb.topk
        s.cand_blocks, s.cand_in_blocks = pb.cand_blocks, pb.cand_in_blocks
        s.page_rows, s.bt_stride = R, pb.block_table.shape[1]
        s.num_pages = pb.num_pages
        s.k_page_stride = R * 128
        s.s_page_stride = R * 2
        s.q = _ptr(keep(pb.q, np.int8))
        s.q_scale = _ptr(keep(pb.q_scale, np.uint16))
        s.weights = _ptr(keep(pb.weights, np.uint16))
        s.k_base = _ptr(keep(pb.k_pages, np.int8))
        s.s_base = _ptr(keep(pb.s_pages, np.uint16))
        s.block_table = _ptr(keep(pb.block_table, np.int32))
        s.query_start_loc = _ptr(keep(pb.query_start_loc, np.int32))
        s.k_lens = _ptr(keep(pb.k_lens, np.int32))
        s.seq_mod = _ptr(keep(pb.seq_mod, np.int32))
        s.cand_in = _ptr(cand)
        self.s = s

    def run(self, tokens=None, want_scores=False, score_cols=None, nthreads=None):
        pb = self.pb
        if tokens is None:
            tok = None
            n = pb.num_tokens
        else:
            tok = np.ascontiguousarray(tokens, dtype=np.int32)
            n = len(tok)
        topk = np.full((n, pb.topk), -9, np.int32)
        cand = np.full((n, pb.cand_blocks), -9, np.int32) if pb.mode == 2 else None
        cols = score_cols if score_cols is not None else max(pb.max_k_len, 1)
        scores = np.empty((n, cols), np.float32) if want_scores else None
        if nthreads is None:
            nthreads = min(os.cpu_count() or 1, 16)
        rc = lib().oracle_run(C.byref(self.s), _ptr(tok), n, _ptr(topk), _ptr(cand),
                              _ptr(scores), cols, nthreads)
        if rc:
            raise RuntimeError(f"oracle_run failed with {rc}")
        return {"topk": topk, "cand": cand, "scores": scores}

    def token_view(self, t):
        b, V = C.c_int(), C.c_int()
        if lib().oracle_token_view(C.byref(self.s), t, C.byref(b), C.byref(V)):
            raise RuntimeError("inconsistent metadata")
        return b.value, V.value

    def terms(self, t, j):
        out = _Terms()
        if lib().oracle_score_terms(C.byref(self.s), t, j, C.byref(out)):
            raise RuntimeError("oracle_score_terms failed")
        N = self.pb.num_heads
        return {"qk": np.array(out.qk[:N]), "x": np.array(out.x[:N], np.uint16),
                "m": np.array(out.m[:N], np.uint16), "p": np.array(out.p[:N], np.uint16),
                "score": np.float32(out.score), "sum": np.float32(out.sum),
                "exact_sum_q24": out.exact_sum_q24, "abs_sum": out.abs_sum}


def run(pb, tokens=None, want_scores=False, cand_in=None, nthreads=None, score_cols=None):
    return OracleProblem(pb, cand_in).run(tokens, want_scores, score_cols, nthreads)


def f16_round(x):
    x = np.ascontiguousarray(x, dtype=np.float64)
    out = np.empty(x.shape, np.uint16)
    lib().oracle_f16_round_array(x.ctypes.data, out.ctypes.data, x.size)
    return out


def f16_value(h):
    h = np.ascontiguousarray(h, dtype=np.uint16)
    out = np.empty(h.shape, np.float64)
    lib().oracle_f16_value_array(h.ctypes.data, out.ctypes.data, h.size)
    return out


# ---- query quantization and index-K cache write (qli_quant_oracle.c) ----

DTYPE_F32, DTYPE_BF16 = 0, 1


def _dtype_code(a):
    if a.dtype == np.float32:
        return DTYPE_F32
    if a.dtype == np.uint16:  # bfloat16 bit patterns
        return DTYPE_BF16
    raise TypeError("rows must be float32 or bfloat16 bits (uint16)")


def quantize_rows(x):
    """Symmetric INT8 quantization of rows of 128 values with an FP16 scale.
    x: float32 or bfloat16 bits (uint16), shape [..., 128].  Returns
    (q int8 [..., 128], scale fp16 bits uint16 [...])."""
    x = np.ascontiguousarray(x)
    assert x.shape[-1] == 128
    rows = int(np.prod(x.shape[:-1], dtype=np.int64))
    q = np.zeros(x.shape, np.int8)
    sc = np.zeros(x.shape[:-1], np.uint16)
    L = lib()
    L.oracle_quantize_rows.restype = None
    L.oracle_quantize_rows.argtypes = [C.c_void_p, C.c_int, C.c_int64, C.c_void_p, C.c_void_p]
    L.oracle_quantize_rows(_ptr(x), C.c_int(_dtype_code(x)), C.c_int64(rows), _ptr(q), _ptr(sc))
    return q, sc


def round_weights(w):
    """FP16 (RNE) bits of float32 or bfloat16-bit values."""
    w = np.ascontiguousarray(w)
    out = np.zeros(w.shape, np.uint16)
    L = lib()
    L.oracle_round_weights.restype = None
    L.oracle_round_weights.argtypes = [C.c_void_p, C.c_int, C.c_int64, C.c_void_p]
    L.oracle_round_weights(_ptr(w), C.c_int(_dtype_code(w)), C.c_int64(w.size), _ptr(out))
    return out


def write_k(x, slot, kpages, spages):
    """Quantize K rows x [M, 128] and scatter them into copies of the compact
    pool (kpages [P, R, 128] int8, spages [P, R] fp16 bits) at flat slots
    page * R + row (negative or out of range: skipped).  Returns the copies."""
    x = np.ascontiguousarray(x)
    slot = np.ascontiguousarray(slot, dtype=np.int64)
    kp = np.array(kpages, dtype=np.int8, copy=True, order="C")
    sp = np.array(spages, dtype=np.uint16, copy=True, order="C")
    P, R = sp.shape
    L = lib()
    L.oracle_write_k.restype = None
    L.oracle_write_k.argtypes = [C.c_void_p, C.c_int, C.c_void_p, C.c_int64, C.c_int, C.c_int64,
                                 C.c_void_p, C.c_void_p]
    L.oracle_write_k(_ptr(x), C.c_int(_dtype_code(x)), _ptr(slot), C.c_int64(slot.size),
                     C.c_int(R), C.c_int64(P), _ptr(kp), _ptr(sp))
    return kp, sp


# ---------------------------------------------------------------------------
# sparse attention over the indexer's positions (qli_attn_oracle.c)
# ---------------------------------------------------------------------------

class _AttnProblem(C.Structure):
    _fields_ = [
        ("num_heads", C.c_int32), ("head_dim", C.c_int32), ("batch", C.c_int32),
        ("num_tokens", C.c_int32), ("topk", C.c_int32), ("window", C.c_int32),
        ("c_page_rows", C.c_int32), ("c_bt_stride", C.c_int32),
        ("r_page_rows", C.c_int32), ("r_bt_stride", C.c_int32),
        ("c_page_stride", C.c_int64), ("r_page_stride", C.c_int64),
        ("scale", C.c_double),
        ("q", C.c_void_p), ("c_kv", C.c_void_p), ("c_bt", C.c_void_p), ("c_lens", C.c_void_p),
        ("r_kv", C.c_void_p), ("r_bt", C.c_void_p), ("r_lens", C.c_void_p),
        ("query_start_loc", C.c_void_p), ("indices", C.c_void_p), ("sinks", C.c_void_p),
    ]


def sparse_attn(ap, tokens=None, indices=None):
    """(out float64 [n, H, D], lse float64 [n, H]) of the attention call
    ``ap`` (a qli_workloads.attn.AttnProblem) for ``tokens`` (default: all);
    ``indices`` overrides ap.indices."""
    keep = []

    def arr(a, dt):
        a = np.ascontiguousarray(a, dtype=dt)
        keep.append(a)
        return a.ctypes.data

    idx = ap.indices if indices is None else indices
    s = _AttnProblem()
    s.num_heads, s.head_dim, s.batch = ap.num_heads, ap.head_dim, ap.batch
    s.num_tokens, s.topk, s.window = ap.num_tokens, int(idx.shape[1]), ap.window
    s.c_page_rows, s.c_bt_stride = ap.c_page_rows, int(ap.c_bt.shape[1])
    s.r_page_rows, s.r_bt_stride = ap.r_page_rows, int(ap.r_bt.shape[1])
    s.c_page_stride, s.r_page_stride = ap.c_page_stride, ap.r_page_stride
    s.scale = float(ap.scale)
    s.q = arr(ap.q, np.uint16)
    s.c_kv = ap.c_pages.ctypes.data
    s.c_bt = arr(ap.c_bt, np.int32)
    s.c_lens = arr(ap.c_lens, np.int32)
    s.r_kv = ap.r_pages.ctypes.data
    s.r_bt = arr(ap.r_bt, np.int32)
    s.r_lens = arr(ap.r_lens, np.int32)
    s.query_start_loc = arr(ap.query_start_loc, np.int32)
    s.indices = arr(idx, np.int32)
    s.sinks = None if ap.sinks is None else arr(ap.sinks, np.float32)
    tok = np.arange(ap.num_tokens, dtype=np.int32) if tokens is None else \
        np.ascontiguousarray(tokens, dtype=np.int32)
    n = int(tok.size)
    out = np.zeros((n, ap.num_heads, ap.head_dim), dtype=np.float64)
    lse = np.zeros((n, ap.num_heads), dtype=np.float64)
    L = lib()
    L.oracle_sparse_attn.restype = C.c_int
    L.oracle_sparse_attn.argtypes = [C.POINTER(_AttnProblem), C.c_void_p, C.c_int, C.c_void_p, C.c_void_p]
    rc = L.oracle_sparse_attn(C.byref(s), tok.ctypes.data, n, out.ctypes.data, lse.ctypes.data)
    if rc != 0:
        raise RuntimeError(f"oracle_sparse_attn failed with {rc}")
    return out, lse
