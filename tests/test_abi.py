"""The C ABI on the CPU: the library loads, exports every declared entry
point, its struct layout matches the header, and every host-side rejection
path returns the documented status without touching a GPU (validation runs
before any launch, and a call with no tokens launches nothing)."""
import ctypes as C
import os
import re
import subprocess

import pytest

import quantized_top_indexer_amd as Q

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "qli.h")


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(Q.LIB_PATH):
        from quantized_top_indexer_amd import build
        build.build()
    return Q.load_library()


def declared_functions(header=HEADER):
    src = open(header).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return re.findall(r"^\s*(?:const\s+)?\w+\**\s+\**(qli_\w+)\s*\(", src, flags=re.M)


def exported(path):
    out = subprocess.run(["nm", "-D", "--defined-only", path], capture_output=True,
                         text=True, check=True).stdout
    return set(re.findall(r" T (qli_\w+)$", out, flags=re.M))


def test_exports_every_declared_symbol(lib):
    names = declared_functions()
    assert set(names) == set(Q.EXPORTS)
    assert set(names) <= exported(Q.LIB_PATH)
    for n in names:
        assert hasattr(lib, n)


def test_probes_live_in_their_own_library(lib):
    """The ceiling probes (measurement only) are not part of the indexer
    library: libqli_probe.so exports what include/qli_probe.h declares."""
    names = declared_functions(os.path.join(ROOT, "include", "qli_probe.h"))
    assert set(names) == set(Q.PROBE_EXPORTS)
    assert set(names) <= exported(Q.PROBE_LIB_PATH)
    assert not (set(names) & exported(Q.LIB_PATH))


def test_abi_version(lib):
    assert Q.qli_abi_version() == Q.QLI_ABI_VERSION == 6


@pytest.mark.parametrize("struct", ["qli_params", "qli_quant_params", "qli_kwrite_params", "qli_attn_params"])
def test_struct_layout_matches_header(tmp_path, struct):
    cls = getattr(Q, struct)
    fields = [f[0] for f in cls._fields_]
    prog = tmp_path / "layout.c"
    body = "\n".join(f'  printf("{f} %zu\\n", offsetof({struct}, {f}));' for f in fields)
    prog.write_text(f'#include <stdio.h>\n#include <stddef.h>\n#include "qli.h"\n'
                    f'int main(void) {{\n{body}\n  printf("sizeof %zu\\n", sizeof({struct}));\n'
                    f'  return 0;\n}}\n')
    exe = tmp_path / "layout"
    subprocess.run(["gcc", "-std=c11", "-I", os.path.dirname(HEADER), str(prog), "-o", str(exe)],
                   check=True)
    got = dict(line.split() for line in subprocess.run([str(exe)], capture_output=True, text=True,
                                                       check=True).stdout.splitlines())
    for f in fields:
        assert int(got[f]) == getattr(cls, f).offset, f
    assert int(got["sizeof"]) == C.sizeof(cls)


def base_params(mode=2, ratio=2, T=4):
    """Scalars of a valid call with fake (never dereferenced) device pointers."""
    p = Q.new_params()
    p.mode, p.ratio, p.num_heads = mode, ratio, 32
    p.batch, p.num_tokens, p.topk = 1, T, 16
    p.cand_blocks, p.cand_in_blocks = 64, 64
    p.page_rows = 128 // ratio
    p.bt_stride, p.num_pages, p.max_k_len = 4, 8, 128
    p.k_page_stride = 131072 if ratio == 2 else 147712
    p.s_page_stride = p.k_page_stride
    fake = 0x7F0000000000
    for i, f in enumerate(("q", "q_scale", "weights", "k_cache", "k_scale", "block_table",
                           "query_start_loc", "k_lens", "topk_out", "cand_out")):
        setattr(p, f, fake + 4096 * i)
    p.seq_mod = fake + 4096 * 20 if ratio == 2 else None
    p.cand_in = fake + 4096 * 21 if mode == 3 else None
    p.workspace = fake + (1 << 30)
    p.workspace_bytes = 1 << 30
    return p


def test_valid_params_pass(lib):
    for mode in (1, 2, 3):
        for ratio in (1, 2):
            assert Q.qli_validate(base_params(mode, ratio)) == Q.QLI_OK


@pytest.mark.parametrize("field,value,code", [
    ("dbg_qk", 0x7F0000100000, Q.QLI_ERR_INVALID_ARG),  # debug q.k without debug scores
    ("struct_size", 8, Q.QLI_ERR_INVALID_ARG),
    ("head_dim", 64, Q.QLI_ERR_UNSUPPORTED),
    ("quant_mode", 1, Q.QLI_ERR_UNSUPPORTED),
    ("num_heads", 16, Q.QLI_ERR_UNSUPPORTED),
    ("num_heads", 128, Q.QLI_ERR_UNSUPPORTED),
    ("mode", 0, Q.QLI_ERR_INVALID_ARG),
    ("mode", 4, Q.QLI_ERR_INVALID_ARG),
    ("ratio", 4, Q.QLI_ERR_INVALID_ARG),
    ("page_rows", 128, Q.QLI_ERR_INVALID_ARG),
    ("topk", 0, Q.QLI_ERR_INVALID_ARG),
    ("topk", 2049, Q.QLI_ERR_INVALID_ARG),
    ("cand_blocks", 32, Q.QLI_ERR_INVALID_ARG),
    ("cand_blocks", 100, Q.QLI_ERR_INVALID_ARG),
    ("cand_blocks", 2112, Q.QLI_ERR_INVALID_ARG),
    ("batch", 0, Q.QLI_ERR_INVALID_ARG),
    ("num_tokens", -1, Q.QLI_ERR_INVALID_ARG),
    ("max_k_len", -1, Q.QLI_ERR_INVALID_ARG),
    ("max_k_len", (1 << 24) + 1, Q.QLI_ERR_UNSUPPORTED),
    ("bt_stride", 1, Q.QLI_ERR_INVALID_ARG),   # 1 page * 64 rows < max_k_len 128
    ("num_pages", 0, Q.QLI_ERR_INVALID_ARG),
    ("k_page_stride", 131072 + 8, Q.QLI_ERR_INVALID_ARG),
    ("k_page_stride", 64 * 128 - 16, Q.QLI_ERR_INVALID_ARG),
    ("s_page_stride", 131073, Q.QLI_ERR_INVALID_ARG),
    ("s_page_stride", 131072 + 8, Q.QLI_ERR_INVALID_ARG),
    ("k_scale", 0x7F0000000000 + 4096 * 4 + 2, Q.QLI_ERR_INVALID_ARG),
    ("reserved0", 1, Q.QLI_ERR_INVALID_ARG),
    ("q", None, Q.QLI_ERR_INVALID_ARG),
    ("k_cache", None, Q.QLI_ERR_INVALID_ARG),
    ("topk_out", None, Q.QLI_ERR_INVALID_ARG),
    ("cand_out", None, Q.QLI_ERR_INVALID_ARG),
    ("seq_mod", None, Q.QLI_ERR_INVALID_ARG),           # ratio 2 needs the residual
    ("q", 0x7F0000000000 + 8, Q.QLI_ERR_INVALID_ARG),   # not 16-B aligned
    ("workspace", None, Q.QLI_ERR_WORKSPACE),
    ("workspace_bytes", 1024, Q.QLI_ERR_WORKSPACE),
])
def test_rejections(lib, field, value, code):
    p = base_params(mode=2, ratio=2)
    setattr(p, field, value)
    assert Q.qli_validate(p) == code
    # the enqueue entry point rejects identically, before any launch
    assert lib.qli_score_topk(C.byref(p), None) == code


def test_residual_must_be_absent_at_ratio_1(lib):
    p = base_params(mode=2, ratio=1)
    p.seq_mod = 0x7F0000100000
    assert Q.qli_validate(p) == Q.QLI_ERR_INVALID_ARG


def test_consumer_without_source(lib):
    p = base_params(mode=3)
    p.cand_in = None
    assert Q.qli_validate(p) == Q.QLI_ERR_NO_SOURCE
    p = base_params(mode=3)
    p.cand_in_blocks = 65
    assert Q.qli_validate(p) == Q.QLI_ERR_INVALID_ARG


def test_zero_tokens_is_a_noop(lib):
    p = base_params(mode=2, T=0)
    for f in ("q", "k_cache", "topk_out", "workspace"):
        setattr(p, f, None)
    p.workspace_bytes = 0
    assert lib.qli_score_topk(C.byref(p), None) == Q.QLI_OK


def test_workspace_bytes(lib):
    p = base_params(mode=2, ratio=2, T=4)
    # keys: 4 tokens * roundup(128, 256) slots * 4 B; block keys: 4 * 64 * 4 B;
    # plan header 256 B, groups 2 * 4 * 32 B, group prefixes 2 * 5 * 4 B (each 256-B aligned),
    # 2048 workgroup start entries of 64 B, per-token visible counts 4 * 4 B
    starts = 2048 * 64 + 256
    assert Q.qli_workspace_bytes(p) == 4 * 256 * 4 + 4 * 64 * 4 + 256 + 256 + 256 + starts
    p = base_params(mode=3, ratio=2, T=4)
    # keys: 4 * 64*8 * 4; plan 3 * 256; slots + page rows: 2 * 4 * 64 * 4; counts 256
    assert Q.qli_workspace_bytes(p) == 4 * 512 * 4 + 3 * 256 + starts + 2 * 4 * 64 * 4 + 256
    p.head_dim = 3
    assert Q.qli_workspace_bytes(p) == 0


def test_status_strings(lib):
    for code in range(6):
        assert Q.qli_status_string(code).startswith("QLI_")
    assert "unknown" in Q.qli_status_string(99)


def test_output_shapes():
    assert Q.output_shapes(7, 16, 64, Q.QLI_MODE_SOURCE) == ((7, 1, 16), (7, 1, 64))
    assert Q.output_shapes(7, 16, 64, Q.QLI_MODE_CONSUMER) == ((7, 1, 16), None)


def test_one_hip_runtime_per_process():
    """Loading the library before torch must not bring a second HIP runtime
    into the process (torch's streams would be foreign to it)."""
    code = ("import quantized_top_indexer_amd as Q; Q.load_library(); import torch; "
            "m = open('/proc/self/maps').read().splitlines(); "
            "print(len({l.split()[-1] for l in m if 'libamdhip64' in l}))")
    out = subprocess.run(["python", "-c", code], capture_output=True, text=True, check=True,
                         cwd=ROOT).stdout.strip()
    assert out == "1"


FAKE = 0x7F0000000000


def quant_params(rows=8, nw=8):
    p = Q.qli_quant_params()
    p.struct_size = C.sizeof(Q.qli_quant_params)
    p.num_rows, p.head_dim, p.x_dtype, p.num_weights, p.w_dtype = rows, 128, Q.QLI_DTYPE_BF16, nw, \
        Q.QLI_DTYPE_F32
    p.x, p.q, p.q_scale, p.w, p.w_out = FAKE, FAKE + 4096, FAKE + 8192, FAKE + 12288, FAKE + 16384
    return p


def kwrite_params(rows=8):
    p = Q.qli_kwrite_params()
    p.struct_size = C.sizeof(Q.qli_kwrite_params)
    p.num_rows, p.head_dim, p.x_dtype, p.page_rows = rows, 128, Q.QLI_DTYPE_F32, 64
    p.num_pages, p.k_page_stride, p.s_page_stride = 16, 131072, 131072
    p.x, p.slot, p.k_cache, p.k_scale = FAKE, FAKE + 4096, FAKE + 8192, FAKE + 8192 + 73728
    return p


@pytest.mark.parametrize("field,value,code", [
    ("struct_size", 4, Q.QLI_ERR_INVALID_ARG),
    ("head_dim", 64, Q.QLI_ERR_UNSUPPORTED),
    ("x_dtype", 2, Q.QLI_ERR_UNSUPPORTED),
    ("w_dtype", -1, Q.QLI_ERR_UNSUPPORTED),
    ("num_rows", -1, Q.QLI_ERR_INVALID_ARG),
    ("num_weights", -3, Q.QLI_ERR_INVALID_ARG),
    ("x", None, Q.QLI_ERR_INVALID_ARG),
    ("q", None, Q.QLI_ERR_INVALID_ARG),
    ("q_scale", None, Q.QLI_ERR_INVALID_ARG),
    ("w", None, Q.QLI_ERR_INVALID_ARG),
    ("w_out", None, Q.QLI_ERR_INVALID_ARG),
    ("x", FAKE + 8, Q.QLI_ERR_INVALID_ARG),
    ("q", FAKE + 4096 + 4, Q.QLI_ERR_INVALID_ARG),
    ("q_scale", FAKE + 8192 + 1, Q.QLI_ERR_INVALID_ARG),
    ("w", FAKE + 12288 + 2, Q.QLI_ERR_INVALID_ARG),  # f32 weights need 4-byte alignment
])
def test_quantize_rejections(lib, field, value, code):
    p = quant_params()
    setattr(p, field, value)
    assert Q.qli_quantize_query(p, 0) == code


def test_quantize_noop_and_optional_weights(lib):
    p = quant_params(rows=0, nw=0)
    p.x = p.q = p.q_scale = p.w = p.w_out = None
    assert Q.qli_quantize_query(p, 0) == Q.QLI_OK  # nothing to do: no launch
    p = quant_params(rows=0, nw=5)
    p.w = None
    assert Q.qli_quantize_query(p, 0) == Q.QLI_ERR_INVALID_ARG


@pytest.mark.parametrize("field,value,code", [
    ("struct_size", 8, Q.QLI_ERR_INVALID_ARG),
    ("head_dim", 256, Q.QLI_ERR_UNSUPPORTED),
    ("x_dtype", 5, Q.QLI_ERR_UNSUPPORTED),
    ("num_rows", -2, Q.QLI_ERR_INVALID_ARG),
    ("reserved0", 1, Q.QLI_ERR_INVALID_ARG),
    ("page_rows", 32, Q.QLI_ERR_INVALID_ARG),
    ("num_pages", 0, Q.QLI_ERR_INVALID_ARG),
    ("k_page_stride", 64 * 128 - 16, Q.QLI_ERR_INVALID_ARG),
    ("k_page_stride", 131072 + 8, Q.QLI_ERR_INVALID_ARG),
    ("s_page_stride", 127, Q.QLI_ERR_INVALID_ARG),
    ("s_page_stride", 131073, Q.QLI_ERR_INVALID_ARG),
    ("x", None, Q.QLI_ERR_INVALID_ARG),
    ("slot", None, Q.QLI_ERR_INVALID_ARG),
    ("k_cache", None, Q.QLI_ERR_INVALID_ARG),
    ("k_scale", None, Q.QLI_ERR_INVALID_ARG),
    ("slot", FAKE + 4096 + 4, Q.QLI_ERR_INVALID_ARG),
    ("k_cache", FAKE + 8192 + 8, Q.QLI_ERR_INVALID_ARG),
    ("k_scale", FAKE + 8192 + 73728 + 1, Q.QLI_ERR_INVALID_ARG),
    ("status_out", FAKE + 2, Q.QLI_ERR_INVALID_ARG),
])
def test_write_k_rejections(lib, field, value, code):
    p = kwrite_params()
    setattr(p, field, value)
    assert Q.qli_write_index_k(p, 0) == code


def test_write_k_noop(lib):
    p = kwrite_params(rows=0)
    p.x = p.slot = p.k_cache = p.k_scale = None
    assert Q.qli_write_index_k(p, 0) == Q.QLI_OK
    p.page_rows = 100  # scalars are still checked with no rows
    assert Q.qli_write_index_k(p, 0) == Q.QLI_ERR_INVALID_ARG


@pytest.mark.parametrize("field,mode", [("status_out", 2), ("cand_out", 2), ("dbg_scores", 2),
                                        ("seq_mod", 2), ("cand_in", 3)])
def test_word_pointer_alignment(lib, field, mode):
    """Optional and mode-dependent pointers are read or written as 32-bit
    words (the status word with device atomics): a pointer off a 4-byte
    boundary is rejected before any launch; an aligned one passes."""
    p = base_params(mode=mode, ratio=2)
    setattr(p, field, 0x7F0000300000 + 2)
    assert Q.qli_validate(p) == Q.QLI_ERR_INVALID_ARG
    assert lib.qli_score_topk(C.byref(p), None) == Q.QLI_ERR_INVALID_ARG
    setattr(p, field, 0x7F0000300000)
    assert Q.qli_validate(p) == Q.QLI_OK


def test_noalloc_rejections(lib):
    """The entry point without a workspace checks every argument as
    qli_score_topk does (the workspace fields aside) and rejects a call whose
    scratch need exceeds the static array, before any launch."""
    p = base_params(mode=2, ratio=2)
    p.workspace, p.workspace_bytes = None, 0          # ignored by this entry point
    for field, value in (("topk", 0), ("q", None), ("cand_out", 0x7F0000300002)):
        bad = base_params(mode=2, ratio=2)
        setattr(bad, field, value)
        assert lib.qli_score_topk_noalloc(C.byref(bad), None) == Q.qli_validate(bad) != Q.QLI_OK
    # the call runs in slices of as many tokens as the array holds; only a
    # single token that does not fit is rejected: 2^24 positions need 64 MiB
    # of keys per token
    p.max_k_len, p.bt_stride = 1 << 24, (1 << 24) // 64
    assert Q.qli_workspace_bytes(p) > Q.QLI_STATIC_SCRATCH_BYTES
    assert lib.qli_score_topk_noalloc(C.byref(p), None) == Q.QLI_ERR_SCRATCH_LIMIT
    assert "static scratch" in Q.qli_status_string(Q.QLI_ERR_SCRATCH_LIMIT)
    p.num_tokens = 0                                  # a no-op, nothing looked up
    assert lib.qli_score_topk_noalloc(C.byref(p), None) == Q.QLI_OK


def long_prefill_params(ratio=2, mode=2, T=8192):
    """An 8192-token chunk at 1M raw context (524288 compressed positions at
    ratio 2), fake pointers."""
    p = base_params(mode=mode, ratio=ratio, T=T)
    p.num_heads = 64
    p.max_k_len = (1 << 20) // ratio
    p.bt_stride = p.max_k_len // p.page_rows
    p.topk, p.cand_blocks, p.cand_in_blocks = 2048, 2048, 2048
    return p


@pytest.mark.parametrize("ratio,mode", [(2, 2), (1, 2), (2, 1), (2, 3)])
def test_workspace_bounded_by_slices(lib, ratio, mode):
    """Long-context prefill calls run in token slices that reuse one bounded
    workspace: the recommended size stays within the 4 GiB slice budget
    instead of growing with tokens x context (17-34 GB unsliced), a
    workspace of one token's slice is accepted, and anything smaller is
    rejected before any launch."""
    p = long_prefill_params(ratio, mode)
    need = Q.qli_workspace_bytes(p)
    per_token = p.max_k_len * 4 if mode != 3 else 2048 * 8 * 4
    if mode != 3:
        assert p.num_tokens * per_token > 16e9       # what an unsliced call would need
        assert need <= (4 << 30)
        assert need >= (4 << 30) - 2 * (per_token + (p.max_k_len // 8) * 4)
    p.workspace, p.workspace_bytes = 0x7F0000000000, need
    assert Q.qli_validate(p) == Q.QLI_OK
    one = base_params(mode=mode, ratio=ratio, T=1)     # same scalars, one token
    for f in ("num_heads", "max_k_len", "bt_stride", "topk", "cand_blocks", "cand_in_blocks"):
        setattr(one, f, getattr(p, f))
    p.workspace_bytes = Q.qli_workspace_bytes(one)
    assert Q.qli_validate(p) == Q.QLI_OK
    p.workspace_bytes -= 256
    assert Q.qli_validate(p) == Q.QLI_ERR_WORKSPACE


def test_workspace_unsliced_when_it_fits(lib):
    """Calls within the budget get the whole-call workspace (one slice):
    doubling the tokens of a small call doubles its token-indexed parts."""
    p = base_params(mode=2, ratio=2, T=100)
    q = base_params(mode=2, ratio=2, T=200)
    a, b = Q.qli_workspace_bytes(p), Q.qli_workspace_bytes(q)
    assert b > a and b - a >= 100 * (256 + 64) * 4


def test_debug_qk_alignment(lib):
    p = base_params(mode=2, ratio=2)
    p.dbg_scores = 0x7F0000200000
    p.dbg_qk = 0x7F0000100002
    assert Q.qli_validate(p) == Q.QLI_ERR_INVALID_ARG
    p.dbg_qk = 0x7F0000100000
    assert Q.qli_validate(p) == Q.QLI_OK


def test_probe_rejections(lib):
    fake = 0x7F0000000000
    assert Q.qli_probe_hbm_read(fake, 1 << 20, 64, None, 0) == Q.QLI_ERR_INVALID_ARG   # no sink
    assert Q.qli_probe_hbm_read(fake, 100, 64, fake, 0) == Q.QLI_ERR_INVALID_ARG       # not x16 bytes
    assert Q.qli_probe_hbm_read(fake + 8, 1 << 20, 64, fake, 0) == Q.QLI_ERR_INVALID_ARG
    assert Q.qli_probe_hbm_read(fake, 1 << 20, 0, fake, 0) == Q.QLI_ERR_INVALID_ARG
    assert Q.qli_probe_int8_mfma(0, 10, fake, 0) == Q.QLI_ERR_INVALID_ARG
    assert Q.qli_probe_int8_mfma(16, 0, fake, 0) == Q.QLI_ERR_INVALID_ARG
    assert Q.qli_probe_int8_mfma_ops(2, 3) == 2 * 4 * 3 * 4 * 32 * 32 * 32 * 2


def _attn_params(**kw):
    p = Q.qli_attn_params()
    p.struct_size = C.sizeof(Q.qli_attn_params)
    p.num_heads, p.head_dim, p.batch, p.num_tokens = 64, 512, 1, 0
    p.topk, p.window = 16, 0
    p.c_page_rows, p.c_bt_stride, p.c_num_pages, p.c_page_stride = 64, 4, 8, 131072
    p.scale = 0.04
    for k, v in kw.items():
        setattr(p, k, v)
    return p


@pytest.mark.parametrize("kw,code", [
    ({}, 0),                                           # no tokens: a no-op
    ({"head_dim": 576}, 2), ({"num_heads": 24}, 2), ({"num_heads": 144}, 2),
    ({"topk": 2049}, 1), ({"window": 513}, 1), ({"window": -1}, 1), ({"batch": 0}, 1),
    ({"c_page_stride": 131072 + 8}, 1), ({"c_page_stride": 64 * 1024 - 16}, 1),
    ({"reserved0": 1}, 1), ({"scale": float("inf")}, 1),
    ({"window": 8}, 1),                                 # window without raw pool geometry
    ({"num_tokens": 1}, 1),                             # tokens but no pointers
    ({"struct_size": 8}, 1), ({"c_page_rows": 257}, 1), ({"c_num_pages": 1 << 23}, 1),
])
def test_attention_host_validation(lib, kw, code):
    assert lib.qli_sparse_attention(C.byref(_attn_params(**kw)), None) == code


def _attn_pointers(p):
    # stand-in device addresses (never dereferenced: every case below is
    # rejected on the host before any launch)
    for i, f in enumerate(("q", "c_cache", "c_block_table", "c_lens", "query_start_loc", "indices", "out")):
        setattr(p, f, 0x10000000 + 0x100000 * i)
    return p


@pytest.mark.parametrize("kw", [{"workspace_bytes": -1}, {"workspace": 0x20000000 + 16, "workspace_bytes": 1 << 20},
                                {"out": 0x30000000 + 8}])
def test_attention_workspace_validation(lib, kw):
    p = _attn_pointers(_attn_params(num_tokens=1))
    for k, v in kw.items():
        setattr(p, k, v)
    assert lib.qli_sparse_attention(C.byref(p), None) == 1


@pytest.mark.parametrize("T,H,topk,window,nbytes", [
    (64, 64, 2048, 128, 64 * 4 * 64 * 8 + 64 * 4 * 64 * 2048),  # four splits per token
    (100, 128, 2048, 0, 200 * 2 * 64 * 8 + 200 * 2 * 64 * 2048),  # 200 (token, 64 heads): two
    (64, 32, 2048, 128, 0),      # heads not a multiple of 64: the head-group kernel, no split
    (256, 64, 2048, 128, 0),     # the tokens fill the GPU without a split
    (1, 64, 16, 8, 0),           # one 32-entry step: nothing to split
    (1, 64, 40, 0, 2 * 64 * 8 + 2 * 64 * 2048),  # two steps: two splits
])
def test_attention_workspace_bytes(lib, T, H, topk, window, nbytes):
    p = _attn_params(num_tokens=T, num_heads=H, topk=topk, window=window)
    assert lib.qli_attn_workspace_bytes(C.byref(p)) == nbytes
    assert lib.qli_attn_workspace_bytes(None) == 0
