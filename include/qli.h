/*
 * qli.h - C ABI of the MI355X (gfx950) quantized lightning indexer (QLI)
 * with hierarchical candidate blocks.
 *
 * What one call computes (DeepSeek V4.1 QLI developer guide, "数据流" and
 * "当前 A3 契约" sections):
 *
 *   For every query token t of a TND batch and every compressed position j
 *   of its request that t may see (causal mask mode 3) and that is eligible:
 *     qk   = sum_d q[t,h,d] * k[j,d]                 (exact INT32)
 *     x    = fp16(qk / 1024); x = max(x, +0)        (FP16 ReLU)
 *     m    = fp16(weights[t,h] * q_scale[t,h])       (FP16)
 *     p    = fp16(x * m)                             (FP16)
 *     sum  = p_0 + p_1 + ... + p_{N-1}               (FP32, from +0, ascending h)
 *     score[t,j] = fp32(sum * k_scale[j])            (FP32 K scaling)
 *   Every rounding is IEEE round-to-nearest-even; FP16 subnormals are kept.
 *   The head-sum order is fixed (ascending head), so scores are exactly
 *   reproducible, not merely within a tolerance.
 *
 *   Visibility: the queries of request b are its last n_b raw positions;
 *   the query at raw position p sees compressed entries j < floor((p+1)/r),
 *   where the raw length is S_b = k_lens[b] * r + seq_mod[b].
 *
 *   Outputs (ties: higher score first, then lower position / block id):
 *     topk_out[t, 0, :]  the top min(topk, |E_t|) eligible positions in
 *                        ascending (chronological) order, -1 padding at
 *                        the tail;
 *     cand_out[t, 0, :]  (source mode) candidate block ids: a block is 8
 *                        consecutive compressed positions [8c, 8c+8), its
 *                        score the maximum visible position score; the
 *                        last visible block ceil(V/8)-1 is always kept and
 *                        the best cand_blocks-1 other visible blocks join
 *                        it; ascending ids, -1 tail.  An empty compressed
 *                        context gives all -1.
 *   Modes (runtime parameter, one operator):
 *     QLI_MODE_PLAIN    positions over the whole visible context;
 *     QLI_MODE_SOURCE   positions over the whole visible context, plus the
 *                       candidate blocks;
 *     QLI_MODE_CONSUMER positions restricted to the incoming candidate
 *                       blocks cand_in[t, 0, :] (negative ids ignored,
 *                       duplicates collapse, ids past the visible range add
 *                       nothing).  A consumer without candidates is an
 *                       error (QLI_ERR_NO_SOURCE).
 *
 * Memory: every pointer in qli_params is DEVICE memory owned by the caller
 * (typically torch tensors); the library allocates nothing.  Integer
 * metadata is read on the device only, so a call never synchronises with
 * the host.  Alignment: the 16-B and 2-B cases are stated per field; every
 * other pointer (int32 / uint32 / float arrays, optional ones included when
 * not NULL) must be 4-byte aligned, or the call returns QLI_ERR_INVALID_ARG.
 */
#ifndef QLI_H
#define QLI_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define QLI_ABI_VERSION 6

/* Status codes returned by the host entry points. */
enum qli_status {
  QLI_OK = 0,
  QLI_ERR_INVALID_ARG = 1, /* null pointer, value out of range, bad stride or
                              alignment, residual present at ratio 1 or
                              missing at ratio 2, page_rows != 128/ratio */
  QLI_ERR_UNSUPPORTED = 2, /* num_heads not 32/64, head_dim not 128, quant
                              mode not INT8, sizes past the documented caps */
  QLI_ERR_NO_SOURCE = 3,   /* consumer mode without incoming candidates */
  QLI_ERR_WORKSPACE = 4,   /* workspace missing, misaligned, or too small
                              for a slice of one query token */
  QLI_ERR_HIP = 5,         /* a kernel launch failed */
  QLI_ERR_SCRATCH_LIMIT = 6 /* qli_score_topk_noalloc: the call needs more
                               than QLI_STATIC_SCRATCH_BYTES of scratch */
};

/* Candidate modes: all three run through the same operator (guide, section
   on candidate modes). */
enum qli_mode { QLI_MODE_PLAIN = 1, QLI_MODE_SOURCE = 2, QLI_MODE_CONSUMER = 3 };

/* INT8 is quantisation mode 2 in the guide's numbering of quantisation modes. */
#define QLI_QUANT_INT8 2

/* Bits the kernels OR into *status_out when a device-side metadata value is
 * out of contract.  The affected positions are treated as not eligible, so
 * every memory access stays inside the buffers described here. */
#define QLI_DEV_BAD_PAGE 1u     /* block-table entry < 0 or >= num_pages, or a
                                   page index past bt_stride */
#define QLI_DEV_BAD_LENGTH 2u   /* k_lens[b] < 0 or > max_k_len */
#define QLI_DEV_BAD_METADATA 4u /* seq_mod outside [0, ratio), or a request
                                   with more queries than raw tokens */
#define QLI_DEV_BAD_INDEX 8u    /* qli_sparse_attention: an index at or beyond the request's
                                   compressed length (the entry is skipped) */

/* Documented caps (QLI_ERR_UNSUPPORTED beyond them). */
#define QLI_MAX_TOPK 2048
#define QLI_MAX_CAND_BLOCKS 2048
#define QLI_ATTN_MAX_TOPK 2048   /* qli_sparse_attention: widest index row */
#define QLI_ATTN_MAX_WINDOW 512  /* qli_sparse_attention: longest window */
#define QLI_MAX_K_LEN (1 << 24)

typedef struct qli_params {
  uint32_t struct_size; /* = sizeof(qli_params) */
  int32_t mode;         /* enum qli_mode */
  int32_t ratio;        /* compress ratio r: 1 or 2 */
  int32_t num_heads;    /* N index heads: 32 or 64 */
  int32_t head_dim;     /* must be 128 */
  int32_t quant_mode;   /* must be QLI_QUANT_INT8 */
  int32_t batch;        /* B requests */
  int32_t num_tokens;   /* T query tokens (TND rows) */
  int32_t topk;         /* position top-k, 1..2048 */
  int32_t cand_blocks;  /* source mode: output candidate width, a multiple
                           of 64 in [64, 2048]; ignored otherwise */
  int32_t cand_in_blocks; /* consumer mode: incoming candidate width, a
                             multiple of 64 in [64, 2048]; ignored otherwise */
  int32_t page_rows;    /* rows per page view: 128 / ratio */
  int32_t bt_stride;    /* entries per block-table row (>= 1) */
  int32_t num_pages;    /* pages addressable through k_cache / k_scale */
  int32_t max_k_len;    /* host-side upper bound of k_lens[] (sizes the
                           grid and the workspace without a sync) */
  int32_t reserved0;    /* must be 0 */
  int64_t k_page_stride; /* bytes between page p and p+1 of the K view;
                            multiple of 16, >= page_rows * 128 */
  int64_t s_page_stride; /* bytes between page p and p+1 of the scale
                            view; multiple of 16, >= page_rows * 2 */

  /* inputs (device) */
  const int8_t* q;          /* [T, N, 128] int8, contiguous TND, 16-B aligned */
  const uint16_t* q_scale;  /* [T, N] fp16 bits, per token and head */
  const uint16_t* weights;  /* [T, N] fp16 bits, head weights */
  const int8_t* k_cache;    /* row 0 of page 0 of the index-K view: row j of
                               page p at k_cache + p*k_page_stride + j*128;
                               16-B aligned */
  const void* k_scale;      /* row 0 of page 0 of the fp16 scale view: row j
                               of page p at (char*)k_scale + p*s_page_stride
                               + j*2; 16-B aligned (8 rows are read as one
                               16-byte run) */
  const int32_t* block_table;     /* [B, bt_stride] page ids: compressed
                                     position j of request b lives in page
                                     block_table[b][j / page_rows], row
                                     j % page_rows */
  const int32_t* query_start_loc; /* [B+1] raw query boundaries in TND
                                     order; [0] = 0, non-decreasing,
                                     [B] = T */
  const int32_t* k_lens;          /* [B] compressed K lengths */
  const int32_t* seq_mod;         /* [B] raw length mod ratio; must be NULL
                                     at ratio 1 and non-NULL at ratio 2 */
  const int32_t* cand_in;         /* consumer: [T, 1, cand_in_blocks] block
                                     ids, -1 padded */

  /* outputs (device) */
  int32_t* topk_out;    /* [T, 1, topk] */
  int32_t* cand_out;    /* source: [T, 1, cand_blocks]; else may be NULL */
  float* dbg_scores;    /* optional (NULL in production): [T, max_k_len]
                           FP32 scores by position, written only where a
                           position is eligible */
  int32_t* dbg_qk;      /* optional (NULL in production), needs dbg_scores:
                           [T, N, max_k_len] exact INT32 q.k by token, head
                           and position, written only where the position is
                           eligible */
  uint32_t* status_out; /* optional device word receiving QLI_DEV_* bits
                           (never cleared by the library) */

  /* scratch (device), caller-allocated, 256-B aligned.  The call runs in
     slices of consecutive query tokens, each reusing the whole workspace,
     and takes the largest slice that workspace_bytes holds: the size
     qli_workspace_bytes(p) recommends runs the call in one slice when it
     needs at most 4 GiB and in slices of at most 4 GiB otherwise; any size
     holding a one-token slice is accepted (smaller: QLI_ERR_WORKSPACE). */
  void* workspace;
  size_t workspace_bytes;
} qli_params;

/* ABI version of the loaded library (QLI_ABI_VERSION at build time). */
int qli_abi_version(void);

/* Host-only argument check, exactly the one qli_score_topk() performs
 * before launching anything.  Reads no device memory. Returns a qli_status. */
int qli_validate(const qli_params* p);

/* Recommended workspace bytes for a call with these scalars (host-only;
 * depends on mode, ratio, num_tokens, max_k_len, cand_blocks and
 * cand_in_blocks): the whole call when its workspace is at most 4 GiB,
 * otherwise the largest token slice within 4 GiB (an 8192-token chunk at
 * 1M raw context then needs 4 GiB instead of 17-34 GB).  A larger
 * workspace lets a call run in fewer slices.  0 when p is NULL or when the
 * scalars are invalid. */
size_t qli_workspace_bytes(const qli_params* p);

/* Enqueue the whole indexer on `stream` (a hipStream_t; NULL = the null
 * stream) and return at once: no host-device synchronisation, no
 * allocation.  Validation runs before any launch; num_tokens == 0 is a
 * valid no-op.  Kernel faults surface at the caller's next synchronisation.
 * Re-entrant for calls with distinct workspaces and outputs; calls that
 * share a workspace must be ordered on one stream. Returns a qli_status. */
int qli_score_topk(const qli_params* p, void* stream);

/* Scratch of qli_score_topk_noalloc: a device array of this many bytes
 * inside the library, one per GPU it runs on, held until the process
 * ends. */
#define QLI_STATIC_SCRATCH_BYTES (32u << 20)

/* The same operation as qli_score_topk, for callers that cannot allocate
 * device memory or hand the library a workspace: code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc.  The
 * scratch is the library's own static device array
 * (QLI_STATIC_SCRATCH_BYTES per GPU); p->workspace and p->workspace_bytes
 * are ignored.  Every other field, the validation and the outputs are those
 * of qli_score_topk.  The call runs in token slices that fit the array
 * (decode-sized calls in one: 64 tokens over 32768 positions in source mode
 * need 9.5 MB); a call whose one-token slice exceeds it returns
 * QLI_ERR_SCRATCH_LIMIT before anything is launched.  Nothing here allocates: the first call on a device looks
 * the array up once (hipGetSymbolAddress), no hipMalloc/hipFree and no
 * timing events.  Every call on one GPU shares that GPU's array: calls that
 * overlap in time on one GPU (other streams, other threads) race and give
 * undefined results; calls ordered on one stream are safe, and each call
 * rewrites every scratch word it reads, so nothing needs clearing between
 * calls.  Returns a qli_status. */
int qli_score_topk_noalloc(const qli_params* p, void* stream);

/* Static, human-readable name of a status code. */
const char* qli_status_string(int status);

/* ---- Producers of the indexer's inputs --------------------------------
 *
 * Query quantization (DeepSeek V4.1 QLI developer guide, "数据流": every
 * query head becomes INT8 with a representable FP16 scale, the head weights
 * are FP16; "当前 A3 契约": per-head Q scale, quantization mode 2) and the
 * index-K cache write (the same guide: paged INT8 index K with one FP16
 * scale per compressed position, in 64-row pages at a 131072-byte stride or
 * 128-row pages at 147712 bytes).  The guide gives no formula; this library
 * implements, for one row x[0..127] of query head or K position:
 *   amax = max_d |x_d|;  s = fp16(fp32(amax / 127)) saturated to 65504;
 *   q_d  = clamp(rint(fp32(x_d / s)), -127, 127)   (q = 0 when s == 0)
 * with IEEE round-to-nearest-even everywhere (rint: ties to even), and
 * weights = fp16(w) (RNE, overflow to infinity).  Inputs are FP32 or
 * bfloat16 and must be finite. */
#define QLI_DTYPE_F32 0
#define QLI_DTYPE_BF16 1

typedef struct qli_quant_params {
  int32_t struct_size;  /* sizeof(qli_quant_params) */
  int32_t num_rows;     /* query heads to quantize (T * N), >= 0 */
  int32_t head_dim;     /* must be 128 */
  int32_t x_dtype;      /* QLI_DTYPE_* of x */
  int32_t num_weights;  /* head weights to round (T * N), >= 0 (0: none) */
  int32_t w_dtype;      /* QLI_DTYPE_* of w */
  const void* x;        /* [num_rows, 128] (16-B aligned), read */
  int8_t* q;            /* [num_rows, 128] (16-B aligned), written */
  void* q_scale;        /* fp16 [num_rows] (2-B aligned), written */
  const void* w;        /* [num_weights], read (may be NULL when num_weights == 0) */
  void* w_out;          /* fp16 [num_weights], written */
} qli_quant_params;

/* Enqueue the quantization of num_rows query heads and the rounding of
 * num_weights head weights on `stream`; no allocation, no synchronisation.
 * Validation runs first; num_rows == num_weights == 0 is a no-op.
 * Returns a qli_status. */
int qli_quantize_query(const qli_quant_params* p, void* stream);

typedef struct qli_kwrite_params {
  int32_t struct_size;    /* sizeof(qli_kwrite_params) */
  int32_t num_rows;       /* new K rows, >= 0 */
  int32_t head_dim;       /* must be 128 */
  int32_t x_dtype;        /* QLI_DTYPE_* of x */
  int32_t page_rows;      /* rows per page: 128 (ratio 1) or 64 (ratio 2) */
  int32_t reserved0;      /* must be 0 */
  int64_t num_pages;      /* pages of the pool, >= 1 */
  int64_t k_page_stride;  /* bytes between pages of the K view, multiple of 16, >= page_rows * 128 */
  int64_t s_page_stride;  /* bytes between pages of the scale view, even, >= page_rows * 2 */
  const void* x;          /* [num_rows, 128] new K rows (16-B aligned), read */
  const int64_t* slot;    /* [num_rows] destination page * page_rows + row; < 0: no
                             slot (row skipped); >= num_pages * page_rows: skipped
                             and flagged */
  int8_t* k_cache;        /* row 0 of page 0 of the index-K view (16-B aligned) */
  void* k_scale;          /* fp16 row 0 of page 0 of the scale view (2-B aligned) */
  uint32_t* status_out;   /* optional device word: QLI_DEV_BAD_PAGE is ORed in for a
                             slot beyond the pool (NULL: not reported) */
} qli_kwrite_params;

/* Enqueue the quantization of num_rows K rows and their scatter into the
 * paged index-K cache on `stream`: row i's INT8 values go to
 * k_cache + page * k_page_stride + row * 128 and its FP16 scale to
 * k_scale + page * s_page_stride + row * 2, with page, row = divmod(slot[i],
 * page_rows).  Slots must be distinct (two rows writing one slot race).
 * No allocation, no synchronisation; num_rows == 0 is a no-op.
 * Returns a qli_status. */
int qli_write_index_k(const qli_kwrite_params* p, void* stream);

/* ---- Consumer of the indices: sparse attention ------------------------
 *
 * The step after the indexer ("DeepSeek V4.1-Flash 登陆昇腾 · 需求故事（PR
 * 16925）", section 4: the compressed positions feed the two-stage sparse
 * attention; "DeepSeek V4.1-Flash CED·CSA2 架构拆解 × vllm-ascend 性能协助点",
 * operator table: a sliding window over recent tokens (SWA) and the
 * compressed global stage over the selected positions (CSA), with sinks;
 * BF16 TND queries and PA_BBND paged caches, the only layouts the developer
 * guide's "编译范围" builds).  The pages give no formula; this library
 * computes, for query token t of request b and head h:
 *   entries  E = { compressed rows indices[t][i] : 0 <= indices[t][i] < c_lens[b] }
 *              + { raw rows s : max(0, p - window + 1) <= s <= p },
 *              p = r_lens[b] - (q1 - q0) + (t - q0) the token's raw position
 *              (tokens q0..q1-1 of the request);
 *   z_j = scale * sum_d q[t][h][d] * kv_j[d]  (one latent KV head shared by
 *         all query heads; an entry's D values are its key and its value);
 *   out[t][h] = sum_j e^(z_j - m) kv_j / (sum_j e^(z_j - m) + e^(sink_h - m)),
 *         m the largest logit including the sink (no sink term when sinks is
 *         NULL); lse[t][h] = m + ln(denominator);
 *   no entry and no sink: out = 0, lse = -inf.
 * Products are exact, sums FP32, the softmax in base 2 on FP32 values; the
 * weights of the value sum are rounded to BF16 (the normalizer adds the same
 * rounded weights), and out is rounded to BF16 (RNE).  Tokens outside every
 * request get out = 0 and lse = -inf. */
typedef struct qli_attn_params {
  int32_t struct_size;      /* sizeof(qli_attn_params) */
  int32_t num_heads;        /* H: a multiple of 16, at most 128 */
  int32_t head_dim;         /* D: must be 512 */
  int32_t batch;            /* B >= 1 requests */
  int32_t num_tokens;       /* T >= 0 query tokens (T == 0: no-op) */
  int32_t topk;             /* width of an index row, 0 .. QLI_ATTN_MAX_TOPK */
  int32_t window;           /* raw positions of the window stage, 0 .. QLI_ATTN_MAX_WINDOW */
  int32_t c_page_rows;      /* rows per page of the compressed cache, 1 .. 256 */
  int32_t c_bt_stride;      /* entries per request row of c_block_table, >= 1 */
  int32_t r_page_rows;      /* rows per page of the raw cache, 1 .. 256 (window > 0) */
  int32_t r_bt_stride;      /* entries per request row of r_block_table (window > 0) */
  int32_t reserved0;        /* must be 0 */
  int64_t c_num_pages;      /* pages of the compressed pool, 1 .. 2^23 - 1 */
  int64_t r_num_pages;      /* pages of the raw pool, 1 .. 2^23 - 1 when window > 0 */
  int64_t c_page_stride;    /* bytes between compressed pages: a multiple of 16,
                               >= c_page_rows * D * 2; row r of page g starts at
                               g * c_page_stride + r * D * 2 */
  int64_t r_page_stride;    /* the same for the raw pool (window > 0) */
  float scale;              /* softmax scale, finite */
  int32_t reserved1;        /* must be 0 */
  const void* q;            /* BF16 [T][H][D] (16-B aligned) */
  const void* c_cache;      /* BF16 compressed pool, page 0 row 0 (16-B aligned) */
  const int32_t* c_block_table; /* [B][c_bt_stride] page ids; an id outside
                               [0, c_num_pages) drops the entry and raises
                               QLI_DEV_BAD_PAGE */
  const int32_t* c_lens;    /* [B] compressed lengths (>= 0) */
  const void* r_cache;      /* BF16 raw pool (16-B aligned; NULL when window == 0) */
  const int32_t* r_block_table; /* [B][r_bt_stride] (NULL when window == 0) */
  const int32_t* r_lens;    /* [B] raw lengths; r_lens[b] >= q1 - q0 (else the
                               request's tokens see no window entry and
                               QLI_DEV_BAD_METADATA is raised) */
  const int32_t* query_start_loc; /* [B + 1] non-decreasing, query_start_loc[0] == 0,
                               query_start_loc[B] == T */
  const int32_t* indices;   /* [T][topk] request-local compressed positions; < 0:
                               padding (skipped); >= c_lens[b]: skipped and
                               QLI_DEV_BAD_INDEX raised (NULL when topk == 0) */
  const float* sinks;       /* [H] one logit per head, or NULL */
  void* out;                /* BF16 [T][H][D] written (16-B aligned) */
  float* lse;               /* [T][H] written, or NULL */
  uint32_t* status_out;     /* optional device word receiving QLI_DEV_* bits (ORed) */
  void* workspace;          /* optional device scratch (256-B aligned, no initial
                               contents needed) for calls whose heads are a multiple
                               of 64: a token's entries are then split over several
                               workgroups, whose partial softmax states a second
                               launch merges from here.  Calls that share a workspace
                               must be ordered on one stream.  NULL (or too small for
                               any split): one workgroup per (token, 64 heads), one
                               launch, the same results up to FP32 rounding order */
  int64_t workspace_bytes;  /* bytes at workspace (>= 0) */
} qli_attn_params;

/* Enqueue the attention of num_tokens query tokens on `stream`: one launch
 * (two when the entries are split over a workspace), no allocation, no
 * synchronisation.  The host checks the parameters first
 * (QLI_ERR_INVALID_ARG / QLI_ERR_UNSUPPORTED, nothing launched); pointers
 * must be device memory, and every integer pointer 4-byte aligned.  Device
 * data outside the contract above is never read beyond the pools, tables
 * and arrays described; it is reported through status_out.
 * Returns a qli_status. */
int qli_sparse_attention(const qli_attn_params* p, void* stream);

/* Workspace bytes with which qli_sparse_attention splits each token's
 * entries over the most workgroups it would use for these scalars
 * (num_tokens, num_heads, topk, window; host-only).  0 when no split is
 * taken (p NULL, heads not a multiple of 64, or enough tokens to fill the
 * GPU without one). */
int64_t qli_attn_workspace_bytes(const qli_attn_params* p);

/* Kernels, in launch order within a call (for the timing facility below). */
enum qli_kernel { QLI_KERNEL_CONSUMER_PREP = 0, QLI_KERNEL_PLAN = 1, QLI_KERNEL_SCORE = 2,
                  QLI_KERNEL_SELECT = 3, QLI_KERNEL_QUANTIZE = 4, QLI_KERNEL_WRITE_K = 5,
                  QLI_KERNEL_ATTN = 6, QLI_KERNEL_ATTN_SPLIT = 7,
                  QLI_KERNEL_ATTN_MERGE = 8, QLI_NUM_KERNELS = 9 };

/* Optional per-kernel timing (off by default; process-wide, not thread
 * safe).  While enabled, every call of this library records a HIP event
 * before and after each kernel it launches, on the call's stream.
 * qli_timing_read() waits for the recorded events, adds each kernel's
 * elapsed milliseconds to ms[kernel] and its launch count to count[kernel]
 * (arrays of QLI_NUM_KERNELS entries, accumulated since the last reset),
 * and clears the totals when `reset` is non-zero.  Returns a qli_status. */
int qli_timing_enable(int on);
int qli_timing_read(double* ms, int64_t* count, int reset);

#ifdef __cplusplus
}
#endif

#endif /* QLI_H */
