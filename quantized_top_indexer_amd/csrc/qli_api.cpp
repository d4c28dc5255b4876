// Host entry points of the QLI library: argument validation, workspace
// sizing and status strings.  Validation mirrors the host-side checks the
// QLI developer guide describes ("数据流": unsupported layouts are rejected
// on the host before any kernel runs; the residual tensor must be absent at
// ratio 1) and the contract limits of its "当前 A3 契约" section.
#include <stdint.h>

#include <cmath>
#include <climits>

#include "qli.h"
#include "qli_internal.h"

namespace {

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

bool cand_width_ok(int32_t w) { return w >= 64 && w <= QLI_MAX_CAND_BLOCKS && w % 64 == 0; }

// Checks that need no pointer; shared by qli_validate and qli_workspace_bytes.
int check_scalars(const qli_params* p) {
  if (!p || p->struct_size != sizeof(qli_params)) return QLI_ERR_INVALID_ARG;
  if (p->head_dim != 128) return QLI_ERR_UNSUPPORTED;
  if (p->quant_mode != QLI_QUANT_INT8) return QLI_ERR_UNSUPPORTED;
  if (p->num_heads != 32 && p->num_heads != 64) return QLI_ERR_UNSUPPORTED;
  if (p->mode < QLI_MODE_PLAIN || p->mode > QLI_MODE_CONSUMER) return QLI_ERR_INVALID_ARG;
  if (p->ratio != 1 && p->ratio != 2) return QLI_ERR_INVALID_ARG;
  if (p->page_rows != 128 / p->ratio) return QLI_ERR_INVALID_ARG;
  if (p->batch < 0 || p->num_tokens < 0 || p->reserved0 != 0) return QLI_ERR_INVALID_ARG;
  if (p->num_tokens > 0 && p->batch < 1) return QLI_ERR_INVALID_ARG;
  if (p->topk < 1 || p->topk > QLI_MAX_TOPK) return QLI_ERR_INVALID_ARG;
  if (p->mode == QLI_MODE_SOURCE && !cand_width_ok(p->cand_blocks)) return QLI_ERR_INVALID_ARG;
  if (p->mode == QLI_MODE_CONSUMER && !cand_width_ok(p->cand_in_blocks))
    return QLI_ERR_INVALID_ARG;
  if (p->max_k_len < 0) return QLI_ERR_INVALID_ARG;
  if (p->max_k_len > QLI_MAX_K_LEN) return QLI_ERR_UNSUPPORTED;
  if (p->bt_stride < 1 || p->num_pages < 1) return QLI_ERR_INVALID_ARG;
  if (static_cast<int64_t>(p->bt_stride) * p->page_rows < p->max_k_len) return QLI_ERR_INVALID_ARG;
  if (p->k_page_stride < static_cast<int64_t>(p->page_rows) * 128 || p->k_page_stride % 16)
    return QLI_ERR_INVALID_ARG;
  if (p->s_page_stride < static_cast<int64_t>(p->page_rows) * 2 || p->s_page_stride % 16)
    return QLI_ERR_INVALID_ARG;
  // one workgroup per (token, 256-slot chunk) must fit a 31-bit grid
  const qli::WsLayout w = qli::ws_layout(p, p->num_tokens);
  if (static_cast<int64_t>(p->num_tokens) * (w.ncap / qli::kChunk) >= (int64_t(1) << 31))
    return QLI_ERR_UNSUPPORTED;
  return QLI_OK;
}

// Every check of a call except the workspace's (shared by the two entry
// points that enqueue the indexer).
int check_args(const qli_params* p) {
  int rc = check_scalars(p);
  if (rc != QLI_OK) return rc;
  // residual: the guide requires it to be absent at ratio 1; ratio 2 needs it
  if (p->ratio == 1 && p->seq_mod) return QLI_ERR_INVALID_ARG;
  if (p->mode == QLI_MODE_CONSUMER && !p->cand_in) return QLI_ERR_NO_SOURCE;
  if (p->num_tokens == 0) return QLI_OK;
  if (p->ratio == 2 && !p->seq_mod) return QLI_ERR_INVALID_ARG;
  if (!p->q || !p->q_scale || !p->weights || !p->k_cache || !p->k_scale || !p->block_table ||
      !p->query_start_loc || !p->k_lens || !p->topk_out)
    return QLI_ERR_INVALID_ARG;
  if (p->mode == QLI_MODE_SOURCE && !p->cand_out) return QLI_ERR_INVALID_ARG;
  if (p->dbg_qk && (!p->dbg_scores || !aligned(p->dbg_qk, 4))) return QLI_ERR_INVALID_ARG;
  if (!aligned(p->q, 16) || !aligned(p->k_cache, 16) || !aligned(p->k_scale, 16) ||
      !aligned(p->q_scale, 2) || !aligned(p->weights, 2) || !aligned(p->block_table, 4) ||
      !aligned(p->query_start_loc, 4) || !aligned(p->k_lens, 4) || !aligned(p->topk_out, 4))
    return QLI_ERR_INVALID_ARG;
  // optional and mode-dependent pointers (NULL passes): 32-bit words, and
  // the status word takes device atomics
  if (!aligned(p->seq_mod, 4) || !aligned(p->cand_in, 4) || !aligned(p->cand_out, 4) ||
      !aligned(p->dbg_scores, 4) || !aligned(p->status_out, 4))
    return QLI_ERR_INVALID_ARG;
  return QLI_OK;
}

bool dtype_ok(int32_t d) { return d == QLI_DTYPE_F32 || d == QLI_DTYPE_BF16; }

int check_quant(const qli_quant_params* p) {
  if (!p || p->struct_size != sizeof(qli_quant_params)) return QLI_ERR_INVALID_ARG;
  if (p->head_dim != 128) return QLI_ERR_UNSUPPORTED;
  if (!dtype_ok(p->x_dtype) || !dtype_ok(p->w_dtype)) return QLI_ERR_UNSUPPORTED;
  if (p->num_rows < 0 || p->num_weights < 0) return QLI_ERR_INVALID_ARG;
  if (p->num_rows > 0) {
    if (!p->x || !p->q || !p->q_scale) return QLI_ERR_INVALID_ARG;
    if (!aligned(p->x, 16) || !aligned(p->q, 16) || !aligned(p->q_scale, 2)) return QLI_ERR_INVALID_ARG;
  }
  if (p->num_weights > 0) {
    if (!p->w || !p->w_out) return QLI_ERR_INVALID_ARG;
    if (!aligned(p->w, p->w_dtype == QLI_DTYPE_F32 ? 4 : 2) || !aligned(p->w_out, 2))
      return QLI_ERR_INVALID_ARG;
  }
  return QLI_OK;
}

int check_kwrite(const qli_kwrite_params* p) {
  if (!p || p->struct_size != sizeof(qli_kwrite_params)) return QLI_ERR_INVALID_ARG;
  if (p->head_dim != 128) return QLI_ERR_UNSUPPORTED;
  if (!dtype_ok(p->x_dtype)) return QLI_ERR_UNSUPPORTED;
  if (p->num_rows < 0 || p->reserved0 != 0) return QLI_ERR_INVALID_ARG;
  if (p->page_rows != 64 && p->page_rows != 128) return QLI_ERR_INVALID_ARG;
  // pool rows (num_pages * page_rows) must not overflow a 64-bit slot
  if (p->num_pages < 1 || p->num_pages > (int64_t(1) << 40)) return QLI_ERR_INVALID_ARG;
  if (p->k_page_stride < static_cast<int64_t>(p->page_rows) * 128 || p->k_page_stride % 16)
    return QLI_ERR_INVALID_ARG;
  if (p->s_page_stride < static_cast<int64_t>(p->page_rows) * 2 || p->s_page_stride % 2)
    return QLI_ERR_INVALID_ARG;
  if (p->num_rows == 0) return QLI_OK;
  if (!p->x || !p->slot || !p->k_cache || !p->k_scale) return QLI_ERR_INVALID_ARG;
  if (!aligned(p->x, 16) || !aligned(p->slot, 8) || !aligned(p->k_cache, 16) ||
      !aligned(p->k_scale, 2) || !aligned(p->status_out, 4))
    return QLI_ERR_INVALID_ARG;
  return QLI_OK;
}

int check_attn(const qli_attn_params* p) {
  if (!p || p->struct_size != sizeof(qli_attn_params)) return QLI_ERR_INVALID_ARG;
  if (p->head_dim != 512) return QLI_ERR_UNSUPPORTED;
  if (p->num_heads < 16 || p->num_heads > 128 || p->num_heads % 16) return QLI_ERR_UNSUPPORTED;
  if (p->reserved0 != 0 || p->reserved1 != 0) return QLI_ERR_INVALID_ARG;
  if (p->batch < 1 || p->num_tokens < 0) return QLI_ERR_INVALID_ARG;
  if (p->topk < 0 || p->topk > QLI_ATTN_MAX_TOPK) return QLI_ERR_INVALID_ARG;
  if (p->window < 0 || p->window > QLI_ATTN_MAX_WINDOW) return QLI_ERR_INVALID_ARG;
  if (!std::isfinite(p->scale)) return QLI_ERR_INVALID_ARG;
  const int64_t row_bytes = int64_t(512) * 2;
  // the kernel packs an entry as page (23 bits) and row (8 bits)
  if (p->c_page_rows < 1 || p->c_page_rows > 256 || p->c_bt_stride < 1 || p->c_num_pages < 1 ||
      p->c_num_pages >= (int64_t(1) << 23))
    return QLI_ERR_INVALID_ARG;
  if (p->c_page_stride % 16 || p->c_page_stride < p->c_page_rows * row_bytes) return QLI_ERR_INVALID_ARG;
  // every address the kernel forms stays within 2^62 bytes of the pool base
  if (p->c_num_pages > (int64_t(1) << 62) / p->c_page_stride) return QLI_ERR_INVALID_ARG;
  if (int64_t(p->c_bt_stride) * p->c_page_rows > INT32_MAX) return QLI_ERR_INVALID_ARG;
  if (p->window > 0) {
    if (p->r_page_rows < 1 || p->r_page_rows > 256 || p->r_bt_stride < 1 || p->r_num_pages < 1 ||
        p->r_num_pages >= (int64_t(1) << 23))
      return QLI_ERR_INVALID_ARG;
    if (p->r_page_stride % 16 || p->r_page_stride < p->r_page_rows * row_bytes) return QLI_ERR_INVALID_ARG;
    if (p->r_num_pages > (int64_t(1) << 62) / p->r_page_stride) return QLI_ERR_INVALID_ARG;
    if (int64_t(p->r_bt_stride) * p->r_page_rows > INT32_MAX) return QLI_ERR_INVALID_ARG;
  }
  if (p->num_tokens == 0) return QLI_OK;
  if (!p->q || !p->c_cache || !p->c_block_table || !p->c_lens || !p->query_start_loc || !p->out)
    return QLI_ERR_INVALID_ARG;
  if (p->topk > 0 && !p->indices) return QLI_ERR_INVALID_ARG;
  if (p->window > 0 && (!p->r_cache || !p->r_block_table || !p->r_lens)) return QLI_ERR_INVALID_ARG;
  if (!aligned(p->q, 16) || !aligned(p->c_cache, 16) || !aligned(p->r_cache, 16) || !aligned(p->out, 16))
    return QLI_ERR_INVALID_ARG;
  if (!aligned(p->c_block_table, 4) || !aligned(p->c_lens, 4) || !aligned(p->r_block_table, 4) ||
      !aligned(p->r_lens, 4) || !aligned(p->query_start_loc, 4) || !aligned(p->indices, 4) ||
      !aligned(p->sinks, 4) || !aligned(p->lse, 4) || !aligned(p->status_out, 4))
    return QLI_ERR_INVALID_ARG;
  if (p->workspace_bytes < 0 || !aligned(p->workspace, 256)) return QLI_ERR_INVALID_ARG;
  return QLI_OK;
}

}  // namespace

extern "C" {

int qli_sparse_attention(const qli_attn_params* p, void* stream) {
  const int rc = check_attn(p);
  if (rc != QLI_OK) return rc;
  if (p->num_tokens == 0) return QLI_OK;
  return qli::launch_attention(p, stream);
}

int64_t qli_attn_workspace_bytes(const qli_attn_params* p) {
  if (!p || p->num_tokens <= 0 || p->num_heads <= 0 || p->topk < 0 || p->window < 0) return 0;
  return qli::attention_workspace_bytes(p->num_tokens, p->num_heads, p->topk, p->window,
                                        qli::attention_splits(p->num_tokens, p->num_heads, p->topk, p->window));
}

int qli_quantize_query(const qli_quant_params* p, void* stream) {
  const int rc = check_quant(p);
  if (rc != QLI_OK) return rc;
  if (p->num_rows == 0 && p->num_weights == 0) return QLI_OK;
  return qli::launch_quantize(p, stream);
}

int qli_write_index_k(const qli_kwrite_params* p, void* stream) {
  const int rc = check_kwrite(p);
  if (rc != QLI_OK) return rc;
  if (p->num_rows == 0) return QLI_OK;
  return qli::launch_write_k(p, stream);
}

int qli_abi_version(void) { return QLI_ABI_VERSION; }

int qli_validate(const qli_params* p) {
  const int rc = check_args(p);
  if (rc != QLI_OK || p->num_tokens == 0) return rc;
  // the workspace must hold a slice of at least one token
  if (!p->workspace || !aligned(p->workspace, 256)) return QLI_ERR_WORKSPACE;
  if (qli::slice_layout(p, p->workspace_bytes).tokens < 1) return QLI_ERR_WORKSPACE;
  return QLI_OK;
}

size_t qli_workspace_bytes(const qli_params* p) {
  if (check_scalars(p) != QLI_OK) return 0;
  return qli::default_layout(p).total;
}

int qli_score_topk(const qli_params* p, void* stream) {
  int rc = qli_validate(p);
  if (rc != QLI_OK) return rc;
  if (p->num_tokens == 0) return QLI_OK;
  return qli::launch(p, qli::slice_layout(p, p->workspace_bytes), stream, true);
}

int qli_score_topk_noalloc(const qli_params* p, void* stream) {
  int rc = check_args(p);
  if (rc != QLI_OK) return rc;
  if (p->num_tokens == 0) return QLI_OK;
  // slices of as many tokens as the static array holds
  const qli::WsLayout w = qli::slice_layout(p, QLI_STATIC_SCRATCH_BYTES);
  if (w.tokens < 1) return QLI_ERR_SCRATCH_LIMIT;
  void* scratch = nullptr;
  rc = qli::static_scratch(&scratch);
  if (rc != QLI_OK) return rc;
  qli_params q = *p;
  q.workspace = scratch;
  q.workspace_bytes = QLI_STATIC_SCRATCH_BYTES;
  // no timing events either: recording them creates HIP events
  return qli::launch(&q, w, stream, false);
}


int qli_timing_enable(int on) { return qli::timing_enable(on); }

int qli_timing_read(double* ms, int64_t* count, int reset) {
  return qli::timing_read(ms, count, reset);
}

const char* qli_status_string(int status) {
  switch (status) {
    case QLI_OK: return "QLI_OK";
    case QLI_ERR_INVALID_ARG: return "QLI_ERR_INVALID_ARG: argument out of contract";
    case QLI_ERR_UNSUPPORTED: return "QLI_ERR_UNSUPPORTED: heads/dim/quant mode/size not supported";
    case QLI_ERR_NO_SOURCE: return "QLI_ERR_NO_SOURCE: consumer mode needs incoming candidates";
    case QLI_ERR_WORKSPACE: return "QLI_ERR_WORKSPACE: workspace missing or too small";
    case QLI_ERR_HIP: return "QLI_ERR_HIP: kernel launch failed";
    case QLI_ERR_SCRATCH_LIMIT:
      return "QLI_ERR_SCRATCH_LIMIT: the call needs more than the static scratch of "
             "qli_score_topk_noalloc (QLI_STATIC_SCRATCH_BYTES); use qli_score_topk with a workspace";
    default: return "QLI: unknown status";
  }
}

}  // extern "C"
