/*
 * Oracle of the sparse-attention consumer of the indexer's positions (the
 * step after the indexer).
 *
 * TEST INFRASTRUCTURE ONLY, like qli_oracle.c: a plain, slow CPU
 * implementation in double precision used to check the GPU library; no
 * product code may call it.
 *
 * Sources:
 *   - "DeepSeek V4.1-Flash 登陆昇腾 · 需求故事（PR 16925）", section 4 (the
 *     attention forward excerpt): the indexer's compressed positions feed the
 *     two-stage sparse attention, whose per-head output has the head
 *     dimension and gets an inverse rotary embedding on its rope slice
 *     [nope_head_dim, head_dim) afterwards;
 *   - "DeepSeek V4.1-Flash CED·CSA2 架构拆解 × vllm-ascend 性能协助点", the
 *     operator table: the sparse attention is two stages, a sliding window
 *     over recent tokens (SWA) and the compressed global stage over the
 *     selected positions (CSA), with sinks and a mask mode; TND keeps the
 *     queries as token x head rows and PA_BBND keeps the keys in paged blocks
 *     x head;
 *   - "DeepSeek V4.1 QLI V2 与候选集成" (vllm-ascend developer guide),
 *     "编译范围": the operator is built for BF16 TND / PA_BBND SWA and CSA
 *     calls only.
 *
 * The pages name the stages and layouts but give no formula.  Readings
 * (each listed with its reason in the design notes of the repository):
 *   - one softmax per (query token, head) over the union of both stages'
 *     entries: the CSA entries are the token's row of the indexer's position
 *     top-k (request-local compressed positions, -1 padded) read from the
 *     compressed cache, the SWA entries are the last `window` raw positions
 *     of the token's causal view read from the raw cache;
 *   - one latent KV head shared by all query heads; an entry's D values are
 *     both its key and its value (the output carries the rope slice, which
 *     the excerpt rotates back afterwards);
 *   - logit z = scale * sum_d q[d] k[d] over BF16 q and k;
 *   - a sink is one logit per head that joins the normalizer and carries no
 *     value: out = sum_j e^(z_j - m) v_j / (sum_j e^(z_j - m) + e^(s - m)),
 *     m the largest logit including s; without sinks the last term is
 *     absent; no entry and no sink gives out = 0 and lse = -inf;
 *   - a CSA entry below 0 is padding and one at or beyond the request's
 *     compressed length is out of contract: both are skipped;
 *   - raw position of query token t of request b (tokens q0..q1-1, raw
 *     length S_b): S_b - (q1 - q0) + (t - q0); the window is the positions
 *     max(0, p - window + 1) .. p;
 *   - every entry counts once per occurrence in the lists.
 * Everything is computed in double precision (exact BF16 inputs, exact
 * products); out is returned in double, lse = m + log(den).
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

typedef struct {
  int32_t num_heads;   /* H */
  int32_t head_dim;    /* D: key and value width of an entry */
  int32_t batch;       /* B requests */
  int32_t num_tokens;  /* T query tokens */
  int32_t topk;        /* width of a row of indices */
  int32_t window;      /* SWA window (0: no window stage) */
  int32_t c_page_rows, c_bt_stride; /* compressed cache pages and block table */
  int32_t r_page_rows, r_bt_stride; /* raw cache pages and block table */
  int64_t c_page_stride;            /* bytes between compressed pages */
  int64_t r_page_stride;            /* bytes between raw pages */
  double scale;
  const uint16_t* q;            /* BF16 [T][H][D] */
  const void* c_kv;             /* BF16 rows of D values, paged */
  const int32_t* c_bt;          /* [B][c_bt_stride] */
  const int32_t* c_lens;        /* [B] compressed lengths */
  const void* r_kv;
  const int32_t* r_bt;
  const int32_t* r_lens;        /* [B] raw lengths */
  const int32_t* query_start_loc; /* [B + 1] */
  const int32_t* indices;       /* [T][topk] */
  const float* sinks;           /* [H] or NULL */
} OracleAttn;

static double bf16_value(uint16_t h) {
  uint32_t u = (uint32_t)h << 16;
  float f;
  memcpy(&f, &u, 4);
  return (double)f;
}

/* The D BF16 values of row `pos` of one request's paged cache. */
static const uint16_t* cache_row(const void* base, const int32_t* bt_row, int page_rows, int64_t page_stride,
                                 int D, int pos) {
  const int32_t page = bt_row[pos / page_rows];
  const int row = pos % page_rows;
  return (const uint16_t*)((const char*)base + (int64_t)page * page_stride + (int64_t)row * D * 2);
}

/* Request of global token t, or -1. */
static int request_of_token(const OracleAttn* P, int t) {
  for (int b = 0; b < P->batch; ++b)
    if (P->query_start_loc[b] <= t && t < P->query_start_loc[b + 1]) return b;
  return -1;
}

/* The entries of token t (rows of D BF16 values), CSA first, then SWA;
 * returns their count (at most topk + window). */
static int token_entries(const OracleAttn* P, int t, const uint16_t** rows) {
  const int b = request_of_token(P, t);
  if (b < 0) return 0;
  const int D = P->head_dim;
  int n = 0;
  const int32_t* idx = P->indices + (int64_t)t * P->topk;
  for (int i = 0; i < P->topk; ++i) {
    const int c = idx[i];
    if (c < 0 || c >= P->c_lens[b]) continue;
    rows[n++] = cache_row(P->c_kv, P->c_bt + (int64_t)b * P->c_bt_stride, P->c_page_rows, P->c_page_stride, D, c);
  }
  if (P->window > 0) {
    const int q0 = P->query_start_loc[b], q1 = P->query_start_loc[b + 1];
    const int64_t p = (int64_t)P->r_lens[b] - (q1 - q0) + (t - q0);
    for (int64_t s = p - P->window + 1; s <= p; ++s) {
      if (s < 0) continue;
      rows[n++] = cache_row(P->r_kv, P->r_bt + (int64_t)b * P->r_bt_stride, P->r_page_rows, P->r_page_stride, D,
                            (int)s);
    }
  }
  return n;
}

/* out[i][h][d] and lse[i][h] (either may be NULL) of tokens[0..n). */
int oracle_sparse_attn(const OracleAttn* P, const int32_t* tokens, int n, double* out, double* lse) {
  const int H = P->num_heads, D = P->head_dim;
  if (H <= 0 || D <= 0 || P->topk < 0 || P->window < 0) return 1;
  const int cap = P->topk + P->window;
  const uint16_t** rows = (const uint16_t**)malloc(sizeof(const uint16_t*) * (size_t)(cap > 0 ? cap : 1));
  double* z = (double*)malloc(sizeof(double) * (size_t)(cap > 0 ? cap : 1));
  double* w = (double*)malloc(sizeof(double) * (size_t)(cap > 0 ? cap : 1));
  if (!rows || !z || !w) {
    free(rows);
    free(z);
    free(w);
    return 2;
  }
  for (int i = 0; i < n; ++i) {
    const int t = tokens[i];
    if (t < 0 || t >= P->num_tokens) {
      free(rows);
      free(z);
      free(w);
      return 3;
    }
    const int ne = token_entries(P, t, rows);
    for (int h = 0; h < H; ++h) {
      const uint16_t* qrow = P->q + ((int64_t)t * H + h) * D;
      double m = -INFINITY;
      for (int j = 0; j < ne; ++j) {
        double acc = 0.0;
        for (int d = 0; d < D; ++d) acc += bf16_value(qrow[d]) * bf16_value(rows[j][d]);
        z[j] = P->scale * acc;
        if (z[j] > m) m = z[j];
      }
      const int has_sink = P->sinks != NULL;
      const double s = has_sink ? (double)P->sinks[h] : 0.0;
      if (has_sink && s > m) m = s;
      double den = 0.0;
      for (int j = 0; j < ne; ++j) {
        w[j] = exp(z[j] - m);
        den += w[j];
      }
      if (has_sink) den += exp(s - m);
      double* o = out ? out + ((int64_t)i * H + h) * D : NULL;
      if (o) {
        for (int d = 0; d < D; ++d) {
          double acc = 0.0;
          for (int j = 0; j < ne; ++j) acc += w[j] * bf16_value(rows[j][d]);
          o[d] = den > 0.0 ? acc / den : 0.0;
        }
      }
      if (lse) lse[(int64_t)i * H + h] = den > 0.0 ? m + log(den) : -INFINITY;
    }
  }
  free(rows);
  free(z);
  free(w);
  return 0;
}
