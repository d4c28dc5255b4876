/*
 * Oracle for the DeepSeek V4.1 quantized lightning indexer (QLI) with
 * hierarchical candidate blocks.
 *
 * TEST INFRASTRUCTURE ONLY.  This is a plain, slow, brute-force CPU
 * implementation of what the indexer computes, used to check the GPU
 * library.  It shares no code, header, table or helper with the GPU path,
 * and no product code may call it.
 *
 * Source: "DeepSeek V4.1 QLI V2 与候选集成" (vllm-ascend developer guide),
 *   - "数据流" (data flow): TND queries, paged PA_BBND index K with a
 *     per-token FP16 scale, metadata = raw query boundaries + compressed K
 *     lengths + raw length mod ratio; candidates are INT32 block ids
 *     [tokens, 1, candidate_topk_blocks], -1 padded; a block is 8
 *     compressed positions scored by its maximum position score; the last
 *     visible block is pinned; returned positions are sorted
 *     chronologically with -1 padding moved to the end; an empty
 *     compressed context gives empty indices and, for a source, all
 *     invalid candidates; a consumer without a source is an error.
 *   - "当前 A3 契约" (current A3 contract): INT8 Q/K, FP16 head weights,
 *     per-head Q scale and per-token K scale; 32 or 64 index heads of dim
 *     128 and one K head; ratios 1 and 2 with causal mask mode 3; position
 *     top-k in [1, 2048]; candidate widths multiples of 64 in [64, 2048];
 *     the golden order: INT32 Q.K divided by 1024, FP16 ReLU and
 *     weight * Q_scale, FP32 reduction over heads, then the K scale.
 *
 * Readings taken where the page is silent (each is listed with its reason
 * in the design notes of the repository):
 *   - "divided by 1024" is exact real division followed by one
 *     round-to-nearest-even (RNE) conversion to FP16;
 *   - every rounding is IEEE RNE, FP16 subnormals are kept;
 *   - the FP16 steps are x = fp16(qk/1024), x = max(x, +0),
 *     m = fp16(w * q_scale), p = fp16(x * m); the FP32 head reduction
 *     starts at +0.0f and adds p in ascending head order, one FP32 RNE per
 *     addition; score = fp32(sum * k_scale);
 *   - causal visibility: the queries of a request are its last raw
 *     positions; query at raw position p sees compressed entries
 *     j < floor((p + 1) / ratio);
 *   - ties: higher score first, then lower position (blocks: higher block
 *     score, then lower block id); -0 ranks equal to +0;
 *   - candidate output: the selected block ids in ascending order, -1 tail;
 *   - modes: 1 plain (positions only), 2 candidate source (positions and
 *     candidates), 3 candidate consumer (positions restricted to the
 *     incoming candidate blocks; negative ids ignored, duplicates collapse,
 *     ids without a visible position contribute nothing).
 *
 * Arithmetic is carried in double wherever the intermediate is exact
 * there (qk/1024, a product of two FP16 values, float+fp16 sums of this
 * range), so each documented rounding happens exactly once, in
 * oracle_f16_round() or in a C float operation (SSE, FLT_EVAL_METHOD 0,
 * built with -ffp-contract=off).
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define ORACLE_HEAD_DIM 128
#define ORACLE_BLOCK 8

typedef struct oracle_problem {
  int32_t mode;            /* 1 plain, 2 source, 3 consumer */
  int32_t ratio;           /* 1 or 2 */
  int32_t num_heads;       /* N */
  int32_t batch;           /* B */
  int32_t num_tokens;      /* T */
  int32_t topk;            /* k */
  int32_t cand_blocks;     /* cb (mode 2) */
  int32_t cand_in_blocks;  /* incoming candidate width (mode 3) */
  int32_t page_rows;       /* rows per page view */
  int32_t bt_stride;       /* block-table row length */
  int32_t num_pages;       /* pages in the pool */
  int32_t pad0;
  int64_t k_page_stride;   /* bytes between pages of the K view */
  int64_t s_page_stride;   /* bytes between pages of the scale view */
  const int8_t* q;         /* [T, N, 128] */
  const uint16_t* q_scale; /* fp16 [T, N] */
  const uint16_t* weights; /* fp16 [T, N] */
  const int8_t* k_base;    /* row 0 of page 0, K view */
  const uint8_t* s_base;   /* row 0 of page 0, scale view (fp16) */
  const int32_t* block_table;     /* [B, bt_stride] */
  const int32_t* query_start_loc; /* [B + 1] */
  const int32_t* k_lens;          /* [B] compressed lengths */
  const int32_t* seq_mod;         /* [B] raw length mod ratio, NULL at ratio 1 */
  const int32_t* cand_in;         /* [T, 1, cand_in_blocks] (mode 3) */
} oracle_problem;

/* ---- IEEE binary16 ---------------------------------------------------- */

/* Round a real number (given exactly as a double) to the nearest binary16,
 * ties to even, with gradual underflow and overflow to infinity. */
uint16_t oracle_f16_round(double x) {
  uint16_t sign = signbit(x) ? 0x8000u : 0u;
  if (isnan(x)) return 0x7E00u;
  double a = fabs(x);
  if (a == 0.0) return sign;
  if (isinf(a)) return (uint16_t)(sign | 0x7C00u);
  int e;
  (void)frexp(a, &e); /* a in [2^(e-1), 2^e) */
  int E = e - 1;
  if (E < -14) E = -14; /* subnormals share the quantum 2^-24 */
  double m = nearbyint(ldexp(a, 10 - E)); /* significand in units of 2^(E-10), RNE */
  if (E == -14 && m < 1024.0) return (uint16_t)(sign | (uint16_t)m); /* subnormal or zero */
  if (m >= 2048.0) { /* rounded up into the next binade */
    m = 1024.0;
    E += 1;
  }
  if (E + 15 >= 31) return (uint16_t)(sign | 0x7C00u);
  return (uint16_t)(sign | (uint16_t)((E + 15) << 10) | (uint16_t)(m - 1024.0));
}

double oracle_f16_value(uint16_t h) {
  int e = (h >> 10) & 31, f = h & 1023;
  double v;
  if (e == 0) v = ldexp((double)f, -24);
  else if (e == 31) v = f ? NAN : INFINITY;
  else v = ldexp((double)(f + 1024), e - 25);
  return (h & 0x8000u) ? -v : v;
}

void oracle_f16_round_array(const double* x, uint16_t* out, int64_t n) {
  for (int64_t i = 0; i < n; ++i) out[i] = oracle_f16_round(x[i]);
}

void oracle_f16_value_array(const uint16_t* h, double* out, int64_t n) {
  for (int64_t i = 0; i < n; ++i) out[i] = oracle_f16_value(h[i]);
}

/* ---- metadata --------------------------------------------------------- */

/* Request of token t and the number of compressed entries it sees.
 * Returns 0, or -1 when the metadata is inconsistent. */
int oracle_token_view(const oracle_problem* P, int t, int* b_out, int* V_out) {
  int b = -1;
  for (int r = 0; r < P->batch; ++r)
    if (P->query_start_loc[r] <= t && t < P->query_start_loc[r + 1]) { b = r; break; }
  if (b < 0) return -1;
  int64_t n = P->query_start_loc[b + 1] - P->query_start_loc[b];
  int64_t L = P->k_lens[b];
  int64_t s = P->seq_mod ? P->seq_mod[b] : 0;
  if (L < 0 || s < 0 || s >= P->ratio) return -1;
  int64_t S = L * P->ratio + s; /* raw length */
  if (n > S) return -1;
  int64_t i = t - P->query_start_loc[b];
  int64_t p = S - n + i; /* raw position of this query */
  int64_t V = (p + 1) / P->ratio;
  *b_out = b;
  *V_out = (int)V;
  return 0;
}

/* ---- scoring ------------------------------------------------------------ */

typedef struct {
  int32_t qk[256];
  uint16_t x[256], m[256], p[256];
  float score;
  float sum;
  int64_t exact_sum_q24; /* sum_h p_h exactly, in units of 2^-24 */
  double abs_sum;        /* k_scale * sum_h |p_h| */
} oracle_terms;

static int locate(const oracle_problem* P, int b, int j, const int8_t** krow, uint16_t* ks) {
  int blk = j / P->page_rows, row = j % P->page_rows;
  if (blk >= P->bt_stride) return -1;
  int page = P->block_table[(int64_t)b * P->bt_stride + blk];
  if (page < 0 || page >= P->num_pages) return -1;
  *krow = P->k_base + (int64_t)page * P->k_page_stride + (int64_t)row * ORACLE_HEAD_DIM;
  const uint8_t* sp = P->s_base + (int64_t)page * P->s_page_stride + (int64_t)row * 2;
  *ks = (uint16_t)(sp[0] | (sp[1] << 8));
  return 0;
}

/* Score of compressed position j for token t (request b), following the
 * golden order step by step.  Fills the per-head terms when asked. */
static int score_one(const oracle_problem* P, int t, int b, int j, const uint16_t* mh,
                     float* score_out, oracle_terms* terms) {
  const int8_t* krow;
  uint16_t ks;
  if (locate(P, b, j, &krow, &ks)) return -1;
  const int N = P->num_heads;
  float sum = 0.0f;
  int64_t exact = 0;
  double absum = 0.0;
  for (int h = 0; h < N; ++h) {
    const int8_t* qrow = P->q + ((int64_t)t * N + h) * ORACLE_HEAD_DIM;
    int32_t acc = 0;
    for (int d = 0; d < ORACLE_HEAD_DIM; ++d) acc += (int32_t)qrow[d] * (int32_t)krow[d];
    uint16_t x = oracle_f16_round((double)acc / 1024.0);        /* INT32 / 1024 -> FP16 */
    if (!(oracle_f16_value(x) > 0.0)) x = 0;                      /* FP16 ReLU, +0 */
    uint16_t p = oracle_f16_round(oracle_f16_value(x) * oracle_f16_value(mh[h])); /* FP16 */
    double pv = oracle_f16_value(p);
    sum = sum + (float)pv;                                        /* FP32, ascending h */
    exact += (int64_t)llround(ldexp(pv, 24));
    absum += fabs(pv);
    if (terms) {
      terms->qk[h] = acc;
      terms->x[h] = x;
      terms->m[h] = mh[h];
      terms->p[h] = p;
    }
  }
  float kscale = (float)oracle_f16_value(ks);
  float score = sum * kscale; /* FP32 K scaling after the head reduction */
  *score_out = score;
  if (terms) {
    terms->score = score;
    terms->sum = sum;
    terms->exact_sum_q24 = exact;
    terms->abs_sum = absum * oracle_f16_value(ks);
  }
  return 0;
}

static void head_multipliers(const oracle_problem* P, int t, uint16_t* mh) {
  for (int h = 0; h < P->num_heads; ++h) {
    int64_t o = (int64_t)t * P->num_heads + h;
    mh[h] = oracle_f16_round(oracle_f16_value(P->weights[o]) * oracle_f16_value(P->q_scale[o]));
  }
}

int oracle_score_terms(const oracle_problem* P, int t, int j, oracle_terms* out) {
  int b, V;
  if (P->num_heads > 256 || oracle_token_view(P, t, &b, &V)) return -1;
  uint16_t mh[256];
  head_multipliers(P, t, mh);
  float s;
  return score_one(P, t, b, j, mh, &s, out);
}

/* ---- selection ------------------------------------------------------------ */

typedef struct {
  float key;
  int32_t id;
} ranked;

/* higher key first, then lower id; -0 == +0 under float comparison */
static int by_key_desc_id_asc(const void* pa, const void* pb) {
  const ranked* a = (const ranked*)pa;
  const ranked* b = (const ranked*)pb;
  if (a->key > b->key) return -1;
  if (a->key < b->key) return 1;
  return (a->id > b->id) - (a->id < b->id);
}

static int int_asc(const void* pa, const void* pb) {
  int32_t a = *(const int32_t*)pa, b = *(const int32_t*)pb;
  return (a > b) - (a < b);
}

/* ---- one token -------------------------------------------------------------- */

typedef struct {
  const oracle_problem* P;
  const int32_t* tokens;
  int ntok;
  int32_t* topk_out;
  int32_t* cand_out;
  float* scores_out;
  int score_cols;
  int next;
  int error;
} job;

static int run_token(const oracle_problem* P, int t, int32_t* topk_out, int32_t* cand_out,
                     float* scores_out, int score_cols) {
  int b, V;
  if (oracle_token_view(P, t, &b, &V)) return -1;
  const int k = P->topk;
  for (int s = 0; s < k; ++s) topk_out[s] = -1;
  if (P->mode == 2)
    for (int s = 0; s < P->cand_blocks; ++s) cand_out[s] = -1;
  if (scores_out)
    for (int c = 0; c < score_cols; ++c) scores_out[c] = NAN;
  if (V <= 0) return 0; /* empty compressed context: all -1 */

  const int nblocks = (V + ORACLE_BLOCK - 1) / ORACLE_BLOCK;
  unsigned char* eligible = (unsigned char*)calloc((size_t)V, 1);
  float* score = (float*)malloc(sizeof(float) * (size_t)V);
  ranked* list = (ranked*)malloc(sizeof(ranked) * (size_t)(V > nblocks ? V : nblocks));
  int32_t* chosen = (int32_t*)malloc(sizeof(int32_t) * (size_t)(V > nblocks ? V : nblocks));
  if (!eligible || !score || !list || !chosen) {
    free(eligible); free(score); free(list); free(chosen);
    return -2;
  }
  if (P->mode == 3) {
    for (int s = 0; s < P->cand_in_blocks; ++s) {
      int c = P->cand_in[(int64_t)t * P->cand_in_blocks + s];
      if (c < 0 || c >= nblocks) continue; /* ignored / no visible position */
      for (int j = c * ORACLE_BLOCK; j < (c + 1) * ORACLE_BLOCK && j < V; ++j) eligible[j] = 1;
    }
  } else {
    memset(eligible, 1, (size_t)V);
  }

  uint16_t mh[256];
  head_multipliers(P, t, mh);
  int count = 0, rc = 0;
  for (int j = 0; j < V && !rc; ++j) {
    if (!eligible[j]) continue;
    rc = score_one(P, t, b, j, mh, &score[j], NULL);
    if (rc) break;
    if (scores_out && j < score_cols) scores_out[j] = score[j];
    list[count].key = score[j];
    list[count].id = j;
    ++count;
  }
  if (!rc) {
    /* position top-k: rank by (score desc, position asc), emit ascending */
    qsort(list, (size_t)count, sizeof(ranked), by_key_desc_id_asc);
    int take = count < k ? count : k;
    for (int s = 0; s < take; ++s) chosen[s] = list[s].id;
    qsort(chosen, (size_t)take, sizeof(int32_t), int_asc);
    for (int s = 0; s < take; ++s) topk_out[s] = chosen[s];

    if (P->mode == 2) {
      /* block score = max visible position score; last visible block pinned */
      const int last = nblocks - 1;
      int nb = 0;
      for (int c = 0; c < last; ++c) {
        float m = score[c * ORACLE_BLOCK];
        for (int j = c * ORACLE_BLOCK + 1; j < (c + 1) * ORACLE_BLOCK; ++j)
          if (score[j] > m) m = score[j];
        list[nb].key = m;
        list[nb].id = c;
        ++nb;
      }
      qsort(list, (size_t)nb, sizeof(ranked), by_key_desc_id_asc);
      int cb = P->cand_blocks;
      int others = nb < cb - 1 ? nb : cb - 1;
      for (int s = 0; s < others; ++s) chosen[s] = list[s].id;
      chosen[others] = last;
      qsort(chosen, (size_t)(others + 1), sizeof(int32_t), int_asc);
      for (int s = 0; s <= others; ++s) cand_out[s] = chosen[s];
    }
  }
  free(eligible); free(score); free(list); free(chosen);
  return rc;
}

static void* worker(void* arg) {
  job* J = (job*)arg;
  const oracle_problem* P = J->P;
  for (;;) {
    int i = __sync_fetch_and_add(&J->next, 1);
    if (i >= J->ntok) break;
    int t = J->tokens ? J->tokens[i] : i;
    int rc = run_token(P, t, J->topk_out + (int64_t)i * P->topk,
                       J->cand_out ? J->cand_out + (int64_t)i * P->cand_blocks : NULL,
                       J->scores_out ? J->scores_out + (int64_t)i * J->score_cols : NULL,
                       J->score_cols);
    if (rc) J->error = rc;
  }
  return NULL;
}

/* Run the indexer for the listed tokens (all tokens when tokens == NULL),
 * writing row i of each output for the i-th listed token.
 *   topk_out   [ntok, topk]
 *   cand_out   [ntok, cand_blocks]     (mode 2; may be NULL otherwise)
 *   scores_out [ntok, score_cols] FP32 scores by position, NaN where the
 *              position is not eligible (may be NULL)
 * Returns 0, -1 on inconsistent metadata or page ids, -2 on allocation
 * failure, -3 on an unsupported problem. */
int oracle_run(const oracle_problem* P, const int32_t* tokens, int ntok, int32_t* topk_out,
               int32_t* cand_out, float* scores_out, int score_cols, int nthreads) {
  if (P->num_heads < 1 || P->num_heads > 256 || (P->ratio != 1 && P->ratio != 2) ||
      P->topk < 1 || P->page_rows < 1 || (P->mode < 1 || P->mode > 3))
    return -3;
  if (P->mode == 2 && (P->cand_blocks < 1 || !cand_out)) return -3;
  if (P->mode == 3 && !P->cand_in) return -3; /* a consumer needs its source */
  if (ntok <= 0) return 0;
  job J = {P, tokens, ntok, topk_out, cand_out, scores_out, score_cols, 0, 0};
  if (nthreads < 1) nthreads = 1;
  if (nthreads > ntok) nthreads = ntok;
  if (nthreads == 1) {
    worker(&J);
    return J.error;
  }
  pthread_t* th = (pthread_t*)malloc(sizeof(pthread_t) * (size_t)nthreads);
  if (!th) return -2;
  for (int i = 0; i < nthreads; ++i) pthread_create(&th[i], NULL, worker, &J);
  for (int i = 0; i < nthreads; ++i) pthread_join(th[i], NULL);
  free(th);
  return J.error;
}
