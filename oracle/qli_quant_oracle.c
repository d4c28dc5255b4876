/*
 * Oracle for the two steps around the indexer: query quantization (the
 * producer of the INT8 queries, per-head scales and FP16 head weights the
 * indexer consumes) and the index-K cache write (the producer of the paged
 * INT8 K rows and per-position FP16 scales it streams).
 *
 * TEST INFRASTRUCTURE ONLY, like qli_oracle.c: a plain CPU implementation
 * used to check the GPU library; no product code may call it.
 *
 * Source: "DeepSeek V4.1 QLI V2 与候选集成" (vllm-ascend developer guide),
 *   - "数据流": every Q head is quantized to INT8 together with an FP16
 *     scale that is representable (the scale the quantization divides by
 *     is the FP16 value itself); the head weights and the K scales are
 *     FP16; the index K lives in the paged layout (64-row pages at a
 *     131072-byte stride, 128-row pages at 147712 bytes), one FP16 scale
 *     per compressed position;
 *   - "当前 A3 契约": INT8 Q/K with a per-head Q scale and a per-token K
 *     scale (quantization mode 2); head dimension 128.
 *
 * Readings taken where the page gives no formula (listed with their
 * reasons in the design notes of the repository):
 *   - symmetric INT8 over one row of 128 values: amax = max |x_d| (exact in
 *     FP32 for BF16 or FP32 inputs); s = fp16(fp32(amax / 127)), every
 *     rounding RNE, saturated to the largest finite FP16 (65504);
 *   - q_d = clamp(rint(fp32(x_d / s)), -127, 127) with the FP32 quotient
 *     correctly rounded and rint ties-to-even; a row with s = 0 (all zeros,
 *     or amax below half the smallest FP16 subnormal times 127) gives
 *     q = 0 and scale 0;
 *   - head weights: one RNE conversion to FP16 (IEEE, overflow to inf);
 *   - K cache write: row i goes to flat slot s_i = page * page_rows + row
 *     of the pool, K bytes at page * k_page_stride + row * 128, scale at
 *     page * s_page_stride + row * 2; s_i < 0 means "no slot" and is
 *     skipped, as is a slot beyond the pool.
 */
#include <math.h>
#include <stdint.h>
#include <string.h>

uint16_t oracle_f16_round(double x); /* qli_oracle.c: binary16 RNE */
double oracle_f16_value(uint16_t h);

#define QDIM 128

static float load_value(const void* x, int dtype, int64_t i) {
  if (dtype == 1) { /* bfloat16: the upper half of an IEEE single */
    uint32_t u = (uint32_t)((const uint16_t*)x)[i] << 16;
    float f;
    memcpy(&f, &u, 4);
    return f;
  }
  return ((const float*)x)[i];
}

/* One row: scale bits and 128 INT8 values. */
static void quantize_row(const void* x, int dtype, int64_t row, int8_t* q, uint16_t* scale) {
  float amax = 0.0f;
  for (int d = 0; d < QDIM; ++d) {
    float a = fabsf(load_value(x, dtype, row * QDIM + d));
    if (a > amax) amax = a;
  }
  float s32 = amax / 127.0f;              /* one FP32 rounding */
  uint16_t sh = oracle_f16_round((double)s32); /* one FP16 rounding of that float */
  if ((sh & 0x7FFFu) == 0x7C00u) sh = 0x7BFFu; /* saturate */
  *scale = sh;
  float s = (float)oracle_f16_value(sh);
  for (int d = 0; d < QDIM; ++d) {
    int8_t v = 0;
    if (s != 0.0f) {
      float r = rintf(load_value(x, dtype, row * QDIM + d) / s); /* FP32 quotient, RNE to integer */
      if (r > 127.0f) r = 127.0f;
      if (r < -127.0f) r = -127.0f;
      v = (int8_t)r;
    }
    q[row * QDIM + d] = v;
  }
}

void oracle_quantize_rows(const void* x, int dtype, int64_t rows, int8_t* q, uint16_t* scale) {
  for (int64_t r = 0; r < rows; ++r) quantize_row(x, dtype, r, q, scale + r);
}

void oracle_round_weights(const void* w, int dtype, int64_t n, uint16_t* out) {
  for (int64_t i = 0; i < n; ++i) out[i] = oracle_f16_round((double)load_value(w, dtype, i));
}

/* Quantize rows of K and scatter them into a compact pool copy
 * kpages[num_pages][page_rows][128], spages[num_pages][page_rows]. */
void oracle_write_k(const void* x, int dtype, const int64_t* slot, int64_t rows, int page_rows,
                    int64_t num_pages, int8_t* kpages, uint16_t* spages) {
  int8_t q[QDIM];
  for (int64_t r = 0; r < rows; ++r) {
    int64_t s = slot[r];
    if (s < 0 || s >= num_pages * page_rows) continue;
    uint16_t sc;
    /* quantize this row alone (row index 0 of a one-row view) */
    const void* base = dtype == 1 ? (const void*)((const uint16_t*)x + r * QDIM)
                                  : (const void*)((const float*)x + r * QDIM);
    quantize_row(base, dtype, 0, q, &sc);
    memcpy(kpages + s * QDIM, q, QDIM);
    spages[s] = sc;
  }
}
