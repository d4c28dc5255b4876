// HIP kernels that produce the indexer's quantized inputs on CDNA4 (gfx950):
// query quantization (INT8 query heads with a representable FP16 scale per
// head, FP16 head weights) and the index-K cache write (INT8 K rows with one
// FP16 scale per compressed position, scattered into the paged cache).
//
// Source: DeepSeek V4.1 QLI developer guide, "数据流" (Q heads become INT8
// with an FP16 scale that the FP16 format can represent; the head weights
// and K scales are FP16; the index K is paged, 64-row pages at a
// 131072-byte stride or 128-row pages at 147712 bytes) and "当前 A3 契约"
// (per-head Q scale, per-position K scale, INT8 quantization mode 2).
//
// Per row of 128 values (one query head or one K position):
//   amax = max |x|;  s = fp16(fp32(amax / 127)), saturated to 65504;
//   q    = clamp(rint(fp32(x / s)), -127, 127), q = 0 when s == 0.
//
// Layout of the work: 16 lanes per row, 8 consecutive values per lane (one
// 16-byte load for bfloat16, two for FP32), the row maximum by four DPP
// steps inside the 16-lane row, one 8-byte store of INT8 codes per lane.
// HBM-bound: per row 256 (bf16) or 512 (fp32) bytes in, 130 bytes out.
//
// Exact rounding without a division per value: y = x * rcp(s) is within
// 2^-12 of fp32(x / s) for |y| < 512 (rcp is accurate to 1 ulp, the product
// to half an ulp, the quotient's own rounding to half an ulp: together
// below 2^-22 relative), so rint(y) is already rint(fp32(x / s)) unless y
// lies within 2^-10 of a half-integer; only those values (about one in 500
// for continuous data, every exact tie) take the correctly rounded division.
// Beyond |y| >= 256 both sides clamp to +-127 with the same sign.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "qli.h"
#include "qli_internal.h"

namespace qli {
namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int kQuantThreads = 256;
constexpr int kRowLanes = 16;                          // lanes per 128-value row
constexpr int kRowsPerWG = kQuantThreads / kRowLanes;  // 16
constexpr int kQuantPasses = 4;  // row passes per workgroup on large inputs (1 on small ones)

// Eight consecutive values of one row, as FP32 (bfloat16 widens exactly).
template <int DT>
__device__ __forceinline__ void load8(const void* base, int64_t row, int part, float (&v)[8]) {
  if constexpr (DT == QLI_DTYPE_BF16) {
    const u32x4* p =
        reinterpret_cast<const u32x4*>(static_cast<const uint16_t*>(base) + row * 128 + part * 8);
    const u32x4 u = __builtin_nontemporal_load(p);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      v[2 * i] = __uint_as_float(u[i] << 16);
      v[2 * i + 1] = __uint_as_float(u[i] & 0xFFFF0000u);
    }
  } else {
    const u32x4* p =
        reinterpret_cast<const u32x4*>(static_cast<const float*>(base) + row * 128 + part * 8);
    const u32x4 a = __builtin_nontemporal_load(p);
    const u32x4 b = __builtin_nontemporal_load(p + 1);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      v[i] = __uint_as_float(a[i]);
      v[4 + i] = __uint_as_float(b[i]);
    }
  }
}

// Maximum over the 16 lanes of a DPP row (all lanes of the row receive it).
// Steps: swap neighbours, swap pairs (quad permutations), mirror inside each
// half row (joins the two quads of a half), mirror the whole row.
__device__ __forceinline__ uint32_t row16_max(uint32_t v) {
  v = max(v, static_cast<uint32_t>(__builtin_amdgcn_mov_dpp(static_cast<int>(v), 0xB1, 0xF, 0xF, false)));
  v = max(v, static_cast<uint32_t>(__builtin_amdgcn_mov_dpp(static_cast<int>(v), 0x4E, 0xF, 0xF, false)));
  v = max(v, static_cast<uint32_t>(__builtin_amdgcn_mov_dpp(static_cast<int>(v), 0x141, 0xF, 0xF, false)));
  v = max(v, static_cast<uint32_t>(__builtin_amdgcn_mov_dpp(static_cast<int>(v), 0x140, 0xF, 0xF, false)));
  return v;
}

struct RowCodes {
  u32x2 q;         // 8 INT8 codes, value 0 in the low byte
  uint16_t scale;  // FP16 bits of the row scale
};

// Quantize this lane's 8 values of a row whose 16 lanes all call this.
__device__ __forceinline__ RowCodes quantize8(const float (&v)[8]) {
  uint32_t m = 0;
#pragma unroll
  for (int i = 0; i < 8; ++i) m = max(m, __float_as_uint(v[i]) & 0x7FFFFFFFu);
  // |x| bit patterns of finite values order like the values themselves
  const float amax = __uint_as_float(row16_max(m));
  const _Float16 sh = static_cast<_Float16>(amax / 127.0f);  // IEEE division, one RNE to FP16
  uint16_t sbits = __builtin_bit_cast(uint16_t, sh);
  if (sbits == 0x7C00u) sbits = 0x7BFFu;  // saturate (amax >= 0: never negative)
  const float s = static_cast<float>(__builtin_bit_cast(_Float16, sbits));
  const float r = __builtin_amdgcn_rcpf(s);
  float n[8];
  uint32_t near = 0;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const float y = v[i] * r;
    n[i] = __builtin_rintf(y);
    const float d = __builtin_fabsf(__builtin_fabsf(y - n[i]) - 0.5f);
    if (__builtin_fabsf(y) < 256.0f && d < 0x1p-10f) near |= 1u << i;
  }
  if (near) {
    // rare: settle the rounding with the correctly rounded quotient
#pragma unroll
    for (int i = 0; i < 8; ++i)
      if (near & (1u << i)) n[i] = __builtin_rintf(v[i] / s);
  }
  RowCodes out;
  uint32_t w[2] = {0u, 0u};
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const float c = __builtin_fminf(__builtin_fmaxf(n[i], -127.0f), 127.0f);
    const int32_t qi = s == 0.0f ? 0 : static_cast<int32_t>(c);
    w[i >> 2] |= (static_cast<uint32_t>(qi) & 0xFFu) << (8 * (i & 3));
  }
  out.q = u32x2{w[0], w[1]};
  out.scale = sbits;
  return out;
}

template <int DT>
__device__ __forceinline__ float load_weight(const void* w, int64_t i) {
  if constexpr (DT == QLI_DTYPE_BF16)
    return __uint_as_float(static_cast<uint32_t>(static_cast<const uint16_t*>(w)[i]) << 16);
  else
    return static_cast<const float*>(w)[i];
}

struct QuantArgs {
  const void* x;
  int8_t* q;
  uint16_t* qs;
  const void* w;
  uint16_t* wo;
  int64_t rows;
  int64_t nw;
};

// Block b quantizes rows [16*PASSES*b, 16*PASSES*(b+1)) in PASSES passes of
// 16 consecutive rows (the loads of every pass issued before the first is
// used) and rounds weights b*256 + tid, b*256 + tid + 256*grid, ...
template <int XDT, int WDT, int PASSES>
__global__ void __launch_bounds__(kQuantThreads) quantize_kernel(QuantArgs a) {
  constexpr int kQuantRowsPerWG = kRowsPerWG * PASSES;
  const int64_t b = blockIdx.x;
  const int tid = threadIdx.x;
  for (int64_t wi = b * kQuantThreads + tid; wi < a.nw; wi += static_cast<int64_t>(gridDim.x) * kQuantThreads)
    a.wo[wi] = __builtin_bit_cast(uint16_t, static_cast<_Float16>(load_weight<WDT>(a.w, wi)));
  const int64_t row0 = b * kQuantRowsPerWG + tid / kRowLanes;
  if (b * kQuantRowsPerWG >= a.rows) return;  // whole block past the rows (uniform)
  const int part = tid % kRowLanes;
  // a 16-lane group either has its row or not: the DPP row maximum needs
  // all 16 lanes of the row, and never mixes rows
  float v[PASSES][8];
#pragma unroll
  for (int i = 0; i < PASSES; ++i) {
    // rows past the end load the last row (in bounds, never stored)
    const int64_t row = row0 + i * kRowsPerWG;
    load8<XDT>(a.x, row < a.rows ? row : a.rows - 1, part, v[i]);
  }
#pragma unroll
  for (int i = 0; i < PASSES; ++i) {
    const int64_t row = row0 + i * kRowsPerWG;
    if (row >= a.rows) break;
    const RowCodes c = quantize8(v[i]);
    __builtin_nontemporal_store(c.q, reinterpret_cast<u32x2*>(a.q + row * 128 + part * 8));
    if (part == 0) a.qs[row] = c.scale;
  }
}

struct KWriteArgs {
  const void* x;
  const int64_t* slot;
  int8_t* k;
  uint8_t* ks;
  uint32_t* status;
  int64_t rows;
  int64_t kstride;
  int64_t sstride;
  int64_t pool;  // num_pages * page_rows
  int rlog;      // log2(page_rows)
};

template <int XDT>
__global__ void __launch_bounds__(kQuantThreads) write_k_kernel(KWriteArgs a) {
  const int tid = threadIdx.x;
  const int64_t row = static_cast<int64_t>(blockIdx.x) * kRowsPerWG + tid / kRowLanes;
  const int part = tid % kRowLanes;
  if (row >= a.rows) return;  // the 16 lanes of a row leave together
  const int64_t sl = a.slot[row];
  if (sl < 0) return;
  if (sl >= a.pool) {
    if (part == 0 && a.status) atomicOr(a.status, QLI_DEV_BAD_PAGE);
    return;
  }
  float v[8];
  load8<XDT>(a.x, row, part, v);
  const RowCodes c = quantize8(v);
  const int64_t page = sl >> a.rlog;
  const int64_t r = sl & ((int64_t(1) << a.rlog) - 1);
  int8_t* dst = a.k + page * a.kstride + r * 128 + part * 8;
  *reinterpret_cast<u32x2*>(dst) = c.q;
  if (part == 0) *reinterpret_cast<uint16_t*>(a.ks + page * a.sstride + r * 2) = c.scale;
}

template <int XDT, int PASSES>
void launch_quantize_xp(int wdt, hipStream_t st, const QuantArgs& a) {
  const int64_t gr = (a.rows + kRowsPerWG * PASSES - 1) / (kRowsPerWG * PASSES);
  const int64_t gw = (a.nw + kQuantThreads - 1) / kQuantThreads;
  const unsigned grid = static_cast<unsigned>(gr > gw ? gr : gw);
  if (wdt == QLI_DTYPE_BF16)
    quantize_kernel<XDT, QLI_DTYPE_BF16, PASSES><<<grid, kQuantThreads, 0, st>>>(a);
  else
    quantize_kernel<XDT, QLI_DTYPE_F32, PASSES><<<grid, kQuantThreads, 0, st>>>(a);
}

// Four passes per workgroup once that still leaves two workgroups per CU;
// smaller inputs spread one pass per workgroup over more CUs.
template <int XDT>
void launch_quantize_x(int wdt, hipStream_t st, const QuantArgs& a) {
  if (a.rows >= static_cast<int64_t>(kRowsPerWG) * kQuantPasses * 2 * cu_count())
    launch_quantize_xp<XDT, kQuantPasses>(wdt, st, a);
  else
    launch_quantize_xp<XDT, 1>(wdt, st, a);
}

}  // namespace

int launch_quantize(const qli_quant_params* p, void* stream) {
  hipStream_t st = static_cast<hipStream_t>(stream);
  (void)hipGetLastError();
  QuantArgs a;
  a.x = p->x;
  a.q = p->q;
  a.qs = static_cast<uint16_t*>(p->q_scale);
  a.w = p->w;
  a.wo = static_cast<uint16_t*>(p->w_out);
  a.rows = p->num_rows;
  a.nw = p->num_weights;
  {
    Stamp s(QLI_KERNEL_QUANTIZE, st);
    if (p->x_dtype == QLI_DTYPE_BF16) launch_quantize_x<QLI_DTYPE_BF16>(p->w_dtype, st, a);
    else launch_quantize_x<QLI_DTYPE_F32>(p->w_dtype, st, a);
  }
  return hipGetLastError() == hipSuccess ? QLI_OK : QLI_ERR_HIP;
}

int launch_write_k(const qli_kwrite_params* p, void* stream) {
  hipStream_t st = static_cast<hipStream_t>(stream);
  (void)hipGetLastError();
  KWriteArgs a;
  a.x = p->x;
  a.slot = p->slot;
  a.k = p->k_cache;
  a.ks = static_cast<uint8_t*>(p->k_scale);
  a.status = p->status_out;
  a.rows = p->num_rows;
  a.kstride = p->k_page_stride;
  a.sstride = p->s_page_stride;
  a.pool = p->num_pages * p->page_rows;
  a.rlog = p->page_rows == 128 ? 7 : 6;
  const unsigned grid = static_cast<unsigned>((a.rows + kRowsPerWG - 1) / kRowsPerWG);
  {
    Stamp s(QLI_KERNEL_WRITE_K, st);
    if (p->x_dtype == QLI_DTYPE_BF16) write_k_kernel<QLI_DTYPE_BF16><<<grid, kQuantThreads, 0, st>>>(a);
    else write_k_kernel<QLI_DTYPE_F32><<<grid, kQuantThreads, 0, st>>>(a);
  }
  return hipGetLastError() == hipSuccess ? QLI_OK : QLI_ERR_HIP;
}

}  // namespace qli
