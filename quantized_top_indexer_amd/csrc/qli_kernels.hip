// HIP kernels of the quantized lightning indexer for CDNA4 (gfx950).
//
// One call = three launches in the usual case (DeepSeek V4.1 QLI developer
// guide, "数据流" and "当前 A3 契约"):
//   plan           one workgroup (one wave for decode-sized batches): cut the
//                  batch into groups (up to 4 consecutive query tokens of one
//                  request in plain/source mode, one token in consumer mode)
//                  and prefix-sum their 256-slot work units, so that a
//                  persistent kernel can split any mix of decode tokens and
//                  prefill chunks evenly.  In consumer mode it is block 0 of
//                  the preparation launch (batches of 1024 tokens and more:
//                  a launch of its own before it).
//   consumer_prep  (consumer mode) one workgroup per token: de-duplicate the
//                  incoming candidate block ids, drop ids without a visible
//                  position, resolve each kept block to its page row -> dense
//                  slot list + eligible count.
//   score          persistent, two workgroups per CU.  Each workgroup walks a
//                  contiguous range of work items (group, 256-slot chunk) with
//                  a software pipeline: page lookups and K + scale loads
//                  ahead of use (registers; one to two items), and for the
//                  current item an LDS tile (shared by a group's 4 tokens,
//                  or each wave's own rows for single tokens), INT8 MFMA
//                  (v_mfma_i32_32x32x32_i8, queries x keys), the golden
//                  FP16/FP32 epilogue, block maxima and order keys.
//   select         one workgroup per (token, positions|blocks): keys held in
//                  registers, range-adaptive radix select (2048-bin digits),
//                  then an ordered compaction that emits the winners already
//                  in ascending order, -1 tail.  The workgroup size follows
//                  the row length; batches of many rows of mixed lengths run
//                  one launch per length class.
//
// Exactness: the epilogue applies one IEEE round-to-nearest-even per golden
// step and sums heads in ascending order from +0.0f in a single lane, so the
// scores and every selection are bit-identical to a sequential reference.
// Built with -ffp-contract=off; the two mixed-precision steps that must not
// be re-associated are written as explicit v_fma_mix instructions.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <algorithm>
#include <atomic>
#include <mutex>
#include <type_traits>
#include <vector>

#include "qli.h"
#include "qli_internal.h"

namespace qli {
namespace {

typedef int32_t i32x4 __attribute__((ext_vector_type(4)));
typedef int32_t i32x16 __attribute__((ext_vector_type(16)));
typedef _Float16 h2 __attribute__((ext_vector_type(2)));
typedef int16_t s2 __attribute__((ext_vector_type(2)));

// Work list: list 0 holds multi groups (4 consecutive query tokens of one
// request sharing every K tile: the leading full quadruples of each request
// in plain/source mode), list 1 single-token groups (every other token).
struct PlanHdr {
  int32_t ngroups[2];
  int32_t units[2];
  int32_t pad[60];
};

// A group: ntok consecutive query tokens t0.. of request b sharing K tiles.
//   p0    raw position of t0
//   L     compressed length of the request (0 when its metadata is invalid)
//   n0    eligible slots of t0 (dense: its visible count; consumer: ncount)
//   nlast eligible slots of the group's last token (>= every member's)
//   nch   256-slot work items: ceil(nlast / 256)
struct Group {
  int32_t t0, ntok, b, nch, p0, L, n0, nlast;
};

// Where score workgroup w starts (written by the plan kernel, read with one
// load so that the first K loads follow after a single dependent lookup):
// its list, that list's group count, the group g holding its first item,
// the item index c in g and its first work unit, and the end hi of its unit
// range.  g < 0: the workgroup has no work.
struct WgStart {
  Group grp;
  int32_t list, ng, g, c, unit, hi, pad[2];
};
static_assert(sizeof(WgStart) == kWgStartBytes, "WgStart size");

struct KArgs {
  float one;  // 1.0f
  int mode, ratio, rshift, B, T, topk, cb, cb_in, R, rlog, bt_stride, num_pages, max_k_len;
  // A call runs in slices of consecutive query tokens: T tokens from global
  // token t_base.  Workspace arrays are indexed by the local token (0..T);
  // the per-token inputs and outputs below point at the slice's first
  // token; the request metadata (qsl) keeps global token indices.
  int t_base;
  int score_grid;      // workgroups of the score kernel that walks the single list (all lists
                       // when multi_grid == 0)
  int multi_grid;      // > 0: the multi list runs in a kernel of its own with this many
                       // workgroups, whose start entries come first
  int entry_base;      // first start entry of the launched score kernel
  int nxcd;            // XCDs of the device (accelerator dies, each with its own L2)
  int sel_lo, sel_hi;  // this select launch takes the rows whose length n has sel_lo <= n <= sel_hi
  int64_t kstride, sstride, ncap, nbcap;
  const int8_t* q;
  const uint16_t* qs;
  const uint16_t* w;
  const int8_t* k;
  const uint8_t* ks;
  const int32_t* bt;
  const int32_t* qsl;
  const int32_t* klen;
  const int32_t* smod;
  const int32_t* cand_in;
  int32_t* topk_out;
  int32_t* cand_out;
  float* dbg;
  int32_t* dbg_qk;  // [T, NH, max_k_len] exact q.k (debug only)
  uint32_t* status;
  uint32_t* keys;
  uint32_t* bkeys;
  PlanHdr* hdr;
  Group* groups;    // [2][T]
  int32_t* ustart;  // [2][T + 1]
  WgStart* wgs;     // [score_grid]
  int32_t* slots;
  int32_t* srow;
  int32_t* ncount;
  // [T][2] per token: [0] visible compressed count (plan); [1] == epoch: a
  // block the token may read had an out-of-contract page (score)
  int32_t* tokv;
  uint32_t epoch;   // this launch's stamp (another value in tokv[t][1] is stale)
  int fused;        // the score kernel plans for itself (no plan launch; small batches)
  int plan_wg;      // >= 0: the plan keeps only this workgroup's start entry, in wgs[0]
};

__device__ __forceinline__ void raise_flag(const KArgs& a, uint32_t bit) {
  if (a.status) atomicOr(a.status, bit);
}

// Request metadata, read from global memory or from an LDS copy.
struct Meta {
  const int32_t* qsl;
  const int32_t* klen;
  const int32_t* smod;  // null at ratio 1
};

__device__ __forceinline__ Meta global_meta(const KArgs& a) { return Meta{a.qsl, a.klen, a.smod}; }

// request of token t: the last b with qsl[b] <= t
__device__ __forceinline__ int request_of(const Meta& m, int B, int t) {
  int lo = 0, hi = B - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (m.qsl[mid] <= t) lo = mid;
    else hi = mid - 1;
  }
  return lo;
}

// Per-request causal view (causal mask mode 3): the request's n_b queries
// are its last raw positions, the raw length is L*r + residual, and the
// query at raw position p sees compressed entries j < floor((p+1)/r).
// Out-of-contract metadata gives L = 0 (nothing visible) and a flag.
struct ReqView {
  int q0, q1, L;
  int64_t S;
};

__device__ __forceinline__ ReqView request_view(const KArgs& a, const Meta& m, int b, bool report) {
  ReqView v;
  v.q0 = m.qsl[b];
  v.q1 = m.qsl[b + 1];
  int L = m.klen[b];
  const int s = m.smod ? m.smod[b] : 0;
  if (L < 0 || L > a.max_k_len) {
    if (report) raise_flag(a, QLI_DEV_BAD_LENGTH);
    L = 0;
  } else if (s < 0 || s >= a.ratio) {
    if (report) raise_flag(a, QLI_DEV_BAD_METADATA);
    L = 0;
  } else if (static_cast<int64_t>(v.q1) - v.q0 > static_cast<int64_t>(L) * a.ratio + s) {
    if (report) raise_flag(a, QLI_DEV_BAD_METADATA);
    L = 0;
  }
  v.L = L;
  v.S = L == 0 ? static_cast<int64_t>(v.q1) - v.q0 : static_cast<int64_t>(L) * a.ratio + s;
  return v;
}

// visible count of the query at raw position p
__device__ __forceinline__ int visible(const KArgs& a, int64_t p, int L) {
  const int64_t V = (p + 1) >> a.rshift;
  return static_cast<int>(V < L ? V : L);
}

__device__ __forceinline__ int page_checked(const KArgs& a, int b, int idx) {
  if (idx >= a.bt_stride) return -1;
  const int page = a.bt[static_cast<int64_t>(b) * a.bt_stride + idx];
  return (page >= 0 && page < a.num_pages) ? page : -1;
}

// Order-preserving map of an FP32 score to u32 (-0 ranks as +0).  Finite
// scores map into [0x00800000, 0xFF7FFFFF], so 0 is free to mean "not
// eligible" and 0xFFFFFFFF to mean "pinned".
__device__ __forceinline__ uint32_t order_key(float f) {
  uint32_t u = __float_as_uint(f);
  if (u == 0x80000000u) u = 0u;
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

__device__ __forceinline__ h2 as_h2(uint32_t v) { return __builtin_bit_cast(h2, v); }
__device__ __forceinline__ uint32_t as_u32(h2 v) { return __builtin_bit_cast(uint32_t, v); }

// ReLU of two fp16 values given as bits: an fp16 is negative (or -0) exactly
// when its bit pattern is a negative int16, so max(bits, 0) as int16 gives
// x for x > 0 and +0 otherwise (no NaN can occur here).  Written as one
// instruction in assembly: as a generic int16 max the compiler would pack
// the two converted halves with an extra permute instead of converting the
// second straight into the high half.  Its input is a VALU result, never an
// MFMA result, so no MFMA wait states are involved.
__device__ __forceinline__ uint32_t relu_h2(uint32_t v) {
  uint32_t r;
  asm("v_pk_max_i16 %0, %1, 0" : "=v"(r) : "v"(v));
  return r;
}

// The MFMA accumulator is seeded with the bits of 4.0f (an inline constant
// of the instruction, so the seed costs no registers), and the integer sum
// of the seed and qk is then a float F that carries qk:
//  - qk >= 0: F = 4 + qk * 2^-21 exactly (ulp of [4, 8) is 2^-21, and
//    qk < 2^21 for any int8 operands: |q.k| <= 128 * 127 * 128);
//  - qk < 0: the bits fall below those of 4.0, so F lies in [2, 4).
// Only max(qk, 0) matters after the ReLU, and every negative qk gives F < 4.
// fp16(qk/1024) for qk >= 0 is fp16(2048 * F - 8192) (the fma is exact and
// the conversion rounds once, RNE); for qk < 0 that value is negative and
// the ReLU makes it +0, the golden result.  Two forms, same bits:
//  - qk_to_half: one fma written so that it becomes one v_fma_mixlo/hi_f16
//    (fewest instructions and registers);
//  - qk_over_1024 + a packed conversion of two values: an FP32 fma per
//    value and one v_cvt_pk_f16_f32 per pair, faster where the VALU is the
//    bound (the mixed-precision conversions issue at half rate).  The empty
//    assembly statement keeps the compiler from fusing the two back into
//    the mixed form; it emits no instruction.
// No inline assembly touches MFMA results, so the compiler inserts the
// MFMA-to-VALU wait states.
constexpr int32_t kSeedBits = 0x40800000;  // 4.0f
__device__ __forceinline__ _Float16 qk_to_half(int32_t acc) {
  return static_cast<_Float16>(__builtin_fmaf(__int_as_float(acc), 2048.0f, -8192.0f));
}
__device__ __forceinline__ float qk_over_1024(int32_t acc) {
  float y = __builtin_fmaf(__int_as_float(acc), 2048.0f, -8192.0f);
  asm volatile("" : "+v"(y));
  return y;
}

// Scaled form of the same step with the ReLU folded in: y = F - 4 is
// qk * 2^-21 exactly for qk >= 0 and negative otherwise, so clamping it to
// [0, 1] (the add's clamp bit, 4.0 an inline constant) gives
// max(qk, 0) * 2^-21 in one instruction; fp16(y) = fp16(qk/1024) * 2^-11
// exactly (for qk < 128, y is an fp16 subnormal on the 2^-21 grid; above,
// scaling by a power of two commutes with rounding), so
// fp16(fp16(y) * m * 2^11) equals the golden fp16(relu(fp16(qk/1024)) * m)
// whenever m * 2^11 is still a finite fp16 (|m| < 32).
__device__ __forceinline__ float qk_relu_scaled(int32_t acc) {
  float y = __builtin_amdgcn_fmed3f(__int_as_float(acc) - 4.0f, 0.0f, 1.0f);
  asm volatile("" : "+v"(y));
  return y;
}
constexpr uint32_t kHalfAbs32 = 0x5000u;  // fp16 bits of 32.0

// s + float(h) with one FP32 rounding: fma(h, one, s) with one == 1.0 held
// in a kernel argument (opaque to constant folding) selects v_fma_mix_f32.
__device__ __forceinline__ float add_h(float s, _Float16 h, float one) {
  return __builtin_fmaf(static_cast<float>(h), one, s);
}

// Cross-lane steps on DPP (no LDS traffic).  dpp_or0: lanes without a
// source (shifted out of their row, or rows outside row_mask) read 0.
template <int CTRL, int ROW_MASK>
__device__ __forceinline__ uint32_t dpp_or0(uint32_t v) {
  return static_cast<uint32_t>(
      __builtin_amdgcn_update_dpp(0, static_cast<int>(v), CTRL, ROW_MASK, 0xF, false));
}
template <int CTRL>
__device__ __forceinline__ uint32_t dpp_all(uint32_t v) {
  return static_cast<uint32_t>(
      __builtin_amdgcn_update_dpp(static_cast<int>(v), static_cast<int>(v), CTRL, 0xF, 0xF, false));
}

// Inclusive prefix sum over the 64 lanes: shifts by 1, 2, 4, 8 within each
// row of 16, then the row totals through the row-15 and row-31 broadcasts.
__device__ __forceinline__ uint32_t wave_inclusive_scan(uint32_t v) {
  v += dpp_or0<0x111, 0xF>(v);  // row_shr:1
  v += dpp_or0<0x112, 0xF>(v);  // row_shr:2
  v += dpp_or0<0x114, 0xF>(v);  // row_shr:4
  v += dpp_or0<0x118, 0xF>(v);  // row_shr:8
  v += dpp_or0<0x142, 0xA>(v);  // row_bcast:15 into rows 1 and 3
  v += dpp_or0<0x143, 0xC>(v);  // row_bcast:31 into rows 2 and 3
  return v;
}

// Running maximum over the lanes of a wave (values >= 0), in the steps of
// the prefix sum above.
__device__ __forceinline__ uint32_t wave_inclusive_max(uint32_t v) {
  v = max(v, dpp_or0<0x111, 0xF>(v));
  v = max(v, dpp_or0<0x112, 0xF>(v));
  v = max(v, dpp_or0<0x114, 0xF>(v));
  v = max(v, dpp_or0<0x118, 0xF>(v));
  v = max(v, dpp_or0<0x142, 0xA>(v));
  v = max(v, dpp_or0<0x143, 0xC>(v));
  return v;
}

// op over the 64 lanes (result in every lane): butterflies within each row,
// then the four row values.
template <class Op>
__device__ __forceinline__ uint32_t wave_allreduce(uint32_t v, Op op) {
  v = op(v, dpp_all<0xB1>(v));   // quad_perm [1,0,3,2]
  v = op(v, dpp_all<0x4E>(v));   // quad_perm [2,3,0,1]
  v = op(v, dpp_all<0x124>(v));  // row_ror:4
  v = op(v, dpp_all<0x128>(v));  // row_ror:8
  const uint32_t r0 = static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(v), 0));
  const uint32_t r1 = static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(v), 16));
  const uint32_t r2 = static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(v), 32));
  const uint32_t r3 = static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(v), 48));
  return op(op(r0, r1), op(r2, r3));
}

template <int BS>
__device__ uint32_t block_exclusive_scan(uint32_t v, uint32_t* total, uint32_t* sh) {
  constexpr int NW = BS / 64;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const uint32_t inc = wave_inclusive_scan(v);
  if (lane == 63) sh[wave] = inc;
  __syncthreads();
  if (wave == 0) {
    const uint32_t x = lane < NW ? sh[lane] : 0u;
    const uint32_t xi = wave_inclusive_scan(x);
    if (lane < NW) sh[16 + lane] = xi - x;
    if (lane == NW - 1) sh[32] = xi;
  }
  __syncthreads();
  const uint32_t out = sh[16 + wave] + inc - v;
  *total = sh[32];
  __syncthreads();
  return out;
}

// ---------------------------------------------------------------------------
// consumer_prep: sorted unique visible incoming block ids per token
// ---------------------------------------------------------------------------
constexpr int kPrepThreads = 1024;      // preparation with the plan in block 0 (sorting: two ids per thread)
constexpr int kPrepBitmapThreads = 256; // lean bitmap preparation (up to 8 ids and 32 bitmap words per thread)
constexpr int kPrepBitmapWords = 8192;  // bitmap of up to 2^18 block ids (32 KB of LDS)
constexpr int kPrepLeanMinTokens = 1024;  // consumer batches this large plan in a launch of their own

// The request holding global token tg, found by all threads at once (one
// round of loads instead of a dependent binary search); every thread gets it.
template <int PT>
__device__ __forceinline__ int prep_request(const KArgs& a, int tg, int* s_req) {
  const int i0 = threadIdx.x;  // the first round's loads go out before the barrier
  int q0 = 0, q1 = 0;
  if (i0 < a.B) {
    q0 = a.qsl[i0];
    q1 = a.qsl[i0 + 1];
  }
  if (threadIdx.x == 0) *s_req = 0;
  __syncthreads();
  if (i0 < a.B && q0 <= tg && tg < q1) *s_req = i0;
  for (int i = i0 + PT; i < a.B; i += PT)
    if (a.qsl[i] <= tg && tg < a.qsl[i + 1]) *s_req = i;
  __syncthreads();
  return *s_req;
}

// Slot table of token t from its kept block ids in ascending order (sl[0 ..
// total), in LDS): slots, page rows and the eligible count.
template <int PT>
__device__ __forceinline__ void prep_write(const KArgs& a, int t, int b, int V, const int32_t* sl,
                                           int total) {
  int32_t* slots = a.slots + static_cast<int64_t>(t) * a.cb_in;
  int32_t* srow = a.srow + static_cast<int64_t>(t) * a.cb_in;
  bool bad = false;
  for (int i = threadIdx.x; i < total; i += PT) {
    const int blk = sl[i];
    const int pos0 = blk * 8;
    const int page = page_checked(a, b, pos0 >> a.rlog);
    bad |= page < 0;
    slots[i] = blk;
    srow[i] = page < 0 ? -1 : page * a.R + (pos0 & (a.R - 1));
  }
  if (bad) raise_flag(a, QLI_DEV_BAD_PAGE);
  if (threadIdx.x == 0) {
    // every kept block is full except possibly the last visible one, which
    // is the largest id and therefore the last slot
    const int tail = total > 0 ? V - sl[total - 1] * 8 : 0;
    a.ncount[t] = total > 0 ? 8 * (total - 1) + min(tail, 8) : 0;
  }
}

// In consumer mode one launch prepares the tokens and plans the score work:
// block 0 runs the plan (it needs no prepared data: a consumer token's work
// is bounded by min(cb_in, visible blocks) * 8 slots, and the score kernel
// reads the exact eligible count), blocks 1..T prepare token blockIdx.x - 1.
// Both roles carve their LDS from one buffer.
constexpr int kPlanLdsRequests = 4096;  // metadata of up to this many requests is staged in LDS
template <int PT, int NREQ = kPlanLdsRequests>
__device__ void plan_role(const KArgs& a, uint32_t* lds);
// request metadata, scan scratch, one mark per score workgroup
constexpr int kPlanLdsWords = 3 * kPlanLdsRequests + 1 + 64 + kMaxScoreWGs;
constexpr int kPrepLdsWords = kPrepBitmapWords + QLI_MAX_CAND_BLOCKS + 64 + 1;
constexpr int kConsumerLdsWords = kPrepLdsWords > kPlanLdsWords ? kPrepLdsWords : kPlanLdsWords;

// Sorted unique visible incoming block ids per token, through a bitmap of
// the visible block ids: duplicates merge, and a prefix count of set bits
// places every id (contexts of up to 2^18 blocks).
// Preparation of token t through the bitmap: bm (one bit per visible
// block), sl (the kept ids, at most cb_in), sh (64 words of scan scratch)
// and s_req (one word) are LDS.
template <int PT>
__device__ __forceinline__ void prep_bitmap_token(const KArgs& a, int t, uint32_t* bm, int32_t* sl,
                                                  uint32_t* sh, int* s_req) {
  const int tid = threadIdx.x;
  const int tg = t + a.t_base;
  // the incoming ids are loaded first, in flight with the request lookup
  constexpr int CPT = QLI_MAX_CAND_BLOCKS / PT;
  const int32_t* cin = a.cand_in + static_cast<int64_t>(t) * a.cb_in;
  int cv[CPT];
#pragma unroll
  for (int j = 0; j < CPT; ++j) cv[j] = tid + j * PT < a.cb_in ? cin[tid + j * PT] : -1;
  const int b = prep_request<PT>(a, tg, s_req);
  const ReqView r = request_view(a, global_meta(a), b, tid == 0);
  const int V = (tg >= r.q0 && tg < r.q1)
                    ? visible(a, r.S - (r.q1 - r.q0) + (tg - r.q0), r.L) : 0;
  const int nblocks = (V + 7) / 8;
  const int nwords = (nblocks + 31) / 32;  // within the bitmap: V <= max_k_len (checked at launch)
  for (int i = tid; i < nwords; i += PT) bm[i] = 0;
  __syncthreads();
#pragma unroll
  for (int j = 0; j < CPT; ++j) {
    const int c = cv[j];
    if (c >= 0 && c < nblocks) atomicOr(&bm[c >> 5], 1u << (c & 31));
  }
  __syncthreads();
  const int wpt = (nwords + PT - 1) / PT;
  const int w0 = min(nwords, tid * wpt), w1 = min(nwords, w0 + wpt);
  uint32_t cnt = 0;
  for (int w = w0; w < w1; ++w) cnt += __popc(bm[w]);
  uint32_t total;
  uint32_t at = block_exclusive_scan<PT>(cnt, &total, sh);
  for (int w = w0; w < w1; ++w) {
    uint32_t bits = bm[w];
    while (bits) {
      const int j = __ffs(bits) - 1;
      bits &= bits - 1;
      sl[at++] = 32 * w + j;
    }
  }
  __syncthreads();
  prep_write<PT>(a, t, b, V, sl, static_cast<int>(total));
}

__global__ __launch_bounds__(kPrepThreads) void consumer_prep_kernel(KArgs a) {
  constexpr int PT = kPrepThreads;
  __shared__ uint32_t lds[kConsumerLdsWords];
  if (blockIdx.x == 0) {
    plan_role<PT>(a, lds);
    return;
  }
  uint32_t* sh = lds + kPrepBitmapWords + QLI_MAX_CAND_BLOCKS;
  prep_bitmap_token<PT>(a, blockIdx.x - 1, lds, reinterpret_cast<int32_t*>(lds + kPrepBitmapWords), sh,
                        reinterpret_cast<int*>(sh + 64));
}

// Large batches: the plan runs as a launch of its own and every workgroup
// prepares one token in LDS sized for this call (nwcap bitmap words for the
// longest context, cb_in kept ids), so that several workgroups share a CU
// (the plan's metadata staging would otherwise size every workgroup's LDS).
__global__ __launch_bounds__(kPrepBitmapThreads) void consumer_prep_lean_kernel(KArgs a, int nwcap) {
  extern __shared__ uint32_t dlds[];
  uint32_t* sh = dlds + nwcap + a.cb_in;
  prep_bitmap_token<kPrepBitmapThreads>(a, blockIdx.x, dlds, reinterpret_cast<int32_t*>(dlds + nwcap), sh,
                                        reinterpret_cast<int*>(sh + 64));
}

// The same by a bitonic sort of the incoming ids (any context length).
__global__ __launch_bounds__(kPrepThreads) void consumer_prep_sort_kernel(KArgs a) {
  __shared__ uint32_t lds[kConsumerLdsWords];
  if (blockIdx.x == 0) {
    plan_role<kPrepThreads>(a, lds);
    return;
  }
  int32_t* v = reinterpret_cast<int32_t*>(lds);
  int32_t* sl = v + QLI_MAX_CAND_BLOCKS;
  uint32_t* sh = lds + 2 * QLI_MAX_CAND_BLOCKS;
  int* s_req = reinterpret_cast<int*>(sh + 64);
  const int t = blockIdx.x - 1;
  const int tg = t + a.t_base;
  const int tid = threadIdx.x;
  const int b = prep_request<kPrepThreads>(a, tg, s_req);
  const ReqView r = request_view(a, global_meta(a), b, tid == 0);
  const int V = (tg >= r.q0 && tg < r.q1)
                    ? visible(a, r.S - (r.q1 - r.q0) + (tg - r.q0), r.L) : 0;
  const int nblocks = (V + 7) / 8;
  const int cbi = a.cb_in;
  int n2 = 64;
  while (n2 < cbi) n2 <<= 1;
  const int32_t* cin = a.cand_in + static_cast<int64_t>(t) * cbi;
  for (int i = tid; i < n2; i += kPrepThreads) {
    int c = i < cbi ? cin[i] : INT32_MAX;
    if (c < 0 || c >= nblocks) c = INT32_MAX;
    v[i] = c;
  }
  __syncthreads();
  for (int size = 2; size <= n2; size <<= 1) {  // bitonic sort, ascending
    for (int stride = size >> 1; stride > 0; stride >>= 1) {
      for (int i = tid; i < n2 / 2; i += kPrepThreads) {
        const int lo = 2 * i - (i & (stride - 1));
        const int hi = lo + stride;
        const bool up = (lo & size) == 0;
        const int x = v[lo], y = v[hi];
        if ((x > y) == up) {
          v[lo] = y;
          v[hi] = x;
        }
      }
      __syncthreads();
    }
  }
  const int i0 = 2 * tid;
  bool f[2];
  uint32_t cnt = 0;
#pragma unroll
  for (int e = 0; e < 2; ++e) {
    const int i = i0 + e;
    f[e] = i < n2 && v[i] != INT32_MAX && (i == 0 || v[i] != v[i - 1]);
    cnt += f[e] ? 1u : 0u;
  }
  uint32_t total;
  uint32_t at = block_exclusive_scan<kPrepThreads>(cnt, &total, sh);
#pragma unroll
  for (int e = 0; e < 2; ++e)
    if (f[e]) sl[at++] = v[i0 + e];
  __syncthreads();
  prep_write<kPrepThreads>(a, t, b, V, sl, static_cast<int>(total));
}

// ---------------------------------------------------------------------------
// plan: groups and their work-unit prefix
// ---------------------------------------------------------------------------
constexpr int kPlanThreads = 1024;

// 0: global token tg belongs to a multi group it does not start; 1: starts
// a multi group; 2: forms a single group.  A quadruple that the slice
// [t_base, t_base + T) cuts is scored as single tokens (same results).
__device__ __forceinline__ int group_kind(const KArgs& a, const ReqView& r, int tg) {
  if (a.mode == QLI_MODE_CONSUMER) return 2;
  const int i = tg - r.q0;
  const int full = (r.q1 - r.q0) / kGroupTokens * kGroupTokens;
  if (i < full) {
    const int g0 = tg - i % kGroupTokens;  // the quadruple's first token
    if (g0 >= a.t_base && g0 + kGroupTokens <= a.t_base + a.T) return tg == g0 ? 1 : 0;
  }
  return 2;
}

// Group of ntok tokens starting at local token t (global tg).
__device__ __forceinline__ Group make_group(const KArgs& a, int b, const ReqView& r, int t, int tg,
                                            int ntok) {
  Group g;
  g.t0 = t;
  g.ntok = ntok;
  g.b = b;
  g.L = r.L;
  const int64_t p0 = r.S - (r.q1 - r.q0) + (tg - r.q0);
  g.p0 = static_cast<int>(p0);
  if (a.mode == QLI_MODE_CONSUMER) {
    // a bound on the eligible slots (the prepared count may not exist yet):
    // every kept block is an incoming id below ceil(V / 8)
    const int64_t nb = (static_cast<int64_t>(visible(a, p0, r.L)) + 7) / 8;
    g.n0 = static_cast<int>(8 * min(nb, static_cast<int64_t>(a.cb_in)));
    g.nlast = g.n0;
  } else {
    g.n0 = visible(a, p0, r.L);
    g.nlast = visible(a, p0 + ntok - 1, r.L);
  }
  g.nch = (g.nlast + kChunk - 1) / kChunk;
  return g;
}

// floor(p / q) for 0 <= p < 2^53 and 0 < q < 2^31: the correctly rounded
// double quotient is within one of the floor, and one integer check fixes it
// (a 64-bit integer divide would be a long software sequence); operands
// below 2^32 take one unsigned 32-bit division.
__device__ __forceinline__ int64_t floor_div(int64_t p, int64_t q) {
  if (((p | q) >> 32) == 0)  // both below 2^32: one unsigned 32-bit division
    return static_cast<uint32_t>(p) / static_cast<uint32_t>(q);
  int64_t f = static_cast<int64_t>(static_cast<double>(p) / static_cast<double>(q));
  if (f * q > p) --f;
  else if ((f + 1) * q <= p) ++f;
  return f;
}

__device__ __forceinline__ int64_t ceil_div(int64_t x, int64_t y) {
  return x <= 0 ? 0 : floor_div(x + y - 1, y);
}

// Score workgroups of the multi list: a share of the grid in proportion to
// its work units (at least one for each non-empty list).
__device__ __forceinline__ int multi_workgroups(int W, int Um, int Us) {
  if (Um <= 0) return 0;
  if (Us <= 0) return W;
  const int share = static_cast<int>(floor_div(static_cast<int64_t>(W) * Um,
                                               static_cast<int64_t>(Um) + Us));
  return min(W - 1, max(1, share));
}

// Exclusive prefix of N values at once over a workgroup of BS threads
// (BS/64 <= 16 waves); total[i] receives the sums.  Uses sh[0 .. 16 N).
template <int BS, int N>
__device__ __forceinline__ void block_exclusive_scan_n(uint32_t (&v)[N], uint32_t (&total)[N],
                                                       uint32_t* sh) {
  constexpr int NW = BS / 64;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  uint32_t inc[N];
#pragma unroll
  for (int i = 0; i < N; ++i) inc[i] = wave_inclusive_scan(v[i]);
  if (lane == 63) {
#pragma unroll
    for (int i = 0; i < N; ++i) sh[16 * i + wave] = inc[i];
  }
  __syncthreads();
#pragma unroll
  for (int i = 0; i < N; ++i) {
    uint32_t before = 0, t = 0;
#pragma unroll
    for (int w = 0; w < NW; ++w) {
      const uint32_t x = sh[16 * i + w];
      before += w < wave ? x : 0u;
      t += x;
    }
    v[i] = before + inc[i] - v[i];
    total[i] = t;
  }
  __syncthreads();
}

// One list's split of the score grid: nw workgroups over U work units;
// workgroup w owns the items whose first unit lies in
// [floor(w*U/nw), floor((w+1)*U/nw)).
struct Split {
  int list, ng, NT, nw, U, base;
};

// First item of a workgroup whose range starts at unit lo, in group gidx
// (first unit unit0): the first of the group's items (starts unit0 + c*NT)
// at or past lo.
__device__ __forceinline__ WgStart start_entry_of(const Split& sp, int gidx, const Group& g, int unit0, int lo,
                                                  int hi) {
  const int off = lo - unit0;
  const int c = off <= 0 ? 0 : (sp.NT == 1 ? off : (off + 3) >> 2);  // NT is 1 or 4
  WgStart st;
  st.grp = g;
  st.list = sp.list;
  st.ng = sp.ng;
  st.g = gidx;
  st.c = c;
  st.unit = unit0 + c * sp.NT;
  st.hi = hi;
  st.pad[0] = st.pad[1] = 0;
  return st;
}

// Every group of a list has the same token count NT, so group g (units
// [a, a + nch*NT)) holds the first item of exactly the workgroups whose
// range starts in (a - NT, a + (nch - 1)*NT].  A workgroup that plans for
// itself (plan_wg) keeps its own entry, written by the thread that writes
// the group holding it.
__device__ void write_own_start(const KArgs& a, const Split& sp, int gidx, const Group& g, int unit0) {
  const int w = a.plan_wg - sp.base;
  if (w < 0 || w >= sp.nw) return;
  const int lo = static_cast<int>(floor_div(static_cast<int64_t>(w) * sp.U, sp.nw));
  const int64_t e = unit0 + static_cast<int64_t>(g.nch - 1) * sp.NT;
  if (lo <= unit0 - sp.NT || lo > e) return;
  const int hi = static_cast<int>(floor_div(static_cast<int64_t>(w + 1) * sp.U, sp.nw));
  a.wgs[0] = start_entry_of(sp, gidx, g, unit0, lo, hi);
}

// A whole-grid plan (plan_wg < 0): the thread that writes group g (index
// gidx in its list) also writes the entry of the first workgroup whose range
// starts inside it, if any, and marks it: own[base + w] = rank + 1, where
// rank orders the groups of list 0 and then those of list 1.  Ownership is
// contiguous, so the running maximum of the marks gives every later
// workgroup of the group its group.
__device__ __forceinline__ void mark_start(const KArgs& a, const Split& sp, int gidx, int rank, const Group& g,
                                           int unit0, uint32_t* own) {
  const int NT = sp.NT, nw = sp.nw;
  const int w0 = static_cast<int>(ceil_div((static_cast<int64_t>(unit0) - NT + 1) * nw, sp.U));
  if (w0 >= nw) return;
  const int lo = static_cast<int>(floor_div(static_cast<int64_t>(w0) * sp.U, nw));
  if (lo > unit0 + static_cast<int64_t>(g.nch - 1) * NT) return;
  const int hi = static_cast<int>(floor_div(static_cast<int64_t>(w0 + 1) * sp.U, nw));
  a.wgs[sp.base + w0] = start_entry_of(sp, gidx, g, unit0, lo, hi);
  own[sp.base + w0] = static_cast<uint32_t>(rank + 1);
}

// The start entries of the unmarked score workgroups (see mark_start), once
// the lists are in memory: a running maximum over the W marks in LDS
// (contiguous spans per thread; own[e] becomes 2 max + marked), then each
// thread takes K entries per round, their loads of the group and its first
// unit issued together.  A workgroup of a list (nw workgroups over U units)
// whose range starts past the list's last item start (lo + NT > U) has no
// work.
template <int PT>
__device__ void write_all_starts(const KArgs& a, const Split& s0, const Split& s1, uint32_t* own, uint32_t* sh) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  constexpr int NW = PT / 64;
  const int W = s0.nw + s1.nw;
  const int C = (W + PT - 1) / PT;
  const int e_lo = min(W, tid * C), e_hi = min(W, e_lo + C);
  uint32_t m = 0;
  for (int e = e_lo; e < e_hi; ++e) m = max(m, own[e]);
  // maximum over the threads before this one
  const uint32_t inc = wave_inclusive_max(m);
  if constexpr (NW > 1) {
    if (lane == 63) sh[wave] = inc;
    __syncthreads();
  }
  uint32_t before = static_cast<uint32_t>(__shfl_up(static_cast<int>(inc), 1));
  if (lane == 0) before = 0;
#pragma unroll
  for (int w = 0; w < NW - 1; ++w)
    if (w < wave) before = max(before, sh[w]);
  for (int e = e_lo; e < e_hi; ++e) {
    const uint32_t v = own[e];
    before = max(before, v);
    own[e] = 2 * before + (v != 0 ? 1u : 0u);
  }
  __syncthreads();
  constexpr int K = PT >= 1024 ? 2 : 8;
  for (int e0 = tid; e0 < W; e0 += K * PT) {
    int l[K], g[K], lo[K];
    bool live[K], done[K];
    Group grp[K];
    int u0[K];
#pragma unroll
    for (int k = 0; k < K; ++k) {
      const int e = e0 + k * PT;
      l[k] = e >= s0.nw ? 1 : 0;
      const Split& s = l[k] ? s1 : s0;
      lo[k] = 0;
      g[k] = 0;
      live[k] = false;
      done[k] = true;
      if (e < W) {
        const uint32_t x = own[e];
        done[k] = (x & 1u) != 0;  // written with its group
        lo[k] = static_cast<int>(floor_div(static_cast<int64_t>(e - s.base) * s.U, s.nw));
        live[k] = !done[k] && lo[k] + s.NT <= s.U;
        g[k] = static_cast<int>(x >> 1) - 1 - (l[k] ? s0.ng : 0);
      }
    }
#pragma unroll
    for (int k = 0; k < K; ++k) {
      if (live[k]) {
        grp[k] = a.groups[static_cast<int64_t>(l[k]) * a.T + g[k]];
        u0[k] = a.ustart[static_cast<int64_t>(l[k]) * (a.T + 1) + g[k]];
      }
    }
#pragma unroll
    for (int k = 0; k < K; ++k) {
      const int e = e0 + k * PT;
      if (done[k]) continue;
      const Split& s = l[k] ? s1 : s0;
      WgStart st = {};
      st.g = -1;
      if (live[k]) {
        const int hi = static_cast<int>(floor_div(static_cast<int64_t>(e - s.base + 1) * s.U, s.nw));
        st = start_entry_of(s, g[k], grp[k], u0[k], lo[k], hi);
      }
      a.wgs[e] = st;
    }
  }
}

// The plan proper, on request metadata m (an LDS copy or global memory), by
// PT threads.  A plan for the whole grid (plan_wg < 0, GRID) marks the
// workgroups' first groups in own (kMaxScoreWGs LDS words, zero on entry)
// and writes the start entries after the lists; a workgroup planning for
// itself (plan_wg >= 0) keeps its own entry only.
template <int PT, bool GRID>
__device__ __forceinline__ void plan_body(const KArgs& a, const Meta& m, uint32_t* sh, uint32_t* own) {
  const int tid = threadIdx.x;
  const int T = a.T;
  const int per = (T + PT - 1) / PT;
  const int t_lo = min(T, tid * per);
  const int t_hi = min(T, t_lo + per);
  uint32_t cnt[4] = {0, 0, 0, 0};  // groups and units of list 0, then of list 1
  // with one token per thread (T <= 1024) the second pass reuses the first's
  // results instead of looking the request up again
  int kind1 = 0, tv1 = 0;
  Group g1c{};
  if (t_lo < t_hi) {
    int b = request_of(m, a.B, t_lo + a.t_base);
    ReqView r = request_view(a, m, b, true);
    for (int t = t_lo; t < t_hi; ++t) {
      const int tg = t + a.t_base;
      while (tg >= r.q1 && b + 1 < a.B) r = request_view(a, m, ++b, true);
      if (tg < r.q0 || tg >= r.q1) continue;
      if (per == 1) tv1 = visible(a, r.S - (r.q1 - r.q0) + (tg - r.q0), r.L);
      const int kind = group_kind(a, r, tg);
      if (kind == 0) continue;
      const Group g = make_group(a, b, r, t, tg, kind == 1 ? kGroupTokens : 1);
      if (per == 1) {
        kind1 = kind;
        g1c = g;
      }
      const uint32_t units = static_cast<uint32_t>(g.nch * g.ntok);
      if (kind == 1) {
        cnt[0] += 1;
        cnt[1] += units;
      } else {
        cnt[2] += 1;
        cnt[3] += units;
      }
    }
  }
  uint32_t tot[4];
  block_exclusive_scan_n<PT, 4>(cnt, tot, sh);  // also orders the clears below
  // one grid shared by the lists in proportion to their units, or (when the
  // multi list has a kernel of its own) one grid per list
  const int W = a.multi_grid > 0 ? a.multi_grid + a.score_grid : a.score_grid;
  const int Wm = a.multi_grid > 0 ? a.multi_grid
                                  : multi_workgroups(W, static_cast<int>(tot[1]), static_cast<int>(tot[3]));
  auto split = [&](int l) {
    Split sp;
    sp.list = l;
    sp.ng = static_cast<int>(tot[2 * l]);
    sp.NT = l == 0 ? kGroupTokens : 1;
    sp.nw = l == 0 ? Wm : W - Wm;
    sp.U = static_cast<int>(tot[2 * l + 1]);
    sp.base = l == 0 ? 0 : Wm;
    return sp;
  };
  const Split sp0 = split(0), sp1 = split(1);
  if (per == 1 && t_lo < t_hi) {
    a.tokv[2 * t_lo] = tv1;
    if (kind1 != 0) {
      const int l = kind1 - 1;
      const uint32_t gi = l == 0 ? cnt[0] : cnt[2], ui = l == 0 ? cnt[1] : cnt[3];
      a.groups[l * T + gi] = g1c;
      a.ustart[l * (T + 1) + gi] = static_cast<int32_t>(ui);
      if (g1c.nch > 0) {
        if (a.plan_wg >= 0)
          write_own_start(a, l == 0 ? sp0 : sp1, static_cast<int>(gi), g1c, static_cast<int>(ui));
        else if (GRID)
          mark_start(a, l == 0 ? sp0 : sp1, static_cast<int>(gi), static_cast<int>(gi + (l == 0 ? 0u : tot[0])),
                     g1c, static_cast<int>(ui), own);
      }
    }
  } else if (t_lo < t_hi) {
    // running group index and first unit of list 0, then of list 1
    uint32_t g0 = cnt[0], u0 = cnt[1], g1 = cnt[2], u1 = cnt[3];
    int b = request_of(m, a.B, t_lo + a.t_base);
    ReqView r = request_view(a, m, b, false);
    for (int t = t_lo; t < t_hi; ++t) {
      const int tg = t + a.t_base;
      while (tg >= r.q1 && b + 1 < a.B) r = request_view(a, m, ++b, false);
      const bool in = tg >= r.q0 && tg < r.q1;
      a.tokv[2 * t] = in ? visible(a, r.S - (r.q1 - r.q0) + (tg - r.q0), r.L) : 0;
      if (!in) continue;
      const int kind = group_kind(a, r, tg);
      if (kind == 0) continue;
      const int l = kind - 1;
      const Group g = make_group(a, b, r, t, tg, kind == 1 ? kGroupTokens : 1);
      const uint32_t gi = l == 0 ? g0 : g1, ui = l == 0 ? u0 : u1;
      a.groups[l * T + gi] = g;
      a.ustart[l * (T + 1) + gi] = static_cast<int32_t>(ui);
      if (g.nch > 0) {
        if (a.plan_wg >= 0)
          write_own_start(a, l == 0 ? sp0 : sp1, static_cast<int>(gi), g, static_cast<int>(ui));
        else if (GRID)
          mark_start(a, l == 0 ? sp0 : sp1, static_cast<int>(gi), static_cast<int>(gi + (l == 0 ? 0u : tot[0])),
                     g, static_cast<int>(ui), own);
      }
      const uint32_t units = static_cast<uint32_t>(g.nch * g.ntok);
      if (l == 0) {
        g0 += 1;
        u0 += units;
      } else {
        g1 += 1;
        u1 += units;
      }
    }
  }
  if (tid == 0) {
    for (int l = 0; l < 2; ++l) {
      if (a.hdr) {
        a.hdr->ngroups[l] = static_cast<int32_t>(tot[2 * l]);
        a.hdr->units[l] = static_cast<int32_t>(tot[2 * l + 1]);
      }
      a.ustart[l * (T + 1) + tot[2 * l]] = static_cast<int32_t>(tot[2 * l + 1]);
    }
  }
  if (GRID && a.plan_wg < 0) {
    __syncthreads();  // the lists and the marks are written
    write_all_starts<PT>(a, sp0, sp1, own, sh);
  }
}

// Every request holds exactly one query token (qsl[b] = b for b <= B, B <=
// 64) and the slice's tokens are requests' tokens (t_base + T <= B): the
// usual decode batch.  Every wave evaluates it (same result).
__device__ __forceinline__ bool plan_one_token_per_request(const KArgs& a, const Meta& m) {
  const int lane = threadIdx.x & 63;
  const bool ok = (lane > a.B || m.qsl[lane] == lane) && (a.B < 64 || m.qsl[64] == 64);
  return __ballot(ok) == ~0ull && a.t_base + a.T <= a.B;
}

// The lists of a batch whose requests hold one token each (the same lists
// as plan_body), by wave 0: token t (lane t) is request t_base + t, a single
// group of ceil(V/256) units; the unit prefix is one wave scan.  Returns
// the lane's group, its first unit and unit count, and the total.
struct SingleLane {
  Group g;
  uint32_t excl, units, U;
};
__device__ __forceinline__ SingleLane single_token_lists(const KArgs& a, const Meta& m) {
  const int t = threadIdx.x;
  const int T = a.T;
  const bool in = t < T;
  SingleLane s{};
  if (in) {
    const int b = t + a.t_base;
    const ReqView r = request_view(a, m, b, true);
    s.g = make_group(a, b, r, t, b, 1);
    s.units = static_cast<uint32_t>(s.g.nch);
    a.tokv[2 * t] = s.g.n0;
  }
  const uint32_t incl = wave_inclusive_scan(s.units);
  s.excl = incl - s.units;
  s.U = static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(incl), 63));
  if (in) {
    a.groups[T + t] = s.g;                      // list 1 (single groups)
    a.ustart[(T + 1) + t] = static_cast<int32_t>(s.excl);
  }
  if (t == 0) {
    a.ustart[0] = 0;                            // list 0 is empty
    a.ustart[(T + 1) + T] = static_cast<int32_t>(s.U);
  }
  return s;
}

// Start entry of workgroup w of W over the single list (U units), whose
// range starts at unit lo inside group gi (first unit excl).
__device__ __forceinline__ WgStart single_start(const Group& g, int gi, int ng, uint32_t excl, int64_t lo,
                                                int w, int W, uint32_t U) {
  WgStart st;
  st.grp = g;
  st.list = 1;
  st.ng = ng;
  st.g = gi;
  st.c = static_cast<int>(lo - excl);
  st.unit = static_cast<int>(lo);
  st.hi = static_cast<int>(floor_div(static_cast<int64_t>(w + 1) * U, W));
  st.pad[0] = st.pad[1] = 0;
  return st;
}

// That plan for the one workgroup plan_wg: the group holding unit
// floor(w U / W) is found with one ballot.
__device__ void plan_single_tokens(const KArgs& a, const Meta& m) {
  if (threadIdx.x >= 64) return;
  const int t = threadIdx.x;
  const SingleLane s = single_token_lists(a, m);
  const int W = a.score_grid;
  const int w = a.plan_wg;
  const int64_t lo = floor_div(static_cast<int64_t>(w) * s.U, W);
  const bool holds = t < a.T && s.units > 0 && s.excl <= lo && lo < s.excl + s.units;
  const uint64_t mask = __ballot(holds);
  if (mask != 0 && t == __builtin_ctzll(mask)) a.wgs[0] = single_start(s.g, t, a.T, s.excl, lo, w, W, s.U);
}

// That plan for the whole grid, by PT threads: after the lists, every
// thread takes workgroups w, w + PT, ...: the group holding unit
// floor(w U / W) is the last token whose first unit is at most that (a
// binary search over the 64 prefixes in LDS; tokens without units share
// their successor's prefix and are never the last such).  A workgroup whose
// range starts at U or beyond has no work.
template <int PT>
__device__ void plan_single_tokens_grid(const KArgs& a, const Meta& m, uint32_t* sh) {
  const int tid = threadIdx.x;
  const int T = a.T;
  if (tid < 64) {
    const SingleLane s = single_token_lists(a, m);
    sh[tid] = s.excl;
    if (tid == 0) sh[64] = s.U;  // the first word past the scan scratch (marks are unused here)
  }
  __syncthreads();  // the prefixes in LDS, the groups in memory
  const uint32_t U = sh[64];
  const int W = a.score_grid;
  for (int w = tid; w < W; w += PT) {
    const int64_t lo = floor_div(static_cast<int64_t>(w) * U, W);
    WgStart st = {};
    st.g = -1;
    if (lo < static_cast<int64_t>(U)) {
      int t = 0;  // sh[0] = 0 <= lo
#pragma unroll
      for (int step = 32; step > 0; step >>= 1)
        if (t + step < T && sh[t + step] <= lo) t += step;
      st = single_start(a.groups[T + t], t, T, sh[t], lo, w, W, U);
    }
    a.wgs[w] = st;
  }
}

// PT threads (a consumer-prep workgroup, a plan workgroup, one wave for
// small batches, where no cross-wave barrier is needed, or a score
// workgroup planning for itself).  The metadata of up to NREQ requests is
// staged in LDS (3 NREQ + 65 words); a plan for the whole grid (the
// default NREQ, kPlanLdsWords words) also keeps one mark per score
// workgroup after them (a score workgroup planning for itself does not).
template <int PT, int NREQ>
__device__ void plan_role(const KArgs& a, uint32_t* lds) {
  constexpr bool kGrid = NREQ == kPlanLdsRequests;
  int32_t* s_qsl = reinterpret_cast<int32_t*>(lds);
  int32_t* s_klen = s_qsl + NREQ + 1;
  int32_t* s_smod = s_klen + NREQ;
  uint32_t* sh = reinterpret_cast<uint32_t*>(s_smod + NREQ);
  uint32_t* own = sh + 64;
  const int tid = threadIdx.x;
  if (kGrid && a.plan_wg < 0)
    for (int w = tid; w < a.multi_grid + a.score_grid; w += PT) own[w] = 0;
  // a workgroup that plans for itself begins with "no work" (the barriers
  // below order this store before the plan's); a plan for the whole grid
  // writes every entry after the lists
  if (a.plan_wg >= 0 && tid == 0) {
    WgStart st = {};
    st.g = -1;
    a.wgs[0] = st;
  }
  if (a.B <= NREQ) {
    for (int i = tid; i <= a.B; i += PT) {
      s_qsl[i] = a.qsl[i];
      if (i < a.B) {
        s_klen[i] = a.klen[i];
        s_smod[i] = a.smod ? a.smod[i] : 0;
      }
    }
    __syncthreads();
    const Meta m{s_qsl, s_klen, a.smod ? s_smod : nullptr};
    if (a.multi_grid == 0 && a.B <= 64 && plan_one_token_per_request(a, m)) {
      if (a.plan_wg >= 0) {
        plan_single_tokens(a, m);  // wave 0; the caller's barrier publishes the lists
        return;
      }
      if (kGrid) {
        plan_single_tokens_grid<PT>(a, m, sh);
        return;
      }
    }
    plan_body<PT, kGrid>(a, m, sh, own);
  } else {
    plan_body<PT, kGrid>(a, global_meta(a), sh, own);
  }
}

template <int PT>
__global__ __launch_bounds__(PT) void plan_kernel(KArgs a) {
  __shared__ uint32_t lds[kPlanLdsWords];
  plan_role<PT>(a, lds);
}

// ---------------------------------------------------------------------------
// score: persistent, pipelined
// ---------------------------------------------------------------------------
constexpr int kScoreThreads = 256;
// batches of at most this many tokens and requests plan inside the score kernel
constexpr int kFusedTokens = 64;

// Work-item cursor over one list (wave-uniform).
struct Cursor {
  int g, c, unit;
  bool valid;
  Group grp;
};

struct ListView {
  const Group* groups;
  const int32_t* ustart;
  int ng;
};

__device__ __forceinline__ void load_group(const ListView& L, int g, Cursor& cu) {
  cu.g = g;
  const Group gr = L.groups[g];  // wave-uniform (LDS reads land in vector registers)
  cu.grp.t0 = __builtin_amdgcn_readfirstlane(gr.t0);
  cu.grp.ntok = __builtin_amdgcn_readfirstlane(gr.ntok);
  cu.grp.b = __builtin_amdgcn_readfirstlane(gr.b);
  cu.grp.nch = __builtin_amdgcn_readfirstlane(gr.nch);
  cu.grp.p0 = __builtin_amdgcn_readfirstlane(gr.p0);
  cu.grp.L = __builtin_amdgcn_readfirstlane(gr.L);
  cu.grp.n0 = __builtin_amdgcn_readfirstlane(gr.n0);
  cu.grp.nlast = __builtin_amdgcn_readfirstlane(gr.nlast);
  cu.unit = __builtin_amdgcn_readfirstlane(L.ustart[g]);
  cu.c = 0;
}

__device__ Cursor next_item(const ListView& L, Cursor cu, int hi) {
  if (!cu.valid) return cu;
  cu.c += 1;
  cu.unit += cu.grp.ntok;
  while (cu.c >= cu.grp.nch) {
    if (cu.g + 1 >= L.ng) {
      cu.valid = false;
      return cu;
    }
    load_group(L, cu.g + 1, cu);
  }
  cu.valid = cu.unit < hi;
  return cu;
}

// Staging of one work item.  The block lookups run ahead of the K loads and
// every global load is issued unconditionally (a block without K rows reads
// page 0, row 0, which always exists, and is masked through its scale), so
// that the number of loads in flight is fixed and known to the compiler.
//
// Lane j < 8 of wave w owns block q of the item's 32 blocks of 8 slots:
// q = 4j + w when the waves share the item (multi groups), q = 8w + j when
// each wave stages the 64 slots it scores itself (OWN, single groups: the
// waves then need no workgroup barrier per item).  stage_addr only issues
// the lookup of that block's page (dense: block-table entry; consumer: the
// prepared page row of the slot block) and records what it needs to check
// it; resolve() uses the loaded value later.
struct Addr {
  int raw;   // loaded block-table entry / prepared page row
  int meta;  // bit 31: block wanted; bit 30: table index in range; low bits: row in page
  int t0, ntok;  // the tokens sharing the block (marked when its page is out of contract)
};

// A token with a block on an out-of-contract page gets tokv[t][1] = the
// launch's epoch: its selection then takes the general path, which leaves
// out its zero keys.  Plain stores of one value by every writer; a stale
// entry that happens to equal the epoch only sends a token down the
// general path, which returns the same selection when every key is valid.

template <bool CONSUMER, bool OWN>
__device__ __forceinline__ void stage_addr(const KArgs& a, const Group& gr, int c, bool valid,
                                           int wave, int lane, Addr& ad) {
  const int j = lane & 7;
  const int q = OWN ? 8 * wave + j : 4 * j + wave;
  ad.t0 = gr.t0;
  ad.ntok = gr.ntok;
  if (CONSUMER) {
    const int s = c * 32 + q;
    ad.raw = a.srow[static_cast<int64_t>(gr.t0) * a.cb_in + min(s, a.cb_in - 1)];
    ad.meta = (valid && 8 * s < gr.n0) ? (3 << 30) : 0;
  } else {
    const int pos0 = c * kChunk + 8 * q;
    const int idx = pos0 >> a.rlog;
    ad.raw = a.bt[static_cast<int64_t>(gr.b) * a.bt_stride + min(idx, a.bt_stride - 1)];
    ad.meta = ((valid && pos0 < gr.nlast) ? (1 << 31) : 0) | (idx < a.bt_stride ? (1 << 30) : 0) |
              (pos0 & (a.R - 1));
  }
}

// page * page_rows + first row of the lane's block, or -1 (no K rows).
template <bool CONSUMER>
__device__ __forceinline__ int resolve(const KArgs& a, const Addr& ad, bool& bad) {
  const bool want = ad.meta < 0;  // bit 31
  if (CONSUMER) return want && ad.raw >= 0 ? ad.raw : -1;
  const bool ok = want && (ad.meta & (1 << 30)) && ad.raw >= 0 && ad.raw < a.num_pages;
  if (want && !ok) {  // rare: mark every token of the group
    bad = true;
    for (int i = 0; i < ad.ntok; ++i) a.tokv[2 * (ad.t0 + i) + 1] = static_cast<int32_t>(a.epoch);
  }
  return ok ? ad.raw * a.R + (ad.meta & (a.R - 1)) : -1;
}

// K rows of the wave's 8 blocks (8 x 16 B per lane) and their scales
// (16 B per block; lanes j and j + 8k all read block j's run), given the
// resolved block rows v (lane j holds block j's row, or -1).  STREAM: K
// rows are read once per call (decode single-token groups), so they bypass
// cache retention (non-temporal loads).
template <bool STREAM>
__device__ __forceinline__ void stage_load(const KArgs& a, int v, int lane, i32x4 (&kr)[8],
                                           i32x4& sc) {
  // the scales first: consumed first (stage_store), so waiting for them
  // never waits for anything issued after the K rows
  const int row = v < 0 ? 0 : v;
  sc = *reinterpret_cast<const i32x4*>(a.ks + static_cast<int64_t>(row >> a.rlog) * a.sstride +
                                       static_cast<int64_t>(row & (a.R - 1)) * 2);
  const int lane_off = (lane >> 3) * 128 + (lane & 7) * 16;
#pragma unroll
  for (int u = 0; u < 8; ++u) {
    const int vu = __builtin_amdgcn_readlane(v, u);
    const int row = vu < 0 ? 0 : vu;
    const int8_t* src = a.k + static_cast<int64_t>(row >> a.rlog) * a.kstride +
                        static_cast<int64_t>(row & (a.R - 1)) * 128 + lane_off;
    const i32x4* p = reinterpret_cast<const i32x4*>(src);
    kr[u] = STREAM ? __builtin_nontemporal_load(p) : *p;
  }
}

// 16-byte slot of column group col (0..7) of tile row row (128 bytes).  The
// LDS serves a 128-bit read 16 lanes at a time over 64 four-byte banks, so
// two consecutive rows share the banks once and 16 consecutive rows reading
// one column group (an MFMA B operand) must spread over the 8 slots in both
// halves: slot = col ^ ((row / 2) mod 8).  Writes of one row (8 lanes, all
// column groups) stay conflict-free as well.
__device__ __forceinline__ int tile_slot(int row, int col) { return col ^ ((row >> 1) & 7); }

// Into LDS: K tile rows with the XOR swizzle, scales of valid blocks (0xFFFF
// halves mark a block without K rows).
template <bool OWN>
__device__ __forceinline__ void stage_store(int8_t* tile, uint16_t* ksc, const i32x4 (&kr)[8],
                                            const i32x4& sc, int v, int wave, int lane) {
  if (lane < 8) {
    const i32x4 none = {-1, -1, -1, -1};
    *reinterpret_cast<i32x4*>(ksc + 8 * (OWN ? 8 * wave + lane : 4 * lane + wave)) = v < 0 ? none : sc;
  }
#pragma unroll
  for (int u = 0; u < 8; ++u) {
    const int row = 8 * (OWN ? 8 * wave + u : 4 * u + wave) + (lane >> 3);
    const int col = lane & 7;
    *reinterpret_cast<i32x4*>(tile + row * 128 + (tile_slot(row, col) << 4)) = kr[u];
  }
}

// Queries of one token as MFMA A operands, and its fp16 head multipliers.
// A rows are permuted so that the C register i of lane group g of a head
// tile is the head that the epilogue needs there (see score_subtile):
//   SPLIT (32-head tiles scored one after the other): tile m, group g,
//     register i -> head 32m + 16g + i;
//   otherwise (all tiles interleaved): tile m, group g, register i ->
//     head g*N/2 + 16m + i.
template <int NH, bool SPLIT>
struct QState {
  i32x4 qa[NH / 32][4];
  h2 mh[NH / 4];  // pairs of multipliers in the order the epilogue consumes them
  int tok;
  bool scaled;    // mh holds m * 2^11 (every |m| < 32): the scaled epilogue applies
};

template <int NH, bool SPLIT>
__device__ __forceinline__ void load_q(const KArgs& a, int t, int lane, QState<NH, SPLIT>& qs) {
  constexpr int HALF = NH / 2;
  const int r = lane & 31, g = lane >> 5;
#pragma unroll
  for (int m = 0; m < NH / 32; ++m) {
    const int head = SPLIT ? 32 * m + ((r >> 2) & 1) * 16 + 4 * (r >> 3) + (r & 3)
                           : ((r >> 2) & 1) * HALF + 16 * m + 4 * (r >> 3) + (r & 3);
    const int8_t* qrow = a.q + (static_cast<int64_t>(t) * NH + head) * 128 + 64 * g;
#pragma unroll
    for (int s = 0; s < 4; ++s) qs.qa[m][s] = *reinterpret_cast<const i32x4*>(qrow + 16 * s);
  }
  const uint32_t* wr = reinterpret_cast<const uint32_t*>(a.w + static_cast<int64_t>(t) * NH);
  const uint32_t* qr = reinterpret_cast<const uint32_t*>(a.qs + static_cast<int64_t>(t) * NH);
#pragma unroll
  for (int j = 0; j < HALF / 2; ++j) {
    // pair j covers heads (SPLIT) 32*(j/8) + 16g + 2*(j%8) or (else) g*N/2 + 2j
    const int h0 = SPLIT ? 32 * (j >> 3) + 16 * g + 2 * (j & 7) : g * HALF + 2 * j;
    qs.mh[j] = as_h2(wr[h0 >> 1]) * as_h2(qr[h0 >> 1]);  // fp16 RNE
  }
  // the scaled epilogue needs m * 2^11 finite for every head of the token
  // (NaN and infinite multipliers fail the test as well)
  bool small = true;
#pragma unroll
  for (int j = 0; j < HALF / 2; ++j) {
    const uint32_t u = as_u32(qs.mh[j]);
    small = small && (u & 0x7FFFu) < kHalfAbs32 && ((u >> 16) & 0x7FFFu) < kHalfAbs32;
  }
  qs.scaled = __builtin_amdgcn_ballot_w64(!small) == 0;
  if (qs.scaled) {
    const h2 k2048 = {static_cast<_Float16>(2048.0f), static_cast<_Float16>(2048.0f)};
#pragma unroll
    for (int j = 0; j < HALF / 2; ++j) qs.mh[j] = qs.mh[j] * k2048;  // exact
  }
  qs.tok = t;
}

// Query sources for score_subtile: fragments and multipliers in registers
// (multi groups: every wave may hold another token), or in LDS (single
// groups: the four waves share the token).
template <int NH, bool SPLIT>
struct QRegs {
  const QState<NH, SPLIT>& q;
  __device__ __forceinline__ i32x4 frag(int m, int s, int) const { return q.qa[m][s]; }
  __device__ __forceinline__ h2 mul(int j, int) const { return q.mh[j]; }
};

// LDS layout: frag[m][s][lane] (16 B each), mul[j][group] (packed pairs).
template <int NH>
struct QLds {
  const i32x4* fr;
  const uint32_t* ml;
  __device__ __forceinline__ i32x4 frag(int m, int s, int lane) const {
    return fr[(m * 4 + s) * 64 + lane];
  }
  __device__ __forceinline__ h2 mul(int j, int lane) const { return as_h2(ml[j * 2 + (lane >> 5)]); }
};

// Fill QLds for token t (SPLIT layout), all threads of the workgroup.
// TRY_SCALED: when every head multiplier of the token has |m| < 32, ml
// holds m * 2^11 and ml[NH / 2] = 1 (the scaled epilogue applies);
// otherwise ml holds m and ml[NH / 2] = 0.
template <int NH, bool TRY_SCALED = false>
__device__ __forceinline__ void load_q_lds(const KArgs& a, int t, i32x4* fr, uint32_t* ml) {
  constexpr int MT = NH / 32;
  const int tid = threadIdx.x;
#pragma unroll
  for (int e = tid; e < MT * 256; e += kScoreThreads) {
    const int m = e >> 8, s = (e >> 6) & 3, l = e & 63;
    const int r = l & 31, g = l >> 5;
    const int head = 32 * m + ((r >> 2) & 1) * 16 + 4 * (r >> 3) + (r & 3);
    fr[e] = *reinterpret_cast<const i32x4*>(a.q + (static_cast<int64_t>(t) * NH + head) * 128 + 64 * g +
                                            16 * s);
  }
  if (tid < 64) {  // wave 0: pair j = tid >> 1 of group g = tid & 1: heads 32*(j/8) + 16g + 2*(j%8)
    uint32_t u = 0;
    bool small = true;
    if (tid < NH / 2) {
      const int j = tid >> 1, g = tid & 1;
      const int h0 = 32 * (j >> 3) + 16 * g + 2 * (j & 7);
      const uint32_t* wr = reinterpret_cast<const uint32_t*>(a.w + static_cast<int64_t>(t) * NH);
      const uint32_t* qr = reinterpret_cast<const uint32_t*>(a.qs + static_cast<int64_t>(t) * NH);
      u = as_u32(as_h2(wr[h0 >> 1]) * as_h2(qr[h0 >> 1]));  // fp16 RNE
      small = (u & 0x7FFFu) < kHalfAbs32 && ((u >> 16) & 0x7FFFu) < kHalfAbs32;
    }
    if (TRY_SCALED) {
      // m * 2^11 must stay a finite fp16 for every head (NaN and infinite
      // multipliers fail the test as well)
      const bool scaled = __builtin_amdgcn_ballot_w64(!small) == 0;
      const h2 k2048 = {static_cast<_Float16>(2048.0f), static_cast<_Float16>(2048.0f)};
      if (scaled) u = as_u32(as_h2(u) * k2048);  // exact
      if (tid == 0) ml[NH / 2] = scaled ? 1u : 0u;
    }
    if (tid < NH / 2) ml[tid] = u;
  }
}

// Scoring of one (token, 64-slot sub-tile) of the current item, in 32-head
// passes: mfma_pass, then epi_pass per pass, then finish_subtile.
//
// MFMA operands (v_mfma_i32_32x32x32_i8, 64 lanes): A = queries, lane l
// supplies row l%32 of a 32-head tile, 16 bytes of the head dimension;
// B = keys, lane l supplies column l%32 (one position), the same 16 bytes
// (dim d = 64*(l/32) + 16*step + byte for both, so the reduction pairs
// q[h,d] with k[j,d]).  C: lane l holds column l%32, rows 8*(i/4) +
// 4*(l/32) + i%4.  With the A permutation, lanes 0..31 hold heads 32p ..
// 32p+15 and lanes 32..63 heads 32p+16 .. 32p+31 of the same 64 positions,
// and one v_permlane32_swap per register pair leaves each lane L with all
// 32 heads of the pass for slot s0+L, summed in ascending head order.
// The B fragments of one sub-tile (2 x 4 per lane), from the swizzled tile.
__device__ __forceinline__ void load_b(const int8_t* tile, int sub, int lane, i32x4 (&b)[2][4]) {
#pragma unroll
  for (int n = 0; n < 2; ++n) {
    const int row = 64 * sub + 32 * n + (lane & 31);
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      const int col = 4 * (lane >> 5) + s;
      b[n][s] = *reinterpret_cast<const i32x4*>(tile + row * 128 + (tile_slot(row, col) << 4));
    }
  }
}

// One pass from B fragments already in registers (every pass of a
// sub-tile reuses them: the matrix core would otherwise wait on LDS reads).
template <class QSrc>
__device__ __forceinline__ void mfma_pass_b(const QSrc& qs, const i32x4 (&b)[2][4], int ps, int lane,
                                            const i32x16& seed, i32x16 (&acc)[2]) {
#pragma unroll
  for (int n = 0; n < 2; ++n)
#pragma unroll
    for (int s = 0; s < 4; ++s)
      acc[n] = __builtin_amdgcn_mfma_i32_32x32x32_i8(qs.frag(ps, s, lane), b[n][s], s == 0 ? seed : acc[n],
                                                     0, 0, 0);
}

template <class QSrc>
__device__ __forceinline__ void mfma_pass(const QSrc& qs, const int8_t* tile, int sub, int ps, int lane,
                                          const i32x16& seed, i32x16 (&acc)[2]) {
#pragma unroll
  for (int n = 0; n < 2; ++n) {
    const int row = 64 * sub + 32 * n + (lane & 31);
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      const int col = 4 * (lane >> 5) + s;
      const i32x4 bk = *reinterpret_cast<const i32x4*>(tile + row * 128 + (tile_slot(row, col) << 4));
      acc[n] = __builtin_amdgcn_mfma_i32_32x32x32_i8(qs.frag(ps, s, lane), bk, s == 0 ? seed : acc[n],
                                                     0, 0, 0);
    }
  }
}

// x = fp16(qk/1024), ReLU, p = fp16(x * m) (packed two heads per word), then
// the 32 heads of the pass added to sum in ascending order.
// SCALED: the multipliers are m * 2^11 and the ReLU rides on the clamp
// (qk_relu_scaled); same products bit for bit.
template <bool PACKED_CVT, bool SCALED, class QSrc>
__device__ __forceinline__ void epi_pass(const QSrc& qs, const i32x16 (&acc)[2], int ps, int lane,
                                         float one, float& sum) {
  uint32_t pk[2][8];
#pragma unroll
  for (int n = 0; n < 2; ++n)
#pragma unroll
    for (int i = 0; i < 16; i += 2) {
      h2 x;
      if (SCALED) {
        x = h2{static_cast<_Float16>(qk_relu_scaled(acc[n][i])),
               static_cast<_Float16>(qk_relu_scaled(acc[n][i + 1]))};
      } else {
        const h2 x0 = PACKED_CVT ? h2{static_cast<_Float16>(qk_over_1024(acc[n][i])),
                                      static_cast<_Float16>(qk_over_1024(acc[n][i + 1]))}
                                 : h2{qk_to_half(acc[n][i]), qk_to_half(acc[n][i + 1])};
        x = as_h2(relu_h2(as_u32(x0)));
      }
      pk[n][i >> 1] = as_u32(x * qs.mul(ps * 8 + (i >> 1), lane));
    }
  uint32_t hi[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const auto r = __builtin_amdgcn_permlane32_swap(pk[0][j], pk[1][j], false, false);
    const h2 pl = as_h2(static_cast<uint32_t>(r[0]));
    sum = add_h(sum, pl[0], one);
    sum = add_h(sum, pl[1], one);
    hi[j] = r[1];
  }
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const h2 ph = as_h2(hi[j]);
    sum = add_h(sum, ph[0], one);
    sum = add_h(sum, ph[1], one);
  }
}

// Score (× k_scale), key, block maximum and stores of slot s0 + lane, whose
// place in its 256-slot item is 64 * sub + lane: the key goes to
// kp[64 * sub + lane] and the block maximum to bp[(64 * sub + lane) / 8]
// (kp and bp point at the item's keys, in global memory or in an LDS
// staging entry).  Every store is unconditional (slots past n_i receive key
// 0, block maxima are written by all 8 lanes of a block), so the memory
// operations of a sub-tile are fixed.
template <int MODE, bool DBG>
__device__ __forceinline__ void finish_subtile(const KArgs& a, const uint16_t* ksc, int sub, int t, int s0,
                                               int n_i, int lane, float sum, uint32_t* kp, uint32_t* bp) {
  const int slot = s0 + lane;
  const int local = 64 * sub + lane;
  const uint16_t kb = ksc[64 * sub + lane];
  const bool valid = slot < n_i && kb != 0xFFFFu;
  const float score = sum * static_cast<float>(__builtin_bit_cast(_Float16, kb));
  const uint32_t key = valid ? order_key(score) : 0u;
  if (DBG && valid) {
    const int pos = MODE == QLI_MODE_CONSUMER
                        ? a.slots[static_cast<int64_t>(t) * a.cb_in + (slot >> 3)] * 8 + (slot & 7)
                        : slot;
    a.dbg[static_cast<int64_t>(t) * a.max_k_len + pos] = score;
  }
  kp[local] = key;
  if (MODE == QLI_MODE_SOURCE) {
    uint32_t bk = key;
    // maximum over the 8 lanes of the block on DPP (no LDS round trips):
    // pairs, quads, then the half-row mirror, which maps each quad of an
    // 8-lane half-row onto the other
    bk = max(bk, dpp_all<0xB1>(bk));   // quad_perm [1, 0, 3, 2]
    bk = max(bk, dpp_all<0x4E>(bk));   // quad_perm [2, 3, 0, 1]
    bk = max(bk, dpp_all<0x141>(bk));  // row_half_mirror
    bp[local >> 3] = bk;
  }
}

// Debug only: the exact q.k of one pass's accumulators (lane l holds heads
// 32 ps + 16 (l / 32) + i, i < 16, for slot s0 + 32 n + l % 32 of accumulator
// n; the accumulator holds the seed plus q.k), stored where the slot is
// eligible.
template <int NH, int MODE>
__device__ __forceinline__ void dbg_store_qk(const KArgs& a, const i32x16 (&acc)[2], int ps, int t,
                                             int s0, int n_i, const uint16_t* ksc, int sub, int lane) {
  if (!a.dbg_qk) return;
#pragma unroll
  for (int n = 0; n < 2; ++n) {
    const int in_tile = 32 * n + (lane & 31);
    const int slot = s0 + in_tile;
    if (slot >= n_i || ksc[64 * sub + in_tile] == 0xFFFFu) continue;
    const int pos = MODE == QLI_MODE_CONSUMER
                        ? a.slots[static_cast<int64_t>(t) * a.cb_in + (slot >> 3)] * 8 + (slot & 7)
                        : slot;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int head = 32 * ps + 16 * (lane >> 5) + i;
      a.dbg_qk[(static_cast<int64_t>(t) * NH + head) * a.max_k_len + pos] = acc[n][i] - kSeedBits;
    }
  }
}

// One sub-tile, the passes one after the other (a loop: overlapping them
// would keep two head tiles of accumulators live).  scaled (wave-uniform):
// the multipliers are m * 2^11 and the scaled epilogue with a packed
// conversion applies (fewer VALU instructions where they bound the kernel);
// otherwise the plain epilogue with the mixed-precision conversion.
template <int NH, int MODE, bool DBG, class QSrc>
__device__ __forceinline__ void score_subtile(const KArgs& a, const QSrc& qs,
                                              const int8_t* tile, const uint16_t* ksc, int sub,
                                              int t, int s0, int n_i, int lane, const i32x16& seed,
                                              uint32_t* kp, uint32_t* bp, bool scaled = false) {
  float sum = 0.0f;
#pragma unroll 1
  for (int ps = 0; ps < NH / 32; ++ps) {
    i32x16 acc[2];
    mfma_pass(qs, tile, sub, ps, lane, seed, acc);
    if (DBG) dbg_store_qk<NH, MODE>(a, acc, ps, t, s0, n_i, ksc, sub, lane);
    if (scaled) epi_pass<true, true>(qs, acc, ps, lane, a.one, sum);
    else epi_pass<false, false>(qs, acc, ps, lane, a.one, sum);
  }
  finish_subtile<MODE, DBG>(a, ksc, sub, t, s0, n_i, lane, sum, kp, bp);
}

// Multi groups (prefill shapes): each item is 256 slots for 4 consecutive
// tokens of one request; wave w scores the four 64-slot sub-tiles of token
// t0 + w, keeping its queries in registers.  The item's (sub-tile, pass)
// units form a software pipeline: the MFMAs of unit u + 1 are issued
// before the epilogue of unit u, so the matrix core runs under the VALU
// epilogue (two accumulator sets alternate).
//
// K staging, two LDS buffers: item i is scored from buffer i & 1 while,
// halfway through it, each wave writes its part of item i + 1 (loaded into
// registers halfway through item i - 1) into the other buffer and issues
// the loads of item i + 2; the block-table lookups of item i + 2 are issued
// when item i starts.  One workgroup barrier per item, at its end: every
// wave has finished reading buffer i & 1 and written its part of item i + 1.
// Waiting for K rows halfway through an item therefore never waits for
// loads or score stores issued just before (the memory counter is in
// order, so waiting for the last K load also waits for every older store).
template <int NH, int MODE, bool DBG>
__device__ void run_multi(const KArgs& a, const ListView& L, Cursor cur, int hi, int8_t (*tile)[kChunk * 128],
                          uint16_t (*ksc)[kChunk], int wave, int lane, const i32x16& seed, bool& bad) {
  constexpr int P = NH / 32;   // passes per sub-tile
  constexpr int NU = 4 * P;    // (sub-tile, pass) units per item
  constexpr int MID = NU / 2;  // the next tile is written before the epilogue of unit MID
  Cursor n1 = next_item(L, cur, hi);
  Cursor n2 = next_item(L, n1, hi);
  Addr ad;
  i32x4 kr[8];
  i32x4 sc;
  // prologue: item 0 into buffer 0, item 1 into registers
  stage_addr<false, false>(a, cur.grp, cur.c, cur.valid, wave, lane, ad);
  int v = resolve<false>(a, ad, bad);
  stage_load<false>(a, v, lane, kr, sc);
  stage_addr<false, false>(a, n1.grp, n1.c, n1.valid, wave, lane, ad);
  stage_store<false>(tile[0], ksc[0], kr, sc, v, wave, lane);
  v = resolve<false>(a, ad, bad);
  stage_load<false>(a, v, lane, kr, sc);
  __syncthreads();
  QState<NH, true> qs;
  qs.tok = -1;
  int buf = 0;
  const float one = a.one;
  while (cur.valid) {
    stage_addr<false, false>(a, n2.grp, n2.c, n2.valid, wave, lane, ad);  // lookups of item i + 2
    const Group& gr = cur.grp;  // multi groups hold kGroupTokens tokens
    const int t = gr.t0 + wave;
    const int n_i = visible(a, static_cast<int64_t>(gr.p0) + wave, gr.L);
    if (t != qs.tok) load_q<NH, true>(a, t, lane, qs);
    const QRegs<NH, true> q{qs};
    const int8_t* tl = tile[buf];
    // halfway: item i + 1 into the other buffer, loads of item i + 2
    auto stage_next = [&]() {
      stage_store<false>(tile[buf ^ 1], ksc[buf ^ 1], kr, sc, v, wave, lane);
      v = resolve<false>(a, ad, bad);
      stage_load<false>(a, v, lane, kr, sc);
    };
    if (qs.scaled) {
      // the item's units, pipelined, with the scaled epilogue
      i32x16 accA[2], accB[2];
      i32x4 bf[2][4];  // B fragments of the current sub-tile, shared by its passes
      float sum = 0.0f;
      load_b(tl, 0, lane, bf);
      mfma_pass_b(q, bf, 0, lane, seed, accA);
#pragma unroll
      for (int u = 0; u < NU; ++u) {
        if (u + 1 < NU) {
          if ((u + 1) % P == 0) load_b(tl, (u + 1) / P, lane, bf);
          if (u & 1) mfma_pass_b(q, bf, (u + 1) % P, lane, seed, accA);
          else mfma_pass_b(q, bf, (u + 1) % P, lane, seed, accB);
        }
        if (u == MID) stage_next();
        if (DBG)
          dbg_store_qk<NH, MODE>(a, (u & 1) ? accB : accA, u % P, t, cur.c * kChunk + 64 * (u / P), n_i,
                                 ksc[buf], u / P, lane);
        epi_pass<true, true>(q, (u & 1) ? accB : accA, u % P, lane, one, sum);
        if (u % P == P - 1) {
          finish_subtile<MODE, DBG>(a, ksc[buf], u / P, t, cur.c * kChunk + 64 * (u / P), n_i, lane, sum,
                                    a.keys + static_cast<int64_t>(t) * a.ncap + cur.c * kChunk,
                                    MODE == QLI_MODE_SOURCE
                                        ? a.bkeys + static_cast<int64_t>(t) * a.nbcap + cur.c * (kChunk / 8)
                                        : nullptr);
          sum = 0.0f;
        }
        // each step schedules one unit's MFMAs against the previous unit's
        // epilogue, no further (bounds the live registers); inside the step
        // the compiler's own order measured faster than forced interleavings
        // of one to four MFMAs per 12 to 48 VALU instructions
        __builtin_amdgcn_sched_barrier(0);
      }
    } else {
      // a token with some |m| >= 32 (never in practice): the plain
      // epilogue, one sub-tile after the other (wave-uniform branch: each
      // wave scores one token)
#pragma unroll 1
      for (int sub = 0; sub < 4; ++sub) {
        if (sub == 2) stage_next();
        float sum = 0.0f;
#pragma unroll
        for (int ps = 0; ps < P; ++ps) {  // unrolled: the multipliers stay in registers
          i32x16 acc[2];
          mfma_pass(q, tl, sub, ps, lane, seed, acc);
          if (DBG)
            dbg_store_qk<NH, MODE>(a, acc, ps, t, cur.c * kChunk + 64 * sub, n_i, ksc[buf], sub, lane);
          epi_pass<true, false>(q, acc, ps, lane, one, sum);
        }
        finish_subtile<MODE, DBG>(a, ksc[buf], sub, t, cur.c * kChunk + 64 * sub, n_i, lane, sum,
                                  a.keys + static_cast<int64_t>(t) * a.ncap + cur.c * kChunk,
                                  MODE == QLI_MODE_SOURCE
                                      ? a.bkeys + static_cast<int64_t>(t) * a.nbcap + cur.c * (kChunk / 8)
                                      : nullptr);
      }
    }
    __syncthreads();
    cur = n1;
    n1 = n2;
    n2 = next_item(L, n2, hi);
    buf ^= 1;
  }
}

// The dispatcher hands workgroup i to XCD i mod nxcd, and each XCD has its
// own L2.  The plan splits the work lists into contiguous ranges in token
// order (the tokens of a request are neighbours), so workgroup i takes
// start entry (i mod nxcd) * (grid / nxcd) + i / nxcd: every XCD walks one
// contiguous stretch of the lists, and the tokens of a request that read
// the same K rows share an L2 instead of fetching them through all of them.
__device__ __forceinline__ int start_entry(int i, int grid, int nxcd) {
  if (nxcd <= 1 || grid % nxcd) return i;
  return (i % nxcd) * (grid / nxcd) + i / nxcd;
}

// ---------------------------------------------------------------------------
// Multi groups at three or four workgroups per CU (prefill shapes)
// ---------------------------------------------------------------------------
// Each 256-slot item is scored as two 128-slot halves through a two-buffer
// LDS ring of 16 KB halves.  K rows go straight from global memory into the
// ring (global_load_lds, 1 KB per instruction, the tile swizzle applied on
// the global side), so no K data waits in registers; one accumulator set
// per wave.  That fits 168 VGPRs and 33 KB of LDS per workgroup: three
// workgroups per CU (four with 32 heads), the extra waves per SIMD taking
// over the overlap of matrix and vector work that two accumulator sets gave
// one wave.
// Each half: the block-table lookup of the half after next, the loads of
// the next half, then the scoring of this one; at its end every wave waits
// for its loads (the compiler does not order LDS reads after these loads,
// so the wait is explicit) and the workgroup meets at one barrier.
constexpr int kHalf = kChunk / 2;  // slots per half item

// A half item: item cursor + which half.
struct HalfCursor {
  Cursor cu;
  int h;
};

__device__ __forceinline__ HalfCursor next_half(const ListView& L, HalfCursor x, int hi) {
  if (!x.cu.valid) return x;
  if (x.h == 0) {
    x.h = 1;
    return x;
  }
  x.cu = next_item(L, x.cu, hi);
  x.h = 0;
  return x;
}

// Wave w stages rows [32w, 32w + 32) of a half (blocks 4w..4w+3, one page
// at both ratios).  The lookup of that page (one block-table entry per wave).
struct HalfAddr {
  int raw;   // loaded block-table entry
  int pos0;  // first position of the wave's 32 rows
  bool idx_ok, want;
};

__device__ __forceinline__ void half_addr(const KArgs& a, const HalfCursor& x, int wave, HalfAddr& ad) {
  const Group& g = x.cu.grp;
  ad.pos0 = x.cu.c * kChunk + x.h * kHalf + 32 * wave;
  const int idx = ad.pos0 >> a.rlog;
  ad.idx_ok = idx < a.bt_stride;
  ad.want = x.cu.valid && ad.pos0 < g.nlast;
  // one entry per wave: a scalar load (the block table is not written during
  // the call), whose wait (lgkmcnt) does not hold the wave until the K rows
  // already in flight have landed, as a vector load's would
  const auto* bt = (const __attribute__((address_space(4))) int32_t*)(a.bt);
  ad.raw = bt[static_cast<int64_t>(g.b) * a.bt_stride + min(idx, a.bt_stride - 1)];
}

// page * page_rows + row of the wave's first row, or -1 (no K rows: the
// loads then read page 0, which always exists, and the scales mark the
// blocks as not eligible).
__device__ __forceinline__ int half_resolve(const KArgs& a, const HalfCursor& x, const HalfAddr& ad,
                                            bool& bad) {
  if (!ad.want) return -1;
  const bool ok = ad.idx_ok && ad.raw >= 0 && ad.raw < a.num_pages;
  if (!ok) {  // rare: mark every token of the group
    bad = true;
    if ((threadIdx.x & 63) == 0)
      for (int i = 0; i < x.cu.grp.ntok; ++i) a.tokv[2 * (x.cu.grp.t0 + i) + 1] = static_cast<int32_t>(a.epoch);
    return -1;
  }
  return ad.raw * a.R + (ad.pos0 & (a.R - 1));
}

// Loads of the wave's 32 rows into the half tile (4 x 1 KB, straight into
// LDS) and, in lanes 0..3, the scales of its 4 blocks into sc.
__device__ __forceinline__ void half_stage(const KArgs& a, int v, int wave, int lane, int8_t* tile,
                                           i32x4& sc) {
  const int row = v < 0 ? 0 : v;
  const int8_t* base = a.k + static_cast<int64_t>(row >> a.rlog) * a.kstride +
                       static_cast<int64_t>(row & (a.R - 1)) * 128;
  // the scales first: they are read from registers before the half is scored
  sc = *reinterpret_cast<const i32x4*>(a.ks + static_cast<int64_t>(row >> a.rlog) * a.sstride +
                                       static_cast<int64_t>((row & (a.R - 1)) + 8 * (lane & 3)) * 2);
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    const int r = 32 * wave + 8 * u + (lane >> 3);  // tile row
    const int gcol = (lane & 7) ^ ((r >> 1) & 7);   // the column group LDS slot (lane & 7) holds
    const int8_t* src = base + (8 * u + (lane >> 3)) * 128 + gcol * 16;
    __builtin_amdgcn_global_load_lds(src, (__attribute__((address_space(3))) void*)(tile + (32 * wave + 8 * u) * 128),
                                     16, 0, 0);
  }
}

template <int NH, int MODE, bool DBG>
__device__ void run_multi_half(const KArgs& a, const ListView& L, Cursor cur0, int hi, int8_t* tile0,
                               int8_t* tile1, uint16_t (*ksc)[kHalf], int wave, int lane, const i32x16& seed,
                               bool& bad) {
  constexpr int P = NH / 32;  // passes per sub-tile
  HalfCursor cur{cur0, 0};
  HalfCursor n1 = next_half(L, cur, hi);
  HalfAddr ad;
  i32x4 sc;
  auto store_scales = [&](int b, int v, int wave_, const HalfCursor& x) {
    // block 4 wave + lane of the half: eligible rows start below nlast
    if (lane < 4) {
      const bool ok = v >= 0 && x.cu.c * kChunk + x.h * kHalf + 32 * wave_ + 8 * lane < x.cu.grp.nlast;
      const i32x4 none = {-1, -1, -1, -1};
      *reinterpret_cast<i32x4*>(ksc[b] + 8 * (4 * wave_ + lane)) = ok ? sc : none;
    }
  };
  // prologue: half 0 into buffer 0
  half_addr(a, cur, wave, ad);
  int v = half_resolve(a, cur, ad, bad);
  half_stage(a, v, wave, lane, tile0, sc);
  half_addr(a, n1, wave, ad);  // lookup of half 1
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  store_scales(0, v, wave, cur);
  __syncthreads();
  QState<NH, true> qs;
  qs.tok = -1;
  const float one = a.one;
  // One half: the next one's rows go to the other buffer while this one is
  // scored.  The two buffers are distinct LDS arrays and each call below
  // names them as constants, so the compiler can tell that the K rows in
  // flight (loaded straight into LDS) land in the buffer not being read and
  // does not hold the LDS reads until they arrive.
  auto step = [&](const int8_t* tl, int8_t* tn, int buf) {
    const HalfCursor n2 = next_half(L, n1, hi);
    const Group& gr = cur.cu.grp;
    const int t = gr.t0 + wave;
    // the queries before the K rows: waiting for them waits for nothing issued later
    if (t != qs.tok) load_q<NH, true>(a, t, lane, qs);
    // half n1 into the other buffer (its lookup completed at the last wait)
    const int v1 = half_resolve(a, n1, ad, bad);
    if (n1.cu.valid) half_stage(a, v1, wave, lane, tn, sc);
    half_addr(a, n2, wave, ad);  // lookup of the half after next
    const int n_i = visible(a, static_cast<int64_t>(gr.p0) + wave, gr.L);
    const QRegs<NH, true> q{qs};
    const int s0h = cur.cu.c * kChunk + cur.h * kHalf;  // first slot of the half
    uint32_t* kp = a.keys + static_cast<int64_t>(t) * a.ncap + s0h;
    uint32_t* bp = MODE == QLI_MODE_SOURCE ? a.bkeys + static_cast<int64_t>(t) * a.nbcap + s0h / 8 : nullptr;
#pragma unroll 1
    for (int sub = 0; sub < 2; ++sub) {
      // 32 heads: the sub-tile's B fragments once in registers; 64 heads:
      // read from LDS per pass (fits the register budget of three waves)
      i32x4 bf[2][4];
      if (P == 1) load_b(tl, sub, lane, bf);
      float sum = 0.0f;
#pragma unroll
      for (int ps = 0; ps < P; ++ps) {
        i32x16 acc[2];
        if (P == 1) mfma_pass_b(q, bf, ps, lane, seed, acc);
        else mfma_pass(q, tl, sub, ps, lane, seed, acc);
        if (DBG) dbg_store_qk<NH, MODE>(a, acc, ps, t, s0h + 64 * sub, n_i, ksc[buf], sub, lane);
        if (qs.scaled) epi_pass<true, true>(q, acc, ps, lane, one, sum);
        else epi_pass<true, false>(q, acc, ps, lane, one, sum);
      }
      finish_subtile<MODE, DBG>(a, ksc[buf], sub, t, s0h + 64 * sub, n_i, lane, sum, kp, bp);
    }
    // the next half's rows and lookups have landed; its scales go to LDS
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    if (n1.cu.valid) store_scales(buf ^ 1, v1, wave, n1);
    __syncthreads();
    cur = n1;
    n1 = n2;
  };
  while (cur.cu.valid) {
    step(tile0, tile1, 0);
    if (!cur.cu.valid) break;
    step(tile1, tile0, 1);
  }
}

// The multi list in a kernel of its own: four workgroups per CU with 32
// heads (127 VGPRs; 4 x 33 KB of LDS), three with 64 (157 VGPRs; the host
// launches it for 32 heads only).
__host__ __device__ constexpr int multi_wgs_per_cu(int nh) { return nh == 32 ? 4 : 3; }

template <int NH, int MODE, bool DBG>
__global__ __launch_bounds__(kScoreThreads, multi_wgs_per_cu(NH)) void score_multi_kernel(KArgs a) {
  __shared__ __attribute__((aligned(16))) int8_t tile0[kHalf * 128];
  __shared__ __attribute__((aligned(16))) int8_t tile1[kHalf * 128];
  __shared__ __attribute__((aligned(16))) uint16_t ksc[2][kHalf];
  const int wave = __builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x >> 6));
  const int lane = threadIdx.x & 63;
  const WgStart st = a.wgs[start_entry(blockIdx.x, gridDim.x, a.nxcd)];
  if (st.g < 0 || st.unit >= st.hi || st.list != 0) return;
  const ListView L{a.groups, a.ustart, st.ng};
  Cursor cu;
  cu.g = st.g;
  cu.c = st.c;
  cu.unit = st.unit;
  cu.grp = st.grp;
  cu.valid = true;
  i32x16 seed;
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    // in vector registers for the whole kernel: the MFMAs start each
    // accumulator chain from them instead of from copies of a scalar splat
    int x;
    asm volatile("v_mov_b32 %0, %1" : "=v"(x) : "i"(kSeedBits));
    seed[i] = x;
  }
  bool bad = false;
  run_multi_half<NH, MODE, DBG>(a, L, cu, st.hi, tile0, tile1, ksc, wave, lane, seed, bad);
  if (bad) raise_flag(a, QLI_DEV_BAD_PAGE);
}

// Single-token groups (decode shapes): wave w stages and scores sub-tile w
// of every item in its own LDS rows, so inside a token segment the waves
// run independently (an LDS write and a later read of the same wave are
// ordered without a barrier, which also lets one K buffer serve every item:
// a wave's next stores follow its previous reads).  Per segment the queries
// are loaded once (workgroup barriers); inside it the loop body has a fixed
// set of memory operations and keeps two items of K in flight (register
// sets A and B alternate; the body is unrolled twice).
// Each step resolves the block rows looked up one step earlier, issues the
// next lookup, then the K loads: with in-order memory counters a lookup is
// always older than the K loads that must stay in flight.
// The keys (and block maxima) of up to kKeyStage items are staged in LDS
// (the second K buffer, unused here) and written out together when the
// stage is full and at the end of the range: HBM writes spread through the
// K stream cost far more read bandwidth than the same bytes in bursts.
constexpr int kKeyStage = 24;                  // staged items (the second K buffer of the combined kernel)
constexpr int kKeyEntry = kChunk + kChunk / 8;  // u32 words per staged item (keys, block maxima)
static_assert(kKeyStage * kKeyEntry * 4 + kKeyStage * 8 <= kChunk * 128, "key stage exceeds a K buffer");
// Consumer-mode kernels hold only the single-token path: one K tile and a
// key stage of their own, small enough that three workgroups share a CU's
// 160 KB of LDS (K tile 32 KB, queries 4 or 8 KB, stage 11.6 or 16.2 KB).
// With 32 heads the path fits the 168 VGPRs of three waves per SIMD without
// spilling; with 64 heads it needs 210 and keeps two workgroups per CU.
constexpr int key_stage_single(int nh) { return nh == 64 ? 10 : 14; }

template <int MODE>
__device__ __forceinline__ void flush_keys(const KArgs& a, const uint32_t* stage, const int32_t* meta,
                                           int n) {
  __syncthreads();  // every wave's keys of the staged items are in LDS
  const int tid = threadIdx.x;
  for (int e = 0; e < n; ++e) {
    const int t = meta[2 * e], c = meta[2 * e + 1];
    __builtin_nontemporal_store(stage[e * kKeyEntry + tid],
                                a.keys + static_cast<int64_t>(t) * a.ncap + c * kChunk + tid);
    if (MODE == QLI_MODE_SOURCE && tid < kChunk / 8)
      __builtin_nontemporal_store(stage[e * kKeyEntry + kChunk + tid],
                                  a.bkeys + static_cast<int64_t>(t) * a.nbcap + c * (kChunk / 8) + tid);
  }
  __syncthreads();  // the stage is free again
}

// STAGE: items the key stage holds; SCALED_EPI: tokens whose multipliers
// allow it take the scaled epilogue (compute-bound batches).  The queries
// sit in LDS, shared by the four waves (in registers, the 32-head consumer
// path spills at three workgroups per CU and measured slower: mixed batch
// consumer score kernels 1.42 -> 1.52 ms).
template <int NH, int MODE, bool DBG, bool STREAM, int STAGE, bool SCALED_EPI>
__device__ void run_single(const KArgs& a, const ListView& L, Cursor cu, int hi, int8_t* ktile,
                           uint16_t* ksc0, uint32_t* stage, i32x4* qfr, uint32_t* qml, int wave,
                           int lane, const i32x16& seed, bool& bad) {
  static_assert(kScoreThreads == kChunk, "one staged key per thread and item");
  constexpr bool CONSUMER = MODE == QLI_MODE_CONSUMER;
  int32_t* meta = reinterpret_cast<int32_t*>(stage + STAGE * kKeyEntry);
  int ne = 0;  // staged items (the same in every wave)
  bool scaled = false;  // the current token takes the scaled epilogue
  // score item c of token t into staged entry ne, flushing a full stage;
  // cached (non-streaming) batches instead write each wave's 64 keys
  // straight to global memory: their K reads mostly hit the caches, so
  // bursts do not pay, and the block-wide flush (two barriers and a store
  // loop every STAGE items) costs more than the direct stores (mixed batch
  // consumer score kernels 1.42 -> 1.38 ms and 1.18 -> 1.16 ms)
  auto score_item = [&](int t, int c, int n) {
    if constexpr (!STREAM) {
      static_assert(MODE == QLI_MODE_CONSUMER, "only consumer batches read K through the caches");
      uint32_t* kp = a.keys + static_cast<int64_t>(t) * a.ncap + c * kChunk;
      score_subtile<NH, MODE, DBG>(a, QLds<NH>{qfr, qml}, ktile, ksc0, wave, t, c * kChunk + 64 * wave,
                                   n, lane, seed, kp, nullptr, SCALED_EPI && scaled);
      return;
    }
    if (ne == STAGE) {
      flush_keys<MODE>(a, stage, meta, ne);
      ne = 0;
    }
    if (wave == 0 && lane == 0) {
      meta[2 * ne] = t;
      meta[2 * ne + 1] = c;
    }
    uint32_t* kp = stage + ne * kKeyEntry;
    score_subtile<NH, MODE, DBG>(a, QLds<NH>{qfr, qml}, ktile, ksc0, wave, t, c * kChunk + 64 * wave,
                                 n, lane, seed, kp, kp + kChunk, SCALED_EPI && scaled);
    ++ne;
  };
  while (cu.valid) {
    Group gr = cu.grp;
    const int c0 = cu.c;
    const int c_end = min(gr.nch, c0 + (hi - cu.unit));
    const int t = gr.t0;
    // consumer: the plan's bound covers the work; the eligible slots are the
    // prepared count (slots past it are not read and score as not eligible)
    if (CONSUMER) gr.n0 = a.ncount[t];
    const int n = gr.n0;
    __syncthreads();  // the previous segment's last item is scored
    load_q_lds<NH, SCALED_EPI>(a, t, qfr, qml);
    Addr ad;
    i32x4 krA[8], krB[8];
    i32x4 scA, scB;
    stage_addr<CONSUMER, true>(a, gr, c0, true, wave, lane, ad);
    int vA = resolve<CONSUMER>(a, ad, bad);
    stage_addr<CONSUMER, true>(a, gr, c0 + 1, c0 + 1 < c_end, wave, lane, ad);
    stage_load<STREAM>(a, vA, lane, krA, scA);
    int vB = resolve<CONSUMER>(a, ad, bad);
    stage_addr<CONSUMER, true>(a, gr, c0 + 2, c0 + 2 < c_end, wave, lane, ad);
    stage_load<STREAM>(a, vB, lane, krB, scB);
    __syncthreads();  // queries in LDS
    if (SCALED_EPI) scaled = __builtin_amdgcn_readfirstlane(static_cast<int>(qml[NH / 2])) != 0;
    for (int c = c0; c < c_end; c += 2) {
      stage_store<true>(ktile, ksc0, krA, scA, vA, wave, lane);
      vA = resolve<CONSUMER>(a, ad, bad);
      stage_addr<CONSUMER, true>(a, gr, c + 3, c + 3 < c_end, wave, lane, ad);
      stage_load<STREAM>(a, vA, lane, krA, scA);
      __builtin_amdgcn_wave_barrier();
      score_item(t, c, n);
      // the second half of the step runs even past the segment's last item
      // (its rows are then placeholders and nothing is scored): every path
      // back to the loop head leaves the same loads in flight, so the
      // compiler's waits before the next staging keep the other item's rows
      // in flight (with an exit here the merged paths made that wait drain
      // every load)
      stage_store<true>(ktile, ksc0, krB, scB, vB, wave, lane);
      vB = resolve<CONSUMER>(a, ad, bad);
      stage_addr<CONSUMER, true>(a, gr, c + 4, c + 4 < c_end, wave, lane, ad);
      stage_load<STREAM>(a, vB, lane, krB, scB);
      __builtin_amdgcn_wave_barrier();
      if (c + 1 < c_end) score_item(t, c + 1, n);
    }
    // next token segment
    cu.c = c_end - 1;
    cu.unit += (c_end - 1 - c0);
    cu = next_item(L, cu, hi);
  }
  if (STREAM && ne > 0) flush_keys<MODE>(a, stage, meta, ne);
}


// Each workgroup takes its list, first item and unit range from the plan.
// STREAM: K rows of single-token groups are read with non-temporal loads
// (read once per call: decode).  Consumer batches whose requests hold
// several query tokens read them with ordinary loads instead: each token
// reads its own candidate rows, so the rows of a request are read again and
// again and the caches serve the repeats (mixed batch consumer score
// kernels 2.96 -> 1.77 ms and 2.42 -> 1.50 ms in one A/B measurement).
// Consumer tokens are always single groups, so consumer-mode kernels hold
// only that path (three workgroups per CU instead of two); the cached ones
// (compute-bound: each prefill token scores its own candidate rows) take
// the scaled epilogue.
__host__ __device__ constexpr int score_wgs_per_cu(int mode, int nh) {
  return mode == QLI_MODE_CONSUMER && nh == 32 ? 3 : 2;
}

// FUSED: the workgroup plans for itself (small plain/source batches).
template <int NH, int MODE, bool DBG, bool STREAM = true, bool FUSED = false>
__global__ __launch_bounds__(kScoreThreads, score_wgs_per_cu(MODE, NH)) void score_kernel(KArgs a) {
  constexpr bool SINGLE_ONLY = MODE == QLI_MODE_CONSUMER;
  static_assert(!(FUSED && SINGLE_ONLY), "consumer batches are planned by their preparation");
  constexpr int NTILE = SINGLE_ONLY ? 1 : 2;
  constexpr int STAGE = SINGLE_ONLY ? key_stage_single(NH) : kKeyStage;
  __shared__ __attribute__((aligned(16))) int8_t tile[NTILE][kChunk * 128];
  __shared__ __attribute__((aligned(16))) uint16_t ksc[NTILE][kChunk];
  __shared__ __attribute__((aligned(16))) i32x4 qfr[NH / 32 * 256];
  __shared__ uint32_t qml[NH / 2 + 1];
  // single-only kernels: a key stage of their own (the combined kernel
  // stages keys in its second K buffer)
  __shared__ __attribute__((aligned(16))) uint32_t kstage[SINGLE_ONLY ? STAGE * kKeyEntry + 2 * STAGE : 4];

  // small batches plan here (every workgroup the same plan, kept in LDS)
  constexpr int FT = FUSED ? kFusedTokens : 1;
  __shared__ Group fgroups[2 * FT];
  __shared__ int32_t fustart[2 * (FT + 1)];
  __shared__ int32_t ftokv[2 * FT];
  __shared__ WgStart fstart;

  const int wave = __builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x >> 6));
  const int lane = threadIdx.x & 63;
  const int entry = a.entry_base + start_entry(blockIdx.x, gridDim.x, a.nxcd);
  const Group* groups = a.groups;
  const int32_t* ustart = a.ustart;
  WgStart st;
  if constexpr (FUSED) {
    KArgs b = a;
    b.groups = fgroups;
    b.ustart = fustart;
    b.wgs = &fstart;
    b.hdr = nullptr;
    if (blockIdx.x != 0) b.tokv = ftokv;  // workgroup 0 writes the selection's counts
    b.plan_wg = entry;
    plan_role<kScoreThreads, kFusedTokens>(b, reinterpret_cast<uint32_t*>(tile[NTILE - 1]));
    __syncthreads();  // the plan's LDS scratch is the K buffer
    // wave-uniform values (LDS reads land in vector registers)
    const int32_t* sp = reinterpret_cast<const int32_t*>(&fstart);
    int32_t* dp = reinterpret_cast<int32_t*>(&st);
#pragma unroll
    for (int i = 0; i < static_cast<int>(sizeof(WgStart) / 4); ++i) dp[i] = __builtin_amdgcn_readfirstlane(sp[i]);
    groups = fgroups;
    ustart = fustart;
  } else {
    st = a.wgs[entry];
  }
  if (st.g < 0 || st.unit >= st.hi) return;
  const int l = st.list;
  const ListView L{groups + static_cast<int64_t>(l) * a.T, ustart + static_cast<int64_t>(l) * (a.T + 1), st.ng};
  Cursor cu;
  cu.g = st.g;
  cu.c = st.c;
  cu.unit = st.unit;
  cu.grp = st.grp;
  cu.valid = true;

  i32x16 seed;
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    // in vector registers for the whole kernel (the MFMAs start each
    // accumulator chain from them instead of copies of a scalar splat),
    // where the register budget of two workgroups per CU leaves room
    int x = kSeedBits;
    if constexpr (score_wgs_per_cu(MODE, NH) <= 2)
      asm volatile("v_mov_b32 %0, %1" : "=v"(x) : "i"(kSeedBits));
    seed[i] = x;
  }
  bool bad = false;
  if constexpr (SINGLE_ONLY) {
    run_single<NH, MODE, DBG, STREAM, STAGE, !STREAM>(a, L, cu, st.hi, tile[0], ksc[0], kstage, qfr, qml,
                                                      wave, lane, seed, bad);
  } else {
    uint32_t* stage = reinterpret_cast<uint32_t*>(tile[NTILE - 1]);
    if (l == 0)
      run_multi<NH, MODE, DBG>(a, L, cu, st.hi, tile, ksc, wave, lane, seed, bad);
    else
      run_single<NH, MODE, DBG, STREAM, STAGE, false>(a, L, cu, st.hi, tile[0], ksc[0], stage, qfr, qml,
                                                      wave, lane, seed, bad);
  }
  if (bad) raise_flag(a, QLI_DEV_BAD_PAGE);
}

// ---------------------------------------------------------------------------
// select
// ---------------------------------------------------------------------------
// Each thread keeps its share of a chunk of keys in registers: wave w of a
// chunk owns keys [w*KPW, (w+1)*KPW), read as 16-byte vectors so that one
// load instruction covers 1 KB (lane l, vector j: keys 256 j + 4 l .. +3).
// The chunk is 32 keys per thread (4096 for the 256-thread variant); longer
// rows are processed chunk by chunk.  LDS: histogram (2048 bins) and scan
// scratch.
constexpr uint32_t kPinKey = 0xFFFFFFFFu;  // the forced block sorts above every score
constexpr int kSelRank = 64;  // boundary bins this small are resolved by exact ranking (one wave)
constexpr int kSelSampleMin = 24576;  // rows with fewer scores go straight to the radix passes (16384-key rows: 15.3 -> 14.7 us)
// most keys gathered from a sampled bracket (an eighth of a chunk; the bracket
// holds about 4 % of the row)
__host__ __device__ constexpr int sel_cand(int bs) { return (bs == 256 ? 4096 : 32 * bs) / 8; }
__host__ __device__ constexpr int sel_lds_words(int bs) {
  return 2048 + 64 + 8 + 2 * sel_cand(bs) + 2 * kSelRank + QLI_MAX_TOPK;
}

__host__ __device__ constexpr int sel_chunk(int bs) { return bs == 256 ? 4096 : 32 * bs; }
// A shorter chunk for 512 threads (20 keys per thread) for rows of up to
// 10240 keys (prefill tokens up to 10240 compressed positions): fewer live
// registers, so that more workgroups share a CU (sel_min_waves).
constexpr int kSelShortChunk = 10240;

struct MinOp {
  __device__ __forceinline__ uint32_t operator()(uint32_t x, uint32_t y) const { return min(x, y); }
};
struct MaxOp {
  __device__ __forceinline__ uint32_t operator()(uint32_t x, uint32_t y) const { return max(x, y); }
};
struct AddOp {
  __device__ __forceinline__ uint32_t operator()(uint32_t x, uint32_t y) const { return x + y; }
};

// Threshold search among the keys that each(f) visits (f(key, index) for
// this thread's share), restricted to [lo, hi], of which the best krem are
// wanted: radix passes split the range 2048 ways until the boundary bin is
// taken whole, is one key value, or holds at most kSelRank keys, which are
// then ranked exactly by (key desc, index asc) with two ballots each.  On
// return keys > thr are taken plus the first `need` keys == thr.
template <int BS, class Each>
__device__ __forceinline__ void refine_threshold(Each each, uint32_t lo, uint32_t hi, uint32_t krem,
                                                 uint32_t& thr, uint32_t& need, uint32_t* hist,
                                                 uint32_t* sh, uint32_t* misc, uint32_t* rk,
                                                 uint32_t* ri) {
  constexpr int NW = BS / 64;
  constexpr int BPT = 2048 / BS;  // histogram bins per thread
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  int bits = hi == lo ? 0 : 32 - __clz(static_cast<int>(hi - lo));
#pragma unroll 1
  while (true) {
    const int sft = max(0, bits - 11);
#pragma unroll
    for (int j = 0; j < BPT; ++j) hist[tid * BPT + j] = 0;
    __syncthreads();
    each([&](uint32_t key, int) {
      if (key - lo <= hi - lo) atomicAdd(&hist[(key - lo) >> sft], 1u);
    });
    __syncthreads();
    uint32_t c = 0;
    uint32_t hv[BPT];
#pragma unroll
    for (int j = 0; j < BPT; ++j) {
      hv[j] = hist[tid * BPT + j];
      c += hv[j];
    }
    uint32_t total;
    const uint32_t excl = block_exclusive_scan<BS>(c, &total, sh);
    const uint32_t above_t = total - excl - c;  // keys in higher bins
    if (above_t < krem && above_t + c >= krem) {
      uint32_t cum = above_t;
      for (int j = BPT - 1; j >= 0; --j) {
        if (cum + hv[j] >= krem) {
          misc[0] = static_cast<uint32_t>(tid * BPT + j);
          misc[1] = cum;
          misc[2] = hv[j];
          break;
        }
        cum += hv[j];
      }
    }
    __syncthreads();
    const uint32_t b = misc[0], above = misc[1], hb = misc[2];
    krem -= above;
    const uint32_t blo = lo + (b << sft);
    if (hb == krem) {  // the whole boundary bin is taken
      thr = blo - 1;
      need = 0;
      return;
    }
    if (sft == 0) {
      thr = blo;
      need = krem;
      return;
    }
    lo = blo;
    hi = static_cast<uint32_t>(min(static_cast<uint64_t>(hi),
                                   static_cast<uint64_t>(blo) + (1ull << sft) - 1));
    bits = sft;
    if (tid == 0) misc[3] = 0;
    __syncthreads();  // misc is rewritten next
    if (hb <= static_cast<uint32_t>(kSelRank)) {
      each([&](uint32_t key, int idx) {
        if (key - lo <= hi - lo) {
          const uint32_t slot = atomicAdd(&misc[3], 1u);
          rk[slot] = key;
          ri[slot] = static_cast<uint32_t>(idx);
        }
      });
      __syncthreads();
      // lane q holds candidate q; wave w ranks candidates w, w + NW, ...
      const uint32_t m = hb;
      const bool has = static_cast<uint32_t>(lane) < m;
      const uint32_t kq = has ? rk[lane] : 0u, iq = has ? ri[lane] : 0u;
      for (uint32_t i = wave; i < m; i += NW) {
        const uint32_t key = rk[i], idx = ri[i];
        const uint32_t gt = static_cast<uint32_t>(__popcll(__ballot(has && kq > key)));
        const uint32_t eqb = static_cast<uint32_t>(__popcll(__ballot(has && kq == key && iq < idx)));
        const uint32_t eqall = static_cast<uint32_t>(__popcll(__ballot(has && kq == key)));
        if (lane == 0 && gt + eqb == krem - 1) {
          misc[0] = key;
          misc[1] = eqb + 1;
          misc[2] = eqall;
        }
      }
      __syncthreads();
      thr = misc[0];
      need = misc[1];
      // every key equal to the threshold is taken: the same set is "keys >
      // thr - 1" (keys are non-zero), with no tie to resolve
      if (misc[2] == need) {
        thr -= 1;
        need = 0;
      }
      return;
    }
  }
}

// Select the best min(k, #nonzero) of keys[0..n) by (key desc, index asc)
// and write map(index) for them in ascending index order to out[0..k),
// -1 after.  pin (or -1) is forced to the top.  The row holds cap >= n
// keys (a multiple of 64), so whole 16-byte vectors below cap may be read.
//
// Radix select over the range the keys actually occupy: the first digit is
// taken from (key - min) with a shift that leaves at most 2048 bins, and
// each further pass splits the chosen bin 2048 ways.  Scores of one query
// share a narrow band of key values, so fixed top-bit digits would pile
// them into a handful of bins.  A pass ends the search as soon as every key
// of the boundary bin is needed.
// MULTI = false: the caller guarantees n <= CHUNK (one chunk, loaded once).
template <int BS, bool MULTI, int CH, class Map>
__device__ __forceinline__ void select_topk(const uint32_t* keys, int n, int cap, int k, int pin,
                                            int32_t* out, Map map, uint32_t* lds) {
  constexpr int CHUNK = MULTI ? 16 * BS : CH;  // fewer live keys when reloading
  constexpr int NW = BS / 64;
  constexpr int KPW = CHUNK / NW;        // keys per wave per chunk
  constexpr int VPT = CHUNK / (4 * BS);  // 16-byte vectors per thread per chunk
  uint32_t* hist = lds;
  uint32_t* sh = lds + 2048;
  uint32_t* misc = lds + 2048 + 64;
  uint32_t* ck = lds + 2048 + 64 + 8;   // bracket keys, then their indices
  uint32_t* ci = ck + sel_cand(BS);
  uint32_t* rk = ci + sel_cand(BS);     // boundary-bin keys for exact ranking, then indices
  uint32_t* ri = rk + kSelRank;
  int32_t* ol = reinterpret_cast<int32_t*>(ri + kSelRank);  // winners' key indices, in order (<= k)
  auto refine = [&](auto each, uint32_t lo, uint32_t hi, uint32_t kr_, uint32_t& t_, uint32_t& n_) {
    refine_threshold<BS>(each, lo, hi, kr_, t_, n_, hist, sh, misc, rk, ri);
  };
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int nch = MULTI ? (n + CHUNK - 1) / CHUNK : 1;
  // one chunk: the row is spread evenly over the waves in whole vectors
  // (kpw keys per wave), so that a short row keeps every wave busy; the
  // vectors of a wave past its nvec are all zero and their work is skipped
  const int kpw = MULTI ? KPW : min(KPW, ((n + NW - 1) / NW + 255) & ~255);
  const int nvec = MULTI ? VPT : min(min(VPT, max(0, (n - wave * kpw + 255) >> 8)), kpw >> 8);
  uint32_t kr[4 * VPT];
  auto index_of = [&](int ch, int j, int e) {
    return ch * CHUNK + wave * kpw + 256 * j + 4 * lane + e;
  };
  const bool pinned = pin >= 0 && pin < n;
  auto load = [&](int ch) {  // every load is issued before the first use
    i32x4 x[VPT];
#pragma unroll
    for (int j = 0; j < VPT; ++j)
      x[j] = *reinterpret_cast<const i32x4*>(keys + min(index_of(ch, j, 0), cap - 4));
    const int vb = ch * CHUNK + wave * kpw;  // first index of this wave's share
#pragma unroll
    for (int j = 0; j < VPT; ++j) {
      if (j < nvec && vb + 256 * (j + 1) <= n) {  // the whole vector lies in the row
#pragma unroll
        for (int e = 0; e < 4; ++e) kr[4 * j + e] = static_cast<uint32_t>(x[j][e]);
      } else {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          // vectors past nvec may reach into the next wave's keys: zero
          const bool own = j < nvec && index_of(ch, j, e) < n;
          kr[4 * j + e] = own ? static_cast<uint32_t>(x[j][e]) : 0u;
        }
      }
    }
    // the pin, if this wave holds it: one lane's element of one vector
    const int po = pin - vb;
    if (pinned && po >= 0 && po < 256 * nvec) {
#pragma unroll
      for (int j = 0; j < VPT; ++j)
        if (j == (po >> 8)) {
#pragma unroll
          for (int e = 0; e < 4; ++e)
            if (lane == ((po >> 2) & 63) && e == (po & 3)) kr[4 * j + e] = kPinKey;
        }
    }
  };

  // the keys of this thread, as (key, index) pairs (reloading chunks)
  auto each_reg = [&](auto f) {
    for (int ch = 0; ch < nch; ++ch) {
      if (MULTI && nch > 1) load(ch);
#pragma unroll
      for (int j = 0; j < VPT; ++j) {
        if (j >= nvec) continue;
#pragma unroll
        for (int e = 0; e < 4; ++e) f(kr[4 * j + e], index_of(ch, j, e));
      }
    }
  };
  // Bracket [blo, bhi] around the key of rank krem (from the top) from a
  // sample: this thread's samples (each_sample(f) calls f(key)) go into
  // 2048 bins over [lo, hi] (zero keys and the pin skipped); the bins
  // holding the sample ranks rexp -+ (3 sqrt(rexp) + 4) bound it, where
  // rexp = krem * samples / row_keys is the threshold's expected rank among
  // them.  With open ends a bracket reaching the highest (lowest) sample
  // also takes every key above (below) it.  All threads call it.
  auto bracket = [&](auto each_sample, uint32_t lo, uint32_t hi, uint32_t krem, float row_keys, bool open,
                     uint32_t& blo, uint32_t& bhi) {
    const int bits0 = hi == lo ? 0 : 32 - __clz(static_cast<int>(hi - lo));
    const int sft0 = max(0, bits0 - 11);
    constexpr int BPT = 2048 / BS;
#pragma unroll
    for (int j = 0; j < BPT; ++j) hist[tid * BPT + j] = 0;
    if (tid == 0) misc[4] = 0;
    __syncthreads();
    uint32_t ns = 0;
    each_sample([&](uint32_t key) {
      if (key != 0 && key != kPinKey) {
        atomicAdd(&hist[(key - lo) >> sft0], 1u);
        ++ns;
      }
    });
    ns = wave_allreduce(ns, AddOp{});
    if (lane == 0) atomicAdd(&misc[4], ns);
    __syncthreads();
    const uint32_t nsamp = misc[4];
    const float rexp = static_cast<float>(krem) * static_cast<float>(nsamp) / row_keys;
    const float dev = 3.0f * sqrtf(rexp) + 4.0f;
    const uint32_t r_hi = static_cast<uint32_t>(max(0.0f, rexp - dev));  // keys above the bracket
    const uint32_t r_lo = static_cast<uint32_t>(min(static_cast<float>(nsamp), rexp + dev));
    uint32_t c = 0;
    uint32_t hv[BPT];
#pragma unroll
    for (int j = 0; j < BPT; ++j) {
      hv[j] = hist[tid * BPT + j];
      c += hv[j];
    }
    uint32_t total;
    const uint32_t excl = block_exclusive_scan<BS>(c, &total, sh);
    const uint32_t above_t = total - excl - c;
    // bin holding sample rank r (counted from the top, 0-based) -> misc[slot]
    auto find = [&](uint32_t r, int slot) {
      if (above_t <= r && r < above_t + c) {
        uint32_t cum = above_t;
        for (int j = BPT - 1; j >= 0; --j) {
          if (cum + hv[j] > r) {
            misc[slot] = static_cast<uint32_t>(tid * BPT + j);
            break;
          }
          cum += hv[j];
        }
      }
    };
    if (tid == 0) {
      misc[5] = 2047;  // r_hi above every sample: bracket reaches the top
      misc[6] = 0;     // r_lo below every sample: bracket reaches lo
    }
    __syncthreads();
    if (r_hi < total) find(r_hi, 5);
    if (r_lo < total) find(r_lo, 6);
    __syncthreads();
    const uint32_t b_top = r_hi < total ? misc[5] : 2047u;
    const uint32_t b_bot = r_lo < total ? misc[6] : 0u;
    blo = lo + (b_bot << sft0);
    bhi = static_cast<uint32_t>(
        min(static_cast<uint64_t>(hi), static_cast<uint64_t>(lo) + ((static_cast<uint64_t>(b_top) + 1) << sft0) - 1));
    if (open) {
      if (r_hi == 0) bhi = kPinKey - 1;
      if (r_lo + 1 >= total) blo = 1;
    }
  };

  // threshold: keys > thr are taken, then the first `need` keys == thr
  uint32_t thr = 0, need = 0;
  if constexpr (!MULTI) {
    // range and count of the scores (keys other than 0 and the pin): the
    // minimum is taken over key - 1, which sends the zero keys to the top;
    // with a pin the maximum is taken over key + 1, which sends it to 0
    uint32_t mn1 = 0xFFFFFFFFu, mx1 = 0, cnt = 0;
    auto range = [&](const bool P) {
      const uint32_t o = P ? 1u : 0u;
      load(0);
#pragma unroll
      for (int j = 0; j < VPT; ++j) {
        if (j >= nvec) continue;
        const uint32_t v0 = kr[4 * j], v1 = kr[4 * j + 1], v2 = kr[4 * j + 2], v3 = kr[4 * j + 3];
        mx1 = max(max(mx1, v0 + o), v1 + o);
        mx1 = max(max(mx1, v2 + o), v3 + o);
        mn1 = min(min(mn1, v0 - 1u), v1 - 1u);
        mn1 = min(min(mn1, v2 - 1u), v3 - 1u);
        cnt += min(v0, 1u) + min(v1, 1u);
        cnt += min(v2, 1u) + min(v3, 1u);
      }
    };
    if (pinned) range(true);
    else range(false);
    mn1 = wave_allreduce(mn1, MinOp{});
    mx1 = wave_allreduce(mx1, MaxOp{});
    cnt = wave_allreduce(cnt, AddOp{});
    if (lane == 0) {
      sh[wave] = mn1;
      sh[16 + wave] = mx1;
      sh[32 + wave] = cnt;
    }
    __syncthreads();
    mn1 = sh[0];
    mx1 = sh[16];
    cnt = sh[32];
#pragma unroll
    for (int w = 1; w < NW; ++w) {
      mn1 = min(mn1, sh[w]);
      mx1 = max(mx1, sh[16 + w]);
      cnt += sh[32 + w];
    }
    __syncthreads();
    cnt -= pinned ? 1u : 0u;  // the pin was counted as a key
    const uint32_t mn = cnt == 0 ? 0xFFFFFFFFu : mn1 + 1u;
    const uint32_t mx = cnt == 0 ? 0u : mx1 - (pinned ? 1u : 0u);

    if (cnt + (pinned ? 1u : 0u) > static_cast<uint32_t>(k)) {
      uint32_t krem = static_cast<uint32_t>(k) - (pinned ? 1u : 0u);
      if (krem == 0) {
        thr = kPinKey - 1;
      } else {
        bool done = false;
        if (cnt >= static_cast<uint32_t>(kSelSampleMin)) {
          // Two keys per thread bound a bracket; one counting sweep checks
          // that the threshold lies inside; its keys (about 4 % of the row)
          // are gathered and searched alone.
          uint32_t blo, bhi;
          bracket([&](auto f) {
#pragma unroll
                    for (int r = 0; r < 4 * VPT; r += 2 * VPT) f(kr[r]);
                  },
                  mn, mx, krem, static_cast<float>(cnt), false, blo, bhi);
          // keys above the bracket and inside it, packed above << 16 | inside
          // (a chunk holds at most 32768 keys); the prefix places the gather
          // (the pin, if any, lies above bhi and is not counted)
          uint32_t above = 0, inb = 0;
#pragma unroll
          for (int r = 0; r < 4 * VPT; ++r) {
            const uint32_t key = kr[r];
            above += key > bhi ? 1u : 0u;
            inb += key - blo <= bhi - blo ? 1u : 0u;
          }
          uint32_t tot2;
          uint32_t at = block_exclusive_scan<BS>((above << 16) | inb, &tot2, sh) & 0xFFFFu;
          const uint32_t n_above = (tot2 >> 16) - (pinned ? 1u : 0u), n_in = tot2 & 0xFFFFu;
          if (n_above < krem && n_above + n_in >= krem && n_in <= static_cast<uint32_t>(sel_cand(BS))) {
            // gather the bracket's keys and search them alone
#pragma unroll
            for (int j = 0; j < VPT; ++j)
#pragma unroll
              for (int e = 0; e < 4; ++e) {
                const uint32_t key = kr[4 * j + e];
                if (key - blo <= bhi - blo) {
                  ck[at] = key;
                  ci[at] = static_cast<uint32_t>(index_of(0, j, e));
                  ++at;
                }
              }
            __syncthreads();
            auto each_cand = [&](auto f) {
              for (uint32_t i = tid; i < n_in; i += BS) f(ck[i], static_cast<int>(ci[i]));
            };
            krem -= n_above;
            refine(each_cand, blo, bhi, krem, thr, need);
            done = true;
          }
          __syncthreads();  // sh, misc and the candidate lists are reused
        }
        if (!done) refine(each_reg, mn, mx, krem, thr, need);
      }
    }
  } else {
    // Chunked rows (every radix pass over them would read them again):
    // (1) a sample of the row, one key of one 16-byte vector per thread in
    // each of up to SPT chunks spread over the row (in the bracket gather's
    // LDS), bounds a bracket; (2) one sweep over the row counts the keys
    // above it (and the row's range and count), gathers the keys inside it
    // and (3) the search runs on those alone when the threshold lies inside
    // and they fit, else on the whole row.  With the compaction the row is
    // read about 2.1 times instead of once per radix pass and twice besides.
    constexpr int SPT = 2 * sel_cand(BS) / BS;
    const int sstride = (nch + SPT - 1) / SPT;
    const int nsl = (nch + sstride - 1) / sstride;
    uint32_t* samp = ck;
    i32x4 xs[SPT];
#pragma unroll
    for (int s = 0; s < SPT; ++s)  // every load issued before the first use
      xs[s] = *reinterpret_cast<const i32x4*>(keys + min(index_of(min(s, nsl - 1) * sstride, 0, 0), cap - 4));
    uint32_t smn = 0xFFFFFFFFu, smx = 0, sv = 0, snz = 0;
#pragma unroll
    for (int s = 0; s < SPT; ++s) {
      if (s >= nsl) continue;
      const int idx = index_of(s * sstride, 0, 0) + (s & 3);
      uint32_t key = static_cast<uint32_t>(xs[s][s & 3]);
      const bool valid = idx < n && idx != pin;
      key = valid ? key : 0u;
      sv += valid ? 1u : 0u;
      if (key != 0) {
        smn = min(smn, key);
        smx = max(smx, key);
        ++snz;
      }
      samp[s * BS + tid] = key;
    }
    smn = wave_allreduce(smn, MinOp{});
    smx = wave_allreduce(smx, MaxOp{});
    sv = wave_allreduce(sv, AddOp{});
    snz = wave_allreduce(snz, AddOp{});
    if (lane == 0) {
      sh[wave] = smn;
      sh[16 + wave] = smx;
      sh[32 + wave] = sv;
      sh[48 + wave] = snz;
    }
    __syncthreads();
    smn = sh[0];
    smx = sh[16];
    sv = sh[32];
    snz = sh[48];
#pragma unroll
    for (int w = 1; w < NW; ++w) {
      smn = min(smn, sh[w]);
      smx = max(smx, sh[16 + w]);
      sv += sh[32 + w];
      snz += sh[48 + w];
    }
    __syncthreads();
    const uint32_t krem0 = static_cast<uint32_t>(k) - (pinned ? 1u : 0u);
    uint32_t blo = 1, bhi = kPinKey - 1;
    if (snz > 0 && krem0 > 0)
      bracket([&](auto f) {
                for (int s = 0; s < nsl; ++s) f(samp[s * BS + tid]);
              },
              smn, smx, krem0, static_cast<float>(snz) * static_cast<float>(n) / static_cast<float>(sv), true,
              blo, bhi);
    // (2) the sweep
    if (tid == 0) misc[7] = 0;
    __syncthreads();  // the samples are consumed: the gather may overwrite them
    const uint32_t o = pinned ? 1u : 0u;
    uint32_t mn1 = 0xFFFFFFFFu, mx1 = 0, cnt = 0, above = 0;
    for (int ch = 0; ch < nch; ++ch) {
      load(ch);
#pragma unroll
      for (int j = 0; j < VPT; ++j)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const uint32_t key = kr[4 * j + e];
          mx1 = max(mx1, key + o);
          mn1 = min(mn1, key - 1u);
          cnt += min(key, 1u);
          above += key > bhi ? 1u : 0u;
          const bool in = key - blo <= bhi - blo;
          const uint64_t mk = __ballot(in);
          if (mk != 0) {  // one LDS counter step per wave
            uint32_t base = 0;
            if (lane == 0) base = atomicAdd(&misc[7], static_cast<uint32_t>(__popcll(mk)));
            base = static_cast<uint32_t>(__shfl(static_cast<int>(base), 0));
            const uint32_t slot = base + static_cast<uint32_t>(__popcll(mk & ((1ull << lane) - 1ull)));
            if (in && slot < static_cast<uint32_t>(sel_cand(BS))) {
              ck[slot] = key;
              ci[slot] = static_cast<uint32_t>(index_of(ch, j, e));
            }
          }
        }
    }
    mn1 = wave_allreduce(mn1, MinOp{});
    mx1 = wave_allreduce(mx1, MaxOp{});
    cnt = wave_allreduce(cnt, AddOp{});
    above = wave_allreduce(above, AddOp{});
    if (lane == 0) {
      sh[wave] = mn1;
      sh[16 + wave] = mx1;
      sh[32 + wave] = cnt;
      sh[48 + wave] = above;
    }
    __syncthreads();
    mn1 = sh[0];
    mx1 = sh[16];
    cnt = sh[32];
    above = sh[48];
#pragma unroll
    for (int w = 1; w < NW; ++w) {
      mn1 = min(mn1, sh[w]);
      mx1 = max(mx1, sh[16 + w]);
      cnt += sh[32 + w];
      above += sh[48 + w];
    }
    const uint32_t n_in = misc[7];
    __syncthreads();
    cnt -= pinned ? 1u : 0u;  // the pin was counted as a key and as above
    above -= pinned ? 1u : 0u;
    const uint32_t mn = cnt == 0 ? 0xFFFFFFFFu : mn1 + 1u;
    const uint32_t mx = cnt == 0 ? 0u : mx1 - (pinned ? 1u : 0u);
    // (3) the search
    if (cnt + (pinned ? 1u : 0u) > static_cast<uint32_t>(k)) {
      if (krem0 == 0) {
        thr = kPinKey - 1;
      } else if (above < krem0 && above + n_in >= krem0 && n_in <= static_cast<uint32_t>(sel_cand(BS))) {
        auto each_cand = [&](auto f) {
          for (uint32_t i = tid; i < n_in; i += BS) f(ck[i], static_cast<int>(ci[i]));
        };
        refine(each_cand, blo, bhi, krem0 - above, thr, need);
      } else {
        refine(each_reg, mn, mx, krem0, thr, need);
      }
    }
  }

  // ordered compaction over a bitmask of the winners (keys > thr, then the
  // first `need` keys == thr in index order): lane l's four keys of vector
  // j fill one nibble of word (wave * kpw + 256 j) / 32 + l / 8 of the
  // chunk, OR-ed over the 8 lanes of the word on DPP; each thread then takes
  // one word, a block prefix sum of the words' counts places it, and it
  // places the winners (see `sparse`) in LDS, from where they are written
  // out in order.  Words holding no index below n are never read (every
  // word with one is written).
  constexpr int NWD = CHUNK / 32;
  static_assert(NWD <= BS && 2 * NWD <= 2048, "two bitmasks of a chunk in the histogram's place");
  uint32_t* gtw = hist;
  uint32_t* eqw = hist + NWD;
  uint32_t run_gt = 0, run_eq = 0;
  // few winners per word (at most one in eight keys): each word's thread
  // writes them; otherwise every lane writes its own
  const bool sparse = 8 * static_cast<int64_t>(k) <= n;
  for (int ch = 0; ch < nch; ++ch) {
    if (MULTI && nch > 1) load(ch);
#pragma unroll
    for (int j = 0; j < VPT; ++j) {
      if (j >= nvec) continue;
      uint32_t g = 0, q = 0;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const uint32_t key = kr[4 * j + e];
        g |= (key > thr ? 1u : 0u) << e;
        q |= (key == thr ? 1u : 0u) << e;
      }
      const int sft = 4 * (lane & 7);
      g <<= sft;
      g |= dpp_all<0xB1>(g);   // quad_perm [1, 0, 3, 2]
      g |= dpp_all<0x4E>(g);   // quad_perm [2, 3, 0, 1]
      g |= dpp_all<0x141>(g);  // row_half_mirror
      const int w = ((wave * kpw + 256 * j) >> 5) + (lane >> 3);
      if ((lane & 7) == 0) gtw[w] = g;
      if (need != 0) {
        q <<= sft;
        q |= dpp_all<0xB1>(q);
        q |= dpp_all<0x4E>(q);
        q |= dpp_all<0x141>(q);
        if ((lane & 7) == 0) eqw[w] = q;
      }
    }
    __syncthreads();
    const int nwd = (min(CHUNK, n - ch * CHUNK) + 31) >> 5;
    uint32_t gw = 0, qw = 0;
    if (tid < nwd) {
      gw = gtw[tid];
      qw = need != 0 ? eqw[tid] : 0u;
    }
    uint32_t tot;
    const uint32_t ex = block_exclusive_scan<BS>((static_cast<uint32_t>(__popc(gw)) << 16) |
                                                     static_cast<uint32_t>(__popc(qw)),
                                                 &tot, sh);  // ends with a barrier: the words may be rewritten
    if (tid < nwd) {
      const uint32_t eq_before = run_eq + (ex & 0xFFFFu);
      uint32_t m = gw;
      if (qw != 0 && eq_before < need) {
        uint32_t take = qw;  // its lowest need - eq_before ties
        const uint32_t room = need - eq_before;
        while (static_cast<uint32_t>(__popc(take)) > room) take &= ~(0x80000000u >> __clz(take));
        m |= take;
      }
      uint32_t at = run_gt + (ex >> 16) + min(need, eq_before);
      if (sparse) {
        const int base = ch * CHUNK + 32 * tid;
        while (m != 0) {
          const int b = __ffs(m) - 1;
          if (at < static_cast<uint32_t>(k)) ol[at] = base + b;
          ++at;
          m &= m - 1;
        }
      } else {
        gtw[tid] = m;  // the word's winners and its first output slot
        eqw[tid] = at;
      }
    }
    if (!sparse) {
      // each lane writes its own winners: slot = the word's first slot +
      // the winners below the lane's nibble + those before it in the nibble
      __syncthreads();
#pragma unroll
      for (int j = 0; j < VPT; ++j) {
        if (j >= nvec) continue;
        const int w = ((wave * kpw + 256 * j) >> 5) + (lane >> 3);
        const uint32_t m = gtw[w];
        const int sft = 4 * (lane & 7);
        const uint32_t nib = (m >> sft) & 0xFu;
        if (nib != 0) {
          uint32_t at = eqw[w] + static_cast<uint32_t>(__popc(m & ((1u << sft) - 1u)));
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            if ((nib >> e) & 1u) {
              if (at < static_cast<uint32_t>(k)) ol[at] = index_of(ch, j, e);
              ++at;
            }
          }
        }
      }
      __syncthreads();  // the words are rewritten for the next chunk
    }
    run_gt += tot >> 16;
    run_eq += tot & 0xFFFFu;
  }
  __syncthreads();
  const int count = static_cast<int>(run_gt + min(need, run_eq));
  for (int i = tid; i < k; i += BS) out[i] = i < count ? map(ol[i]) : -1;
}

struct MapIdentity {
  __device__ __forceinline__ int32_t operator()(int i) const { return i; }
};

// Candidate slot i -> position: slot i is position i & 7 of incoming block
// slots[i >> 3].
struct MapSlots {
  const int32_t* slots;
  __device__ __forceinline__ int32_t operator()(int i) const { return slots[i >> 3] * 8 + (i & 7); }
};

// Minimum waves per SIMD asked of the compiler: the 512-thread variants
// (rows of 4097..16384 keys, e.g. every prefill token) would take up to 123
// VGPRs and fit two workgroups per CU.  With 32 keys per thread, 80 VGPRs
// (three workgroups per CU) spill a few registers, which costs less than
// the extra workgroup gains (prefill chunk select 141 -> 110 us), while 64
// VGPRs spill too much (127 us).  With 20 keys per thread, 80 VGPRs spill
// nothing (110 -> 100 us) and 64 VGPRs (four workgroups per CU, 134 KB of
// LDS) spill 12 and are faster still (99 -> 88 us).  The 1024-thread
// variants run one workgroup per CU either way.
__host__ __device__ constexpr int sel_min_waves(int bs, int ch) {
  return bs == 512 ? (ch == kSelShortChunk ? 8 : 6) : 1;
}

template <int BS, bool MULTI, int CH = sel_chunk(BS)>
__global__ __launch_bounds__(BS, sel_min_waves(BS, CH)) void select_kernel(KArgs a) {
  __shared__ uint32_t sel_lds[sel_lds_words(BS)];
  const int t = blockIdx.x;
  // plain/source: every position below V and every block below ceil(V/8) is
  // eligible unless a page was out of contract, so when they all fit the
  // selection is all of them, in order (no keys needed)
  auto all_of = [](int32_t* out, int n, int k) {
    for (int i = threadIdx.x; i < k; i += BS) out[i] = i < n ? i : -1;
  };
  // the row's length decides whether this launch takes it (wave-uniform)
  auto mine = [&](int n) { return n >= a.sel_lo && n <= a.sel_hi; };
  if (blockIdx.y == 0) {
    int32_t* out = a.topk_out + static_cast<int64_t>(t) * a.topk;
    const uint32_t* keys = a.keys + static_cast<int64_t>(t) * a.ncap;
    const int cap = static_cast<int>(a.ncap);
    if (a.mode == QLI_MODE_CONSUMER) {
      const int n = a.ncount[t];
      if (!mine(n)) return;
      select_topk<BS, MULTI, CH>(keys, n, cap, a.topk, -1, out,
                      MapSlots{a.slots + static_cast<int64_t>(t) * a.cb_in}, sel_lds);
    } else {
      const int2 tv = reinterpret_cast<const int2*>(a.tokv)[t];  // count and bad-page stamp, one load
      const int V = tv.x;
      if (!mine(V)) return;
      if (tv.y != static_cast<int32_t>(a.epoch) && V <= a.topk) all_of(out, V, a.topk);
      else select_topk<BS, MULTI, CH>(keys, V, cap, a.topk, -1, out, MapIdentity{}, sel_lds);
    }
  } else {
    const int2 tv = reinterpret_cast<const int2*>(a.tokv)[t];
    const int nb = (tv.x + 7) / 8;
    if (!mine(nb)) return;
    int32_t* out = a.cand_out + static_cast<int64_t>(t) * a.cb;
    if (tv.y != static_cast<int32_t>(a.epoch) && nb <= a.cb) all_of(out, nb, a.cb);
    else select_topk<BS, MULTI, CH>(a.bkeys + static_cast<int64_t>(t) * a.nbcap, nb, static_cast<int>(a.nbcap), a.cb,
                           nb - 1, out, MapIdentity{}, sel_lds);
  }
}

}  // namespace

// ---------------------------------------------------------------------------
// optional per-kernel timing (events recorded around each launch)
// ---------------------------------------------------------------------------
namespace {
struct Timed {
  int kernel;
  hipEvent_t start, stop;
};
std::mutex g_timing_mu;
bool g_timing_on = false;
std::vector<Timed> g_pending;
double g_ms[QLI_NUM_KERNELS];
int64_t g_count[QLI_NUM_KERNELS];

int g_cu_count[64];
// per-launch stamps of the bad-page flags (distinct for 2^32 consecutive slices)
std::atomic<uint32_t> g_epoch{0x9E3779B9u};
int g_xcd_count[64];

// Scratch of the entry point that allocates nothing.  In host code the name
// only stands for the array; its device address (one copy per GPU) comes
// from hipGetSymbolAddress and is the only form ever passed to a kernel or
// a copy.
static __device__ __align__(256) unsigned char scratch[QLI_STATIC_SCRATCH_BYTES];
std::mutex g_scratch_mu;
void* g_scratch_ptr[64];
}  // namespace

int static_scratch(void** ptr) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return QLI_ERR_HIP;
  std::lock_guard<std::mutex> g(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;  // looked up with device `dev` current
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return QLI_ERR_HIP;
    g_scratch_ptr[dev] = p;
  }
  *ptr = g_scratch_ptr[dev];
  return QLI_OK;
}

Stamp::Stamp(int k, void* s, bool enabled) : kernel_(k), st_(s) {
  if (!enabled || !g_timing_on) return;
  hipEvent_t a = nullptr, b = nullptr;
  if (hipEventCreate(&a) != hipSuccess) return;
  if (hipEventCreate(&b) != hipSuccess) {
    (void)hipEventDestroy(a);
    return;
  }
  start_ = a;
  stop_ = b;
  (void)hipEventRecord(a, static_cast<hipStream_t>(st_));
}

Stamp::~Stamp() {
  if (!start_ || !stop_) return;
  (void)hipEventRecord(static_cast<hipEvent_t>(stop_), static_cast<hipStream_t>(st_));
  std::lock_guard<std::mutex> g(g_timing_mu);
  g_pending.push_back({kernel_, static_cast<hipEvent_t>(start_), static_cast<hipEvent_t>(stop_)});
}

int cu_count() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  if (!g_cu_count[dev]) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
      n = 256;
    g_cu_count[dev] = n;
  }
  return g_cu_count[dev];
}

int xcd_count() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 1;
  if (!g_xcd_count[dev]) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeNumberOfXccs, dev) != hipSuccess || n <= 0) n = 1;
    g_xcd_count[dev] = n;
  }
  return g_xcd_count[dev];
}

int timing_enable(int on) {
  std::lock_guard<std::mutex> g(g_timing_mu);
  g_timing_on = on != 0;
  return QLI_OK;
}

int timing_read(double* ms, int64_t* count, int reset) {
  std::lock_guard<std::mutex> g(g_timing_mu);
  int rc = QLI_OK;
  for (const Timed& t : g_pending) {
    float e = 0.f;
    if (hipEventSynchronize(t.stop) != hipSuccess || hipEventElapsedTime(&e, t.start, t.stop) != hipSuccess)
      rc = QLI_ERR_HIP;
    g_ms[t.kernel] += e;
    g_count[t.kernel] += 1;
    (void)hipEventDestroy(t.start);
    (void)hipEventDestroy(t.stop);
  }
  g_pending.clear();
  for (int k = 0; k < QLI_NUM_KERNELS; ++k) {
    if (ms) ms[k] = g_ms[k];
    if (count) count[k] = g_count[k];
    if (reset) {
      g_ms[k] = 0.0;
      g_count[k] = 0;
    }
  }
  return rc;
}

template <int NH, int MODE>
void launch_score_dbg(bool dbg, unsigned grid, hipStream_t st, const KArgs& a) {
  if constexpr (MODE != QLI_MODE_CONSUMER) {
    if (a.fused) {
      if (dbg) score_kernel<NH, MODE, true, true, true><<<grid, kScoreThreads, 0, st>>>(a);
      else score_kernel<NH, MODE, false, true, true><<<grid, kScoreThreads, 0, st>>>(a);
      return;
    }
  }
  if (dbg) score_kernel<NH, MODE, true><<<grid, kScoreThreads, 0, st>>>(a);
  else score_kernel<NH, MODE, false><<<grid, kScoreThreads, 0, st>>>(a);
}

// consumer batches with more query tokens than requests: cached K loads
template <int NH>
void launch_score_cached(bool dbg, unsigned grid, hipStream_t st, const KArgs& a) {
  if (dbg) score_kernel<NH, QLI_MODE_CONSUMER, true, false><<<grid, kScoreThreads, 0, st>>>(a);
  else score_kernel<NH, QLI_MODE_CONSUMER, false, false><<<grid, kScoreThreads, 0, st>>>(a);
}

template <int NH>
void launch_score_mode(int mode, bool dbg, bool cached, unsigned grid, hipStream_t st, const KArgs& a) {
  if (mode == QLI_MODE_PLAIN) launch_score_dbg<NH, QLI_MODE_PLAIN>(dbg, grid, st, a);
  else if (mode == QLI_MODE_SOURCE) launch_score_dbg<NH, QLI_MODE_SOURCE>(dbg, grid, st, a);
  else if (cached) launch_score_cached<NH>(dbg, grid, st, a);
  else launch_score_dbg<NH, QLI_MODE_CONSUMER>(dbg, grid, st, a);
}

template <int NH>
void launch_score_multi_nh(int mode, bool dbg, unsigned grid, hipStream_t st, const KArgs& a) {
  static_assert(NH == 32, "the separate multi kernel serves 32 heads");
  if (mode == QLI_MODE_PLAIN) {
    if (dbg) score_multi_kernel<NH, QLI_MODE_PLAIN, true><<<grid, kScoreThreads, 0, st>>>(a);
    else score_multi_kernel<NH, QLI_MODE_PLAIN, false><<<grid, kScoreThreads, 0, st>>>(a);
  } else {
    if (dbg) score_multi_kernel<NH, QLI_MODE_SOURCE, true><<<grid, kScoreThreads, 0, st>>>(a);
    else score_multi_kernel<NH, QLI_MODE_SOURCE, false><<<grid, kScoreThreads, 0, st>>>(a);
  }
}

void launch_score_multi(int heads, int mode, bool dbg, unsigned grid, hipStream_t st, const KArgs& a) {
  (void)heads;  // 32 (see launch())
  launch_score_multi_nh<32>(mode, dbg, grid, st, a);
}

void launch_score(int heads, int mode, bool dbg, bool cached, unsigned grid, hipStream_t st, const KArgs& a) {
  if (heads == 64) launch_score_mode<64>(mode, dbg, cached, grid, st, a);
  else launch_score_mode<32>(mode, dbg, cached, grid, st, a);
}

void launch_slice(const qli_params* p, const WsLayout& w, KArgs a, bool cached, hipStream_t st,
                  bool timed);

int launch(const qli_params* p, const WsLayout& w, void* stream, bool timed) {
  hipStream_t st = static_cast<hipStream_t>(stream);
  (void)hipGetLastError();  // an earlier failure elsewhere on this thread is not ours to report
  KArgs a;
  a.one = 1.0f;
  a.mode = p->mode;
  a.ratio = p->ratio;
  a.rshift = p->ratio == 2 ? 1 : 0;
  a.B = p->batch;
  a.topk = p->topk;
  a.cb = p->cand_blocks;
  a.cb_in = p->cand_in_blocks;
  a.R = p->page_rows;
  a.rlog = p->page_rows == 128 ? 7 : 6;
  a.bt_stride = p->bt_stride;
  a.num_pages = p->num_pages;
  a.max_k_len = p->max_k_len;
  a.kstride = p->k_page_stride;
  a.sstride = p->s_page_stride;
  a.ncap = w.ncap;
  a.nbcap = w.nbcap;
  a.k = p->k_cache;
  a.ks = static_cast<const uint8_t*>(p->k_scale);
  a.bt = p->block_table;
  a.qsl = p->query_start_loc;
  a.klen = p->k_lens;
  a.smod = p->seq_mod;
  a.status = p->status_out;
  char* ws = static_cast<char*>(p->workspace);
  const bool consumer = p->mode == QLI_MODE_CONSUMER;
  const bool source = p->mode == QLI_MODE_SOURCE;
  a.keys = reinterpret_cast<uint32_t*>(ws + w.keys_off);
  a.bkeys = source ? reinterpret_cast<uint32_t*>(ws + w.bkeys_off) : nullptr;
  a.hdr = reinterpret_cast<PlanHdr*>(ws + w.plan_off);
  a.groups = reinterpret_cast<Group*>(ws + w.groups_off);  // [2][T]
  a.ustart = reinterpret_cast<int32_t*>(ws + w.ustart_off);
  a.wgs = reinterpret_cast<WgStart*>(ws + w.wgs_off);
  a.score_grid = std::min(kMaxScoreWGs, std::max(2, score_wgs_per_cu(p->mode, p->num_heads) * cu_count()));
  // batches of prefill shape with 32 heads (at least four query tokens per
  // request on average, so groups of four exist): the multi list runs in a
  // kernel of its own at four workgroups per CU, then the single list
  // (mixed batch source score kernels 3.01 -> 2.83 ms and 1.66 -> 1.38 ms
  // on one box).  With 64 heads the half-item path at three workgroups per
  // CU measured slower than the two-wave path (prefill chunk 752 -> 841 us:
  // the B fragments re-read per pass and the single accumulator set cost
  // more than the third wave gains), so 64-head batches keep the latter.
  a.multi_grid = 0;
  a.entry_base = 0;
  if (p->mode != QLI_MODE_CONSUMER && p->num_heads == 32 &&
      static_cast<int64_t>(p->num_tokens) >= 4 * static_cast<int64_t>(p->batch))
    a.multi_grid = std::min(kMaxScoreWGs - a.score_grid, multi_wgs_per_cu(p->num_heads) * cu_count());
  a.nxcd = xcd_count();
  a.slots = consumer ? reinterpret_cast<int32_t*>(ws + w.slots_off) : nullptr;
  a.srow = consumer ? reinterpret_cast<int32_t*>(ws + w.srow_off) : nullptr;
  a.ncount = consumer ? reinterpret_cast<int32_t*>(ws + w.ncount_off) : nullptr;
  a.tokv = reinterpret_cast<int32_t*>(ws + w.tokv_off);
  a.fused = 0;
  a.plan_wg = -1;

  // some request holds several query tokens (consumer mode: each reads its
  // own candidate rows of the request's K, so the rows are read repeatedly)
  const bool cached = p->num_tokens > p->batch;
  const int64_t NH = p->num_heads;
  for (int64_t t0 = 0; t0 < p->num_tokens; t0 += w.tokens) {
    a.t_base = static_cast<int>(t0);
    a.T = static_cast<int>(std::min<int64_t>(w.tokens, p->num_tokens - t0));
    a.q = p->q + t0 * NH * 128;
    a.qs = p->q_scale + t0 * NH;
    a.w = p->weights + t0 * NH;
    a.cand_in = p->cand_in ? p->cand_in + t0 * p->cand_in_blocks : nullptr;
    a.topk_out = p->topk_out + t0 * p->topk;
    a.cand_out = p->cand_out ? p->cand_out + t0 * p->cand_blocks : nullptr;
    a.dbg = p->dbg_scores ? p->dbg_scores + t0 * p->max_k_len : nullptr;
    a.dbg_qk = p->dbg_qk ? p->dbg_qk + t0 * NH * p->max_k_len : nullptr;
    a.epoch = g_epoch.fetch_add(1, std::memory_order_relaxed);
    launch_slice(p, w, a, cached, st, timed);
  }
  return hipGetLastError() == hipSuccess ? QLI_OK : QLI_ERR_HIP;
}

// The kernels of one slice (a.T tokens from a.t_base).
void launch_slice(const qli_params* p, const WsLayout& w, KArgs a, bool cached, hipStream_t st,
                  bool timed) {
  const bool consumer = p->mode == QLI_MODE_CONSUMER;
  const bool source = p->mode == QLI_MODE_SOURCE;
  const unsigned T = static_cast<unsigned>(a.T);
  const int64_t max_blocks = (static_cast<int64_t>(p->max_k_len) + 7) / 8;
  const bool bitmap = max_blocks <= 32 * static_cast<int64_t>(kPrepBitmapWords);
  if (consumer && bitmap && T >= static_cast<unsigned>(kPrepLeanMinTokens)) {
    // the plan, then one lean workgroup per token
    {
      Stamp s(QLI_KERNEL_PLAN, st, timed);
      plan_kernel<kPlanThreads><<<1, kPlanThreads, 0, st>>>(a);
    }
    Stamp s(QLI_KERNEL_CONSUMER_PREP, st, timed);
    const int nwcap = static_cast<int>((max_blocks + 31) / 32);
    const size_t lds = (static_cast<size_t>(nwcap) + static_cast<size_t>(p->cand_in_blocks) + 65) * 4;
    consumer_prep_lean_kernel<<<T, kPrepBitmapThreads, lds, st>>>(a, nwcap);
  } else if (consumer) {
    // block 0 plans, blocks 1..T prepare the tokens
    Stamp s(QLI_KERNEL_CONSUMER_PREP, st, timed);
    if (bitmap)
      consumer_prep_kernel<<<T + 1, kPrepThreads, 0, st>>>(a);
    else
      consumer_prep_sort_kernel<<<T + 1, kPrepThreads, 0, st>>>(a);
  } else if (w.ncap > 0 && a.multi_grid == 0 && a.T <= kFusedTokens && p->batch <= kFusedTokens) {
    // a decode-sized batch: every score workgroup plans for itself
    a.fused = 1;
  } else {
    Stamp s(QLI_KERNEL_PLAN, st, timed);
    // a small batch is planned by one wave
    if (a.T <= 64 && p->batch <= 256) plan_kernel<64><<<1, 64, 0, st>>>(a);
    else plan_kernel<kPlanThreads><<<1, kPlanThreads, 0, st>>>(a);
  }
  if (w.ncap > 0) {
    Stamp s(QLI_KERNEL_SCORE, st, timed);
    if (a.multi_grid > 0) {
      launch_score_multi(p->num_heads, p->mode, p->dbg_scores != nullptr, static_cast<unsigned>(a.multi_grid),
                         st, a);
      a.entry_base = a.multi_grid;
    }
    launch_score(p->num_heads, p->mode, p->dbg_scores != nullptr, cached, static_cast<unsigned>(a.score_grid),
                 st, a);
  }
  {
    Stamp s(QLI_KERNEL_SELECT, st, timed);
    const int64_t longest = w.ncap > w.nbcap ? w.ncap : w.nbcap;
    const dim3 grid(T, source ? 2 : 1);
    // rows no longer than a chunk (every n <= its row capacity) take the
    // single-chunk variants
    const int64_t rows = static_cast<int64_t>(grid.x) * grid.y;
    a.sel_lo = 0;
    a.sel_hi = INT32_MAX;
    if (rows > 4 * static_cast<int64_t>(cu_count()) && longest > kSelShortChunk) {
      // many rows whose lengths may differ widely (mixed batches): one
      // launch per length class, each taking only its rows, so that short
      // rows run at the occupancy of the narrow variants instead of all at
      // that of the longest row's variant; rows above 16384 keys take the
      // chunked selection at 512 threads (three workgroups per CU, where
      // the 1024-thread variants fit one: mixed batch source selects
      // 1.05 -> 1.00 ms and 0.61 -> 0.55 ms)
      const int bounds[3] = {kSelShortChunk, sel_chunk(512), INT32_MAX};
      for (int c = 0; c < 3; ++c) {
        a.sel_lo = c == 0 ? 0 : bounds[c - 1] + 1;
        a.sel_hi = bounds[c];
        if (a.sel_lo > longest) break;
        if (c == 0) select_kernel<512, false, kSelShortChunk><<<grid, 512, 0, st>>>(a);
        else if (c == 1) select_kernel<512, false><<<grid, 512, 0, st>>>(a);
        else select_kernel<512, true><<<grid, 512, 0, st>>>(a);
      }
    } else if (longest <= sel_chunk(256)) select_kernel<256, false><<<grid, 256, 0, st>>>(a);
    else if (longest <= kSelShortChunk) select_kernel<512, false, kSelShortChunk><<<grid, 512, 0, st>>>(a);
    else if (longest <= sel_chunk(512)) {
      // rows of 10241..16384 keys: when they leave CUs idle (decode-sized
      // batches), 1024 threads with 16 keys each finish a row sooner (76
      // VGPRs, nothing spilled: consumer rows of 16384 keys 14.4 -> 13.4 us);
      // otherwise three 512-thread workgroups share a CU
      if (static_cast<int64_t>(grid.x) * grid.y <= cu_count())
        select_kernel<1024, false, 16384><<<grid, 1024, 0, st>>>(a);
      else
        select_kernel<512, false><<<grid, 512, 0, st>>>(a);
    }
    else if (longest <= sel_chunk(1024)) select_kernel<1024, false><<<grid, 1024, 0, st>>>(a);
    else select_kernel<1024, true><<<grid, 1024, 0, st>>>(a);
  }
}

}  // namespace qli
