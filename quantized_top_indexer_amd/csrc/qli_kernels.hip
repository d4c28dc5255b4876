// HIP kernels of the quantized lightning indexer for CDNA4 (gfx950).
//
// Three kernels per call (DeepSeek V4.1 QLI developer guide, "数据流" and
// "当前 A3 契约"):
//   consumer_prep  (consumer mode only) one workgroup per token: sort and
//                  de-duplicate the incoming candidate block ids, drop ids
//                  without a visible position -> a dense slot list.
//   score          one workgroup (4 waves) per (token, 256-slot chunk):
//                  stage 64 paged K rows per wave in LDS, INT8 MFMA
//                  (v_mfma_i32_32x32x32_i8) of the token's [N x 128] queries
//                  against them, then the golden FP16/FP32 epilogue, the
//                  8-position block maximum, and order-preserving u32 keys.
//   select         one workgroup per token: radix select of the position
//                  top-k (and, in source mode, of the candidate blocks with
//                  the last visible block pinned), emitted in ascending
//                  order by a stream compaction, -1 tail.
//
// Exactness: the epilogue follows the golden order with one IEEE RNE
// rounding per step and sums heads in ascending order from +0.0f, so the
// scores, and therefore every selection, are bit-identical to a sequential
// reference.  The file is built with -ffp-contract=off so that no FP16
// product is fused into the FP32 accumulation.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <mutex>
#include <vector>

#include "qli.h"
#include "qli_internal.h"

namespace qli {
namespace {

typedef int32_t i32x4 __attribute__((ext_vector_type(4)));
typedef int32_t i32x16 __attribute__((ext_vector_type(16)));

struct KArgs {
  int mode, ratio, B, T, topk, cb, cb_in, R, bt_stride, num_pages, max_k_len, nchunks;
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
  uint32_t* status;
  uint32_t* keys;
  uint32_t* bkeys;
  int32_t* slots;
  int32_t* nslots;
};

__device__ __forceinline__ void raise_flag(const KArgs& a, uint32_t bit) {
  if (a.status) atomicOr(a.status, bit);
}

// Request b of token t and its visible compressed count V (causal mask
// mode 3: the queries are the request's last raw positions; the query at
// raw position p sees entries j < floor((p+1)/r)).  Out-of-contract
// metadata is flagged and clamped so that every access stays in bounds.
struct TokView {
  int b;
  int V;
};

__device__ TokView token_view(const KArgs& a, int t, bool report) {
  int lo = 0, hi = a.B - 1;
  while (lo < hi) {
    int mid = (lo + hi + 1) >> 1;
    if (a.qsl[mid] <= t) lo = mid;
    else hi = mid - 1;
  }
  const int b = lo;
  const int q0 = a.qsl[b], q1 = a.qsl[b + 1];
  int L = a.klen[b];
  int s = a.smod ? a.smod[b] : 0;
  if (L < 0 || L > a.max_k_len) {
    if (report) raise_flag(a, QLI_DEV_BAD_LENGTH);
    return {b, 0};
  }
  if (s < 0 || s >= a.ratio) {
    if (report) raise_flag(a, QLI_DEV_BAD_METADATA);
    return {b, 0};
  }
  const int64_t n = static_cast<int64_t>(q1) - q0;
  const int64_t S = static_cast<int64_t>(L) * a.ratio + s;
  if (t < q0 || t >= q1 || n > S) {
    if (report) raise_flag(a, QLI_DEV_BAD_METADATA);
    return {b, 0};
  }
  const int64_t p = S - n + (t - q0);
  int64_t V = (p + 1) / a.ratio;
  if (V > L) V = L;
  return {b, static_cast<int>(V)};
}

// Page holding compressed position `pos` of request b, or -1.
__device__ __forceinline__ int page_of(const KArgs& a, const int32_t* btrow, int pos) {
  const int idx = pos / a.R;
  if (idx >= a.bt_stride) return -1;
  const int page = btrow[idx];
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

__device__ __forceinline__ _Float16 h_from_bits(uint16_t v) { return __builtin_bit_cast(_Float16, v); }
__device__ __forceinline__ uint16_t h_bits(_Float16 v) { return __builtin_bit_cast(uint16_t, v); }

// ---------------------------------------------------------------------------
// score
// ---------------------------------------------------------------------------
//
// Wave w of a workgroup owns slots [s0, s0 + 64).  MFMA operands
// (v_mfma_i32_32x32x32_i8, 64 lanes):
//   A (queries): lane l supplies row l%32 of a 32-head tile, 16 bytes of the
//     head dimension; B (keys): lane l supplies column l%32 (one position),
//     the same 16 bytes.  Dim d = 64*(l/32) + 16*step + byte feeds both, so
//     the K reduction pairs q[h,d] with k[j,d] whatever the hardware order.
//   C: lane l holds column l%32, rows 8*(i/4) + 4*(l/32) + i%4 (i < 16).
// A rows are permuted so that C register i of lane group g = l/32 in head
// tile m is head g*(N/2) + 16*m + i: lanes 0..31 then hold heads
// 0..N/2-1, lanes 32..63 heads N/2..N-1 of the same positions, and one
// v_permlane32_swap gives every lane all N heads of one position in
// ascending order (lane L -> slot s0 + L).
template <int NH, bool CONSUMER>
__global__ __launch_bounds__(256) void score_kernel(KArgs a) {
  constexpr int MT = NH / 32;  // 32-head tiles
  constexpr int HALF = NH / 2;
  const int64_t wg = blockIdx.x;
  const int t = static_cast<int>(wg / a.nchunks);
  const int chunk = static_cast<int>(wg % a.nchunks);
  const TokView tv = token_view(a, t, threadIdx.x == 0 && chunk == 0);
  const int n_t = CONSUMER ? a.nslots[t] * 8 : tv.V;
  const int base = chunk * kChunk;
  if (base >= n_t) return;  // uniform over the workgroup

  const int wave = threadIdx.x >> 6;
  const int lane = threadIdx.x & 63;
  const int s0 = base + wave * 64;
  const int32_t* btrow = a.bt + static_cast<int64_t>(tv.b) * a.bt_stride;
  const int32_t* slots = CONSUMER ? a.slots + static_cast<int64_t>(t) * a.cb_in : nullptr;

  __shared__ __attribute__((aligned(16))) int8_t lds[4 * 64 * 128];
  int8_t* my = lds + wave * (64 * 128);

  // ---- stage K: load u covers slots s0+8u .. s0+8u+7 (one 1 KB run) ------
  uint32_t bad = 0;
#pragma unroll
  for (int u = 0; u < 8; ++u) {
    const int r8 = lane >> 3, col = lane & 7;
    const int row = 8 * u + r8;
    const int slot = s0 + row;
    i32x4 v = {0, 0, 0, 0};
    if (slot < n_t) {
      const int pos = CONSUMER ? slots[slot >> 3] * 8 + (slot & 7) : slot;
      if (pos < tv.V) {
        const int page = page_of(a, btrow, pos);
        if (page >= 0) {
          const int8_t* src = a.k + static_cast<int64_t>(page) * a.kstride +
                              static_cast<int64_t>(pos % a.R) * 128 + col * 16;
          v = *reinterpret_cast<const i32x4*>(src);
        } else {
          bad = 1;
        }
      }
    }
    *reinterpret_cast<i32x4*>(my + row * 128 + ((col ^ (row & 7)) << 4)) = v;
  }
  if (bad) raise_flag(a, QLI_DEV_BAD_PAGE);

  // ---- queries as MFMA A operands ------------------------------------------
  i32x4 qa[MT][4];
  {
    const int r = lane & 31;
    const int g = lane >> 5;
#pragma unroll
    for (int m = 0; m < MT; ++m) {
      const int head = ((r >> 2) & 1) * HALF + 16 * m + 4 * (r >> 3) + (r & 3);
      const int8_t* qrow = a.q + (static_cast<int64_t>(t) * NH + head) * 128 + 64 * g;
#pragma unroll
      for (int s = 0; s < 4; ++s) qa[m][s] = *reinterpret_cast<const i32x4*>(qrow + 16 * s);
    }
  }

  // per-head multipliers m_h = fp16(w_h * q_scale_h) for this lane's heads
  _Float16 mh[HALF];
  {
    const int g = lane >> 5;
    const uint16_t* wr = a.w + static_cast<int64_t>(t) * NH + g * HALF;
    const uint16_t* qr = a.qs + static_cast<int64_t>(t) * NH + g * HALF;
#pragma unroll
    for (int j = 0; j < HALF; ++j) mh[j] = h_from_bits(wr[j]) * h_from_bits(qr[j]);
  }

  __syncthreads();

  // ---- INT8 MFMA -----------------------------------------------------------
  i32x16 acc[MT][2];
#pragma unroll
  for (int m = 0; m < MT; ++m)
#pragma unroll
    for (int n = 0; n < 2; ++n)
#pragma unroll
      for (int i = 0; i < 16; ++i) acc[m][n][i] = 0;

#pragma unroll
  for (int n = 0; n < 2; ++n) {
    const int row = 32 * n + (lane & 31);
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      const int col = 4 * (lane >> 5) + s;
      const i32x4 bk = *reinterpret_cast<const i32x4*>(my + row * 128 + ((col ^ (row & 7)) << 4));
#pragma unroll
      for (int m = 0; m < MT; ++m)
        acc[m][n] = __builtin_amdgcn_mfma_i32_32x32x32_i8(qa[m][s], bk, acc[m][n], 0, 0, 0);
    }
  }

  // ---- golden epilogue -------------------------------------------------------
  // x = fp16(qk/1024) (qk*2^-10 is exact in FP32), ReLU, p = fp16(x*m)
  uint32_t pk[2][HALF / 2];
#pragma unroll
  for (int n = 0; n < 2; ++n) {
#pragma unroll
    for (int m = 0; m < MT; ++m) {
#pragma unroll
      for (int i = 0; i < 16; i += 2) {
        _Float16 p2[2];
#pragma unroll
        for (int e = 0; e < 2; ++e) {
          _Float16 x = static_cast<_Float16>(static_cast<float>(acc[m][n][i + e]) * 0.0009765625f);
          x = x > static_cast<_Float16>(0.0f) ? x : static_cast<_Float16>(0.0f);
          p2[e] = x * mh[16 * m + i + e];
        }
        pk[n][(16 * m + i) >> 1] = static_cast<uint32_t>(h_bits(p2[0])) |
                                   (static_cast<uint32_t>(h_bits(p2[1])) << 16);
      }
    }
  }
  // lanes 0..31: heads lo of tile 0 / lanes 32..63: heads hi of tile 1 stay;
  // the other halves cross over, so each lane ends with all heads of slot s0+lane
  uint32_t lo[HALF / 2], hi[HALF / 2];
#pragma unroll
  for (int j = 0; j < HALF / 2; ++j) {
    auto r = __builtin_amdgcn_permlane32_swap(pk[0][j], pk[1][j], false, false);
    lo[j] = r[0];
    hi[j] = r[1];
  }
  float sum = 0.0f;
#pragma unroll
  for (int j = 0; j < HALF / 2; ++j) {
    sum = sum + static_cast<float>(h_from_bits(static_cast<uint16_t>(lo[j] & 0xFFFFu)));
    sum = sum + static_cast<float>(h_from_bits(static_cast<uint16_t>(lo[j] >> 16)));
  }
#pragma unroll
  for (int j = 0; j < HALF / 2; ++j) {
    sum = sum + static_cast<float>(h_from_bits(static_cast<uint16_t>(hi[j] & 0xFFFFu)));
    sum = sum + static_cast<float>(h_from_bits(static_cast<uint16_t>(hi[j] >> 16)));
  }

  // ---- K scale, key, block max ------------------------------------------------
  const int slot = s0 + lane;
  uint32_t key = 0;
  if (slot < n_t) {
    const int pos = CONSUMER ? slots[slot >> 3] * 8 + (slot & 7) : slot;
    if (pos < tv.V) {
      const int page = page_of(a, btrow, pos);
      if (page >= 0) {
        const uint8_t* sp = a.ks + static_cast<int64_t>(page) * a.sstride +
                            static_cast<int64_t>(pos % a.R) * 2;
        const float kscale = static_cast<float>(h_from_bits(*reinterpret_cast<const uint16_t*>(sp)));
        const float score = sum * kscale;
        key = order_key(score);
        if (a.dbg) a.dbg[static_cast<int64_t>(t) * a.max_k_len + pos] = score;
      }
    }
  }
  a.keys[static_cast<int64_t>(t) * a.ncap + slot] = key;
  if (!CONSUMER && a.mode == QLI_MODE_SOURCE) {
    uint32_t bk = key;
    bk = max(bk, static_cast<uint32_t>(__shfl_xor(static_cast<int>(bk), 1)));
    bk = max(bk, static_cast<uint32_t>(__shfl_xor(static_cast<int>(bk), 2)));
    bk = max(bk, static_cast<uint32_t>(__shfl_xor(static_cast<int>(bk), 4)));
    if ((lane & 7) == 0 && slot < n_t) a.bkeys[static_cast<int64_t>(t) * a.nbcap + (slot >> 3)] = bk;
  }
}

// ---------------------------------------------------------------------------
// block-wide helpers (1024 threads)
// ---------------------------------------------------------------------------
constexpr int kSelThreads = 1024;

__device__ __forceinline__ uint32_t wave_inclusive_scan(uint32_t v, int lane) {
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    uint32_t o = static_cast<uint32_t>(__shfl_up(static_cast<int>(v), d));
    if (lane >= d) v += o;
  }
  return v;
}

// Exclusive prefix of v over the workgroup; *total receives the sum.
__device__ uint32_t block_exclusive_scan(uint32_t v, uint32_t* total, uint32_t* sh) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const uint32_t inc = wave_inclusive_scan(v, lane);
  if (lane == 63) sh[wave] = inc;
  __syncthreads();
  if (wave == 0) {
    uint32_t w = lane < kSelThreads / 64 ? sh[lane] : 0u;
    uint32_t wi = wave_inclusive_scan(w, lane);
    if (lane < kSelThreads / 64) sh[32 + lane] = wi - w;
    if (lane == kSelThreads / 64 - 1) sh[63] = wi;
  }
  __syncthreads();
  const uint32_t out = sh[32 + wave] + inc - v;
  *total = sh[63];
  __syncthreads();
  return out;
}

// Keys of the items a selection ranks.
struct KeySrc {
  const uint32_t* keys;
  int pin;  // index forced to the top, or -1
  __device__ __forceinline__ uint32_t operator()(int i) const {
    return i == pin ? 0xFFFFFFFFu : keys[i];
  }
};

// Select the best min(k, #nonzero) of keys[0..n) by (key desc, index asc)
// and write map(index) for them in ascending index order to out[0..k),
// -1 after.  Radix select over 8-bit digits (MSB first) finds the k-th key
// T; everything above T is taken, plus the lowest-index keys equal to T.
template <class Map>
__device__ void select_topk(KeySrc src, int n, int k, int32_t* out, Map map, uint32_t* hist,
                            uint32_t* sh) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  uint32_t prefix = 0, mask = 0;
  int krem = k;
  bool take_all = false;
  for (int pass = 0; pass < 4; ++pass) {
    const int shift = 24 - 8 * pass;
    if (tid < 256) hist[tid] = 0;
    __syncthreads();
    for (int i = tid; i < n; i += kSelThreads) {
      const uint32_t key = src(i);
      if (key != 0 && (key & mask) == prefix) atomicAdd(&hist[(key >> shift) & 255u], 1u);
    }
    __syncthreads();
    if (wave == 0) {
      // suffix sums: lane l covers bins 4l..4l+3
      uint32_t c = hist[4 * lane] + hist[4 * lane + 1] + hist[4 * lane + 2] + hist[4 * lane + 3];
      // inclusive suffix scan over lanes
      uint32_t s = c;
#pragma unroll
      for (int d = 1; d < 64; d <<= 1) {
        uint32_t o = static_cast<uint32_t>(__shfl_down(static_cast<int>(s), d));
        if (lane + d < 64) s += o;
      }
      const uint32_t above_lane = s - c;  // bins > 4l+3
      const uint32_t total = static_cast<uint32_t>(__shfl(static_cast<int>(s), 0));
      if (pass == 0 && total <= static_cast<uint32_t>(k)) {
        if (lane == 0) sh[0] = 1u;  // every eligible key is selected
      } else {
        if (lane == 0) sh[0] = 0u;
        if (above_lane < static_cast<uint32_t>(krem) && s >= static_cast<uint32_t>(krem)) {
          uint32_t cum = above_lane;
          for (int bidx = 3; bidx >= 0; --bidx) {
            const uint32_t h = hist[4 * lane + bidx];
            if (cum + h >= static_cast<uint32_t>(krem)) {
              sh[1] = static_cast<uint32_t>(4 * lane + bidx);
              sh[2] = cum;
              break;
            }
            cum += h;
          }
        }
      }
    }
    __syncthreads();
    if (sh[0]) {
      take_all = true;
      __syncthreads();
      break;
    }
    const uint32_t digit = sh[1];
    krem -= static_cast<int>(sh[2]);
    prefix |= digit << shift;
    mask |= 255u << shift;
    __syncthreads();
  }

  // stream compaction in ascending index order
  const uint32_t thr = prefix;
  const uint32_t need = take_all ? 0u : static_cast<uint32_t>(krem);
  uint32_t run_sel = 0, run_eq = 0;
  for (int base = 0; base < n; base += kSelThreads * 4) {
    uint32_t keys[4];
    uint32_t neq = 0;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int i = base + tid * 4 + e;
      keys[e] = i < n ? src(i) : 0u;
      if (!take_all && keys[e] == thr && keys[e] != 0) ++neq;
    }
    uint32_t tot_eq;
    uint32_t eq_rank = block_exclusive_scan(neq, &tot_eq, sh) + run_eq;
    bool sel[4];
    uint32_t nsel = 0;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      if (take_all) {
        sel[e] = keys[e] != 0;
      } else {
        const bool eq = keys[e] == thr && keys[e] != 0;
        sel[e] = keys[e] > thr || (eq && eq_rank < need);
        if (eq) ++eq_rank;
      }
      nsel += sel[e] ? 1u : 0u;
    }
    uint32_t tot_sel;
    uint32_t at = block_exclusive_scan(nsel, &tot_sel, sh) + run_sel;
#pragma unroll
    for (int e = 0; e < 4; ++e)
      if (sel[e] && at < static_cast<uint32_t>(k)) out[at++] = map(base + tid * 4 + e);
    run_sel += tot_sel;
    run_eq += tot_eq;
  }
  for (int i = static_cast<int>(run_sel) + tid; i < k; i += kSelThreads) out[i] = -1;
  __syncthreads();
}

struct MapIdentity {
  __device__ __forceinline__ int32_t operator()(int i) const { return i; }
};

struct MapSlots {
  const int32_t* slots;
  __device__ __forceinline__ int32_t operator()(int i) const { return slots[i >> 3] * 8 + (i & 7); }
};

__global__ __launch_bounds__(kSelThreads) void select_kernel(KArgs a) {
  __shared__ uint32_t hist[256];
  __shared__ uint32_t sh[64];
  const int t = blockIdx.x;
  const TokView tv = token_view(a, t, false);
  int32_t* out = a.topk_out + static_cast<int64_t>(t) * a.topk;
  const uint32_t* keys = a.keys + static_cast<int64_t>(t) * a.ncap;
  if (a.mode == QLI_MODE_CONSUMER) {
    const int32_t* slots = a.slots + static_cast<int64_t>(t) * a.cb_in;
    const int n = a.nslots[t] * 8;
    select_topk(KeySrc{keys, -1}, n, a.topk, out, MapSlots{slots}, hist, sh);
  } else {
    select_topk(KeySrc{keys, -1}, tv.V, a.topk, out, MapIdentity{}, hist, sh);
  }
  if (a.mode == QLI_MODE_SOURCE) {
    const int nb = (tv.V + 7) / 8;
    int32_t* cout = a.cand_out + static_cast<int64_t>(t) * a.cb;
    select_topk(KeySrc{a.bkeys + static_cast<int64_t>(t) * a.nbcap, nb - 1}, nb, a.cb, cout,
                MapIdentity{}, hist, sh);
  }
}

// ---------------------------------------------------------------------------
// consumer_prep: sorted unique visible incoming block ids per token
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(kSelThreads) void consumer_prep_kernel(KArgs a) {
  __shared__ int32_t v[QLI_MAX_CAND_BLOCKS];
  __shared__ uint32_t sh[64];
  const int t = blockIdx.x;
  const int tid = threadIdx.x;
  const TokView tv = token_view(a, t, tid == 0);
  const int nblocks = (tv.V + 7) / 8;
  const int cbi = a.cb_in;
  int n2 = 64;
  while (n2 < cbi) n2 <<= 1;
  const int32_t* cin = a.cand_in + static_cast<int64_t>(t) * cbi;
  for (int i = tid; i < n2; i += kSelThreads) {
    int c = i < cbi ? cin[i] : INT32_MAX;
    if (c < 0 || c >= nblocks) c = INT32_MAX;
    v[i] = c;
  }
  __syncthreads();
  // bitonic sort, ascending
  for (int size = 2; size <= n2; size <<= 1) {
    for (int stride = size >> 1; stride > 0; stride >>= 1) {
      for (int i = tid; i < n2 / 2; i += kSelThreads) {
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
  // unique compaction (each thread two consecutive entries)
  int32_t* slots = a.slots + static_cast<int64_t>(t) * cbi;
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
  uint32_t at = block_exclusive_scan(cnt, &total, sh);
#pragma unroll
  for (int e = 0; e < 2; ++e)
    if (f[e]) slots[at++] = v[i0 + e];
  if (tid == 0) a.nslots[t] = static_cast<int32_t>(total);
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

struct Stamp {
  int kernel;
  hipStream_t st;
  hipEvent_t start = nullptr, stop = nullptr;
  Stamp(int k, hipStream_t s) : kernel(k), st(s) {
    if (!g_timing_on) return;
    if (hipEventCreate(&start) != hipSuccess || hipEventCreate(&stop) != hipSuccess) return;
    hipEventRecord(start, st);
  }
  ~Stamp() {
    if (!start || !stop) return;
    hipEventRecord(stop, st);
    std::lock_guard<std::mutex> g(g_timing_mu);
    g_pending.push_back({kernel, start, stop});
  }
};
}  // namespace

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
    hipEventDestroy(t.start);
    hipEventDestroy(t.stop);
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

int launch(const qli_params* p, const WsLayout& w, void* stream) {
  hipStream_t st = static_cast<hipStream_t>(stream);
  KArgs a;
  a.mode = p->mode;
  a.ratio = p->ratio;
  a.B = p->batch;
  a.T = p->num_tokens;
  a.topk = p->topk;
  a.cb = p->cand_blocks;
  a.cb_in = p->cand_in_blocks;
  a.R = p->page_rows;
  a.bt_stride = p->bt_stride;
  a.num_pages = p->num_pages;
  a.max_k_len = p->max_k_len;
  a.nchunks = static_cast<int>(w.ncap / kChunk);
  a.kstride = p->k_page_stride;
  a.sstride = p->s_page_stride;
  a.ncap = w.ncap;
  a.nbcap = w.nbcap;
  a.q = p->q;
  a.qs = p->q_scale;
  a.w = p->weights;
  a.k = p->k_cache;
  a.ks = static_cast<const uint8_t*>(p->k_scale);
  a.bt = p->block_table;
  a.qsl = p->query_start_loc;
  a.klen = p->k_lens;
  a.smod = p->seq_mod;
  a.cand_in = p->cand_in;
  a.topk_out = p->topk_out;
  a.cand_out = p->cand_out;
  a.dbg = p->dbg_scores;
  a.status = p->status_out;
  char* ws = static_cast<char*>(p->workspace);
  a.keys = reinterpret_cast<uint32_t*>(ws + w.keys_off);
  a.bkeys = p->mode == QLI_MODE_SOURCE ? reinterpret_cast<uint32_t*>(ws + w.bkeys_off) : nullptr;
  a.slots = p->mode == QLI_MODE_CONSUMER ? reinterpret_cast<int32_t*>(ws + w.slots_off) : nullptr;
  a.nslots = p->mode == QLI_MODE_CONSUMER ? reinterpret_cast<int32_t*>(ws + w.nslots_off) : nullptr;

  const unsigned T = static_cast<unsigned>(p->num_tokens);
  const bool consumer = p->mode == QLI_MODE_CONSUMER;
  if (consumer) {
    Stamp s(QLI_KERNEL_CONSUMER_PREP, st);
    consumer_prep_kernel<<<T, kSelThreads, 0, st>>>(a);
  }
  if (a.nchunks > 0) {
    Stamp s(QLI_KERNEL_SCORE, st);
    const unsigned grid = T * static_cast<unsigned>(a.nchunks);
    if (p->num_heads == 64) {
      if (consumer) score_kernel<64, true><<<grid, 256, 0, st>>>(a);
      else score_kernel<64, false><<<grid, 256, 0, st>>>(a);
    } else {
      if (consumer) score_kernel<32, true><<<grid, 256, 0, st>>>(a);
      else score_kernel<32, false><<<grid, 256, 0, st>>>(a);
    }
  }
  {
    Stamp s(QLI_KERNEL_SELECT, st);
    select_kernel<<<T, kSelThreads, 0, st>>>(a);
  }
  return hipGetLastError() == hipSuccess ? QLI_OK : QLI_ERR_HIP;
}

}  // namespace qli
