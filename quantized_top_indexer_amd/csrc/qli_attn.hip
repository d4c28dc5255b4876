// Sparse attention over the indexer's positions: the consumer of the
// indices ("DeepSeek V4.1-Flash 登陆昇腾 · 需求故事（PR 16925）", section 4;
// "DeepSeek V4.1-Flash CED·CSA2 架构拆解 × vllm-ascend 性能协助点", operator
// table: a sliding-window stage and the compressed global stage, with
// sinks, over BF16 TND queries and PA_BBND paged caches).  The operation is
// stated in include/qli.h (qli_sparse_attention).
//
// One workgroup per (query token, group of 16 heads); the head groups of a
// token run on one XCD (workgroup i runs on XCD i mod 8), so the rows they
// all read come from HBM once and from that XCD's L2 for the others.
//   1. The token's entries (its valid index positions, then its window) are
//      resolved through the block tables into row addresses, compacted in
//      order into LDS.
//   2. Two pairs of waves take alternate tiles of 16 entries; both waves
//      of a pair score every tile of the pair (the 16 heads' logits) and
//      keep their own online softmax, each for the outputs of half the
//      dims.  A tile's rows go into LDS twice, row-major (keys: A operand
//      of S^T = K Q^T, 16x16x32 BF16 MFMAs over D = 512) and transposed
//      (values: A operand of O^T = V^T P^T, 16x16x16 BF16 MFMAs).  The S^T
//      accumulator of lane l holds head l % 16 for rows 4 (l / 16) .. + 3,
//      which is exactly the B operand P^T needs, so the weights never leave
//      their lanes.  The next step's rows are loaded into registers while a
//      step is scored.
//   3. The two pairs' states meet in LDS; each thread writes 32 outputs of
//      one head.
// Keys and values are the same cache entry (one shared latent KV head).
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "qli.h"
#include "qli_internal.h"

namespace qli {
namespace {

constexpr int kD = 512;               // head dim (key and value width)
constexpr int kHeadsWG = 16;          // heads per workgroup
constexpr int kAttnThreads = 256;     // four waves
constexpr int kTile = 16;             // entries per wave tile
constexpr int kMaxEntries = QLI_ATTN_MAX_TOPK + QLI_ATTN_MAX_WINDOW;
constexpr int kWaveLds = 2 * kTile * kD * 2;  // one tile buffer: row-major and transposed copies, 32 KB
constexpr int kQOff = 4 * kWaveLds;           // the 16 heads' queries after the four tile buffers
constexpr int kEntOff = kQOff + kHeadsWG * kD * 2;  // entries (4 bytes each)
constexpr int kMiscOff = kEntOff + kMaxEntries * 4;
constexpr int kLdsBytes = kMiscOff + 1024;
static_assert(kLdsBytes <= 160 * 1024, "LDS of one workgroup");
// an entry: source (bit 31: raw pool), page (bits 8..30), row (bits 0..7)
constexpr uint32_t kNoEntry = 0xFFFFFFFFu;
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

typedef __bf16 bf8 __attribute__((ext_vector_type(8)));
typedef short s4 __attribute__((ext_vector_type(4)));
typedef float f4 __attribute__((ext_vector_type(4)));
typedef int i4 __attribute__((ext_vector_type(4)));
typedef int i2 __attribute__((ext_vector_type(2)));

struct AttnArgs {
  int H, B, T, topk, window;
  int c_rows, c_bts, r_rows, r_bts;
  int G;  // head groups (H / 16)
  int64_t c_pages, r_pages, c_stride, r_stride;
  float zscale;  // scale * log2(e): logits in base 2
  const uint16_t* q;
  const char* c_cache;
  const int32_t* c_bt;
  const int32_t* c_lens;
  const char* r_cache;
  const int32_t* r_bt;
  const int32_t* r_lens;
  const int32_t* qsl;
  const int32_t* idx;
  const float* sinks;
  uint16_t* out;
  float* lse;
  uint32_t* status;
};

__device__ __forceinline__ void flag(const AttnArgs& a, uint32_t bits) {
  if (a.status) atomicOr(a.status, bits);
}

// BF16 of an FP32 value, round to nearest even (finite inputs).
__device__ __forceinline__ uint32_t bf16_rne(float x) {
  const uint32_t u = __float_as_uint(x);
  return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}

__device__ __forceinline__ float wave_max_heads(float x) {
  // lanes l, l ^ 16, l ^ 32, l ^ 48 hold one head
  x = fmaxf(x, __shfl_xor(x, 16));
  return fmaxf(x, __shfl_xor(x, 32));
}
__device__ __forceinline__ float wave_sum_heads(float x) {
  x += __shfl_xor(x, 16);
  return x + __shfl_xor(x, 32);
}

// Exclusive prefix sum over the 256 threads (sh: four words of LDS).
__device__ uint32_t block_exclusive_scan_attn(uint32_t v, uint32_t* total, uint32_t* sh) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  uint32_t inc = v;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const uint32_t y = static_cast<uint32_t>(__shfl_up(static_cast<int>(inc), o));
    if (lane >= o) inc += y;
  }
  if (lane == 63) sh[wave] = inc;
  __syncthreads();
  uint32_t before = 0, tot = 0;
#pragma unroll
  for (int w = 0; w < kAttnThreads / 64; ++w) {
    const uint32_t x = sh[w];
    before += w < wave ? x : 0u;
    tot += x;
  }
  *total = tot;
  __syncthreads();
  return before + inc - v;
}

// Transposed tile layout: dim d holds the 16 rows' values (32 B) at slot(d);
// the swizzle spreads the rows written by one store instruction (dims 8
// apart) and read by one MFMA operand load (16 consecutive dims) over the
// LDS banks.
__device__ __forceinline__ int vt_offset(int d, int half) {
  const int c = d >> 3, e = d & 7;
  const int slot = (c << 3) | (e ^ (c & 7));
  return slot * 32 + ((half ^ (c >> 3)) & 1) * 16;
}

// The lane index through a move the compiler cannot see through: the LDS
// offsets derived from it are recomputed per tile (a few VALU instructions)
// instead of being hoisted out of the tile loop, where they would hold
// about a hundred registers.
__device__ __forceinline__ int opaque_lane() {
  int l;
  asm volatile("v_mov_b32 %0, %1" : "=v"(l) : "v"(static_cast<int>(threadIdx.x & 63)));
  return l;
}

// Row-major tile layout: chunk ch (16 B) of row i at chunk ch ^ i.
__device__ __forceinline__ int krm_offset(int i, int ch) { return i * (kD * 2) + ((ch ^ i) << 4); }

__global__ __launch_bounds__(kAttnThreads, 1) void sparse_attn_kernel(AttnArgs a) {
  __shared__ __attribute__((aligned(16))) char lds[kLdsBytes];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  // workgroup -> (token, head group); the head groups of a token share i mod 8
  const int x = blockIdx.x & 7, r = blockIdx.x >> 3;
  const int g = r % a.G;
  const int t = x + 8 * (r / a.G);
  if (t >= a.T) return;
  uint32_t* ent = reinterpret_cast<uint32_t*>(lds + kEntOff);
  char* qs = lds + kQOff;
  int* misc = reinterpret_cast<int*>(lds + kMiscOff);
  uint32_t* scan = reinterpret_cast<uint32_t*>(misc + 16);

  // the queries of the workgroup's 16 heads (every wave scores all 16) in
  // LDS, chunk ch (16 B) of head h at chunk ch ^ h
  {
    const uint16_t* qg = a.q + (static_cast<int64_t>(t) * a.H + kHeadsWG * g) * kD;
#pragma unroll
    for (int u = 0; u < kHeadsWG * kD / 8 / kAttnThreads; ++u) {
      const int c = u * kAttnThreads + tid;  // 16-byte chunk of the group's queries
      const int h = c >> 6, ch = c & 63;
      *reinterpret_cast<i4*>(qs + krm_offset(h, ch)) = *reinterpret_cast<const i4*>(qg + 8 * c);
    }
  }

  // 1. request, raw position and the entry list
  if (tid == 0) misc[0] = -1;
  __syncthreads();
  for (int i = tid; i < a.B; i += kAttnThreads)
    if (a.qsl[i] <= t && t < a.qsl[i + 1]) misc[0] = i;
  __syncthreads();
  const int b = misc[0];
  int E = 0;
  if (b >= 0) {
    const int q0 = a.qsl[b], q1 = a.qsl[b + 1];
    // lengths beyond what the request's block-table row can map are cut there
    const int64_t cmax = static_cast<int64_t>(a.c_bts) * a.c_rows, rmax = static_cast<int64_t>(a.r_bts) * a.r_rows;
    int64_t clen = a.c_lens[b];
    int64_t rlen = a.window > 0 ? a.r_lens[b] : 0;
    if (clen < 0 || rlen < 0 || clen > cmax || rlen > rmax) {
      if (tid == 0) flag(a, QLI_DEV_BAD_LENGTH);
      clen = min(max<int64_t>(clen, 0), cmax);
      rlen = min(max<int64_t>(rlen, 0), rmax);
    }
    const int64_t p = rlen - (q1 - q0) + (t - q0);
    if (a.window > 0 && rlen < q1 - q0 && tid == 0) flag(a, QLI_DEV_BAD_METADATA);
    const int64_t s0 = max<int64_t>(0, p - a.window + 1);
    const int nwin = a.window > 0 && p >= 0 ? static_cast<int>(p - s0 + 1) : 0;
    // virtual entries: topk index slots, then the window; each thread a run of them
    const int nv = a.topk + nwin;
    const int per = (nv + kAttnThreads - 1) / kAttnThreads;
    const int v0 = min(nv, tid * per), v1 = min(nv, v0 + per);
    uint32_t bad = 0;
    auto resolve = [&](int v) -> uint32_t {
      if (v < a.topk) {
        const int c = a.idx[static_cast<int64_t>(t) * a.topk + v];
        if (c < 0) return kNoEntry;
        if (c >= clen) {
          bad |= QLI_DEV_BAD_INDEX;
          return kNoEntry;
        }
        const int pg = a.c_bt[static_cast<int64_t>(b) * a.c_bts + c / a.c_rows];
        if (pg < 0 || pg >= a.c_pages) {
          bad |= QLI_DEV_BAD_PAGE;
          return kNoEntry;
        }
        return (static_cast<uint32_t>(pg) << 8) | static_cast<uint32_t>(c % a.c_rows);
      }
      const int s = static_cast<int>(s0) + (v - a.topk);
      const int pg = a.r_bt[static_cast<int64_t>(b) * a.r_bts + s / a.r_rows];
      if (pg < 0 || pg >= a.r_pages) {
        bad |= QLI_DEV_BAD_PAGE;
        return kNoEntry;
      }
      return 0x80000000u | (static_cast<uint32_t>(pg) << 8) | static_cast<uint32_t>(s % a.r_rows);
    };
    uint32_t cnt = 0;
    for (int v = v0; v < v1; ++v) cnt += resolve(v) != kNoEntry ? 1u : 0u;
    uint32_t total;
    uint32_t at = block_exclusive_scan_attn(cnt, &total, scan);
    for (int v = v0; v < v1; ++v) {
      const uint32_t en = resolve(v);
      if (en != kNoEntry) ent[at++] = en;
    }
    if (bad) flag(a, bad);
    E = static_cast<int>(total);
  }
  __syncthreads();

  // 2. the tiles: wave pair pi = wave / 2 takes tiles pi, pi + 2, ...; both
  // waves of a pair score every tile of the pair (the logits of all 16
  // heads) and each keeps the outputs of half the dims, dims
  // 256 eta .. + 255 (eta = wave % 2), so that its accumulators fit the
  // registers.  A pair's tiles alternate between two LDS buffers; each
  // wave stages 8 of a tile's 16 rows.  One workgroup barrier per step.
  const int pi = wave >> 1, eta = wave & 1;
  const int ntiles = (E + kTile - 1) / kTile;
  const int nsteps = (ntiles + 1) / 2;
  float m_run = -INFINITY, l_run = 0.0f;
  constexpr int kOT = kD / 2 / 16;  // output tiles of a wave: 16
  f4 o[kOT];
#pragma unroll
  for (int mt = 0; mt < kOT; ++mt) o[mt] = f4{0.0f, 0.0f, 0.0f, 0.0f};
  auto kbuf = [&](int step) { return lds + (pi * 2 + (step & 1)) * kWaveLds; };

  // this wave's 8 rows of tile k (lane: 16 bytes `lane` of each row),
  // issued together; rows past E read the last entry again (scored as absent)
  auto load = [&](int k, i4 (&rr)[kTile / 2]) {
#pragma unroll
    for (int i = 0; i < kTile / 2; ++i) {
      const int e = min(kTile * k + 8 * eta + i, E - 1);
      const uint32_t en = __builtin_amdgcn_readfirstlane(ent[e]);
      const bool raw = (en >> 31) != 0;
      const char* base = raw ? a.r_cache : a.c_cache;
      const int64_t stride = raw ? a.r_stride : a.c_stride;
      const char* row = base + static_cast<int64_t>((en >> 8) & 0x7FFFFFu) * stride + (en & 0xFFu) * (kD * 2);
      rr[i] = *reinterpret_cast<const i4*>(row + 16 * lane);
    }
  };
  // the rows into both LDS copies of the tile: row-major and transposed
  // (lane holds dims 8 lane .. + 7 of its 8 rows: per dim one 16-byte half,
  // one dword per row pair)
  auto stage = [&](char* kt, const i4 (&rr)[kTile / 2]) {
    const int ln = opaque_lane();
    char* vt = kt + kTile * kD * 2;
#pragma unroll
    for (int i = 0; i < kTile / 2; ++i) *reinterpret_cast<i4*>(kt + krm_offset(8 * eta + i, ln)) = rr[i];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int w = e >> 1;
      const uint32_t sel = (e & 1) ? 0x07060302u : 0x05040100u;
      i4 hv;
#pragma unroll
      for (int j = 0; j < 4; ++j)
        hv[j] = static_cast<int>(__builtin_amdgcn_perm(static_cast<uint32_t>(rr[2 * j + 1][w]),
                                                       static_cast<uint32_t>(rr[2 * j][w]), sel));
      *reinterpret_cast<i4*>(vt + vt_offset(8 * ln + e, eta)) = hv;
    }
  };
  // score one staged tile of n rows (every wave: all 16 heads' logits; its
  // half of the dims for the outputs)
  auto score = [&](const char* kt, int n) {
    const int ln = opaque_lane();
    const char* vt = kt + kTile * kD * 2;
    f4 sacc = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int kg = 0; kg < kD / 32; kg += 4) {  // four k-steps per group: bounded operand prefetch
#pragma unroll
      for (int ks = kg; ks < kg + 4; ++ks) {
        const int ch = 4 * ks + (ln >> 4);
        const i4 kv = *reinterpret_cast<const i4*>(kt + krm_offset(ln & 15, ch));
        const i4 qv = *reinterpret_cast<const i4*>(qs + krm_offset(ln & 15, ch));
        sacc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf8, kv), __builtin_bit_cast(bf8, qv),
                                                       sacc, 0, 0, 0);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
    // sacc[i]: head lane % 16, row 4 (lane / 16) + i
    float z[4];
    float tmax = -INFINITY;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      z[i] = 4 * (lane >> 4) + i < n ? sacc[i] * a.zscale : -INFINITY;
      tmax = fmaxf(tmax, z[i]);
    }
    tmax = wave_max_heads(tmax);
    const float m_new = fmaxf(m_run, tmax);
    const float alpha = m_new == -INFINITY ? 1.0f : exp2f(m_run - m_new);
    uint32_t pb[4];
    float psum = 0.0f;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float pw = z[i] == -INFINITY ? 0.0f : exp2f(z[i] - m_new);
      pb[i] = bf16_rne(pw);
      psum += __uint_as_float(pb[i] << 16);
    }
    l_run = l_run * alpha + psum;
    m_run = m_new;
    const s4 pv = {static_cast<short>(pb[0]), static_cast<short>(pb[1]), static_cast<short>(pb[2]),
                   static_cast<short>(pb[3])};
    const int r0 = 4 * (ln >> 4);
#pragma unroll
    for (int mg = 0; mg < kOT; mg += 8) {  // eight output tiles per group
      i2 vv[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const int d = (kD / 2) * eta + 16 * (mg + j) + (ln & 15);
        vv[j] = *reinterpret_cast<const i2*>(vt + vt_offset(d, r0 >> 3) + (r0 & 7) * 2);
      }
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        o[mg + j] *= alpha;
        o[mg + j] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(s4, vv[j]), pv, o[mg + j], 0, 0, 0);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
  };

  {
    i4 rr[kTile / 2];
    int k = pi;  // this pair's tile of the current step
    if (k < ntiles) load(k, rr);
    for (int step = 0; step < nsteps; ++step) {
      if (k < ntiles) stage(kbuf(step), rr);
      __syncthreads();  // the step's tiles are staged (and the buffers of two steps ago are free)
      const int kn = k + 2;
      if (kn < ntiles) load(kn, rr);
      if (k < ntiles) score(kbuf(step), min(kTile, E - kTile * k));
      k = kn;
    }
  }

  // 3. the pairs' states meet in LDS (over the tile buffers)
  l_run = wave_sum_heads(l_run);
  __syncthreads();  // every wave is done with the tile buffers
  float* mo = reinterpret_cast<float*>(lds);  // [pair][head][D]
  float* ml = reinterpret_cast<float*>(lds + kMiscOff + 256);  // [pair][head]: m, then l
#pragma unroll
  for (int mt = 0; mt < kOT; ++mt) {
    const int d0 = (kD / 2) * eta + 16 * mt + 4 * (lane >> 4);
    *reinterpret_cast<f4*>(mo + (pi * kHeadsWG + (lane & 15)) * kD + d0) = o[mt];
  }
  if (eta == 0 && lane < 16) {
    ml[pi * kHeadsWG + lane] = m_run;
    ml[64 + pi * kHeadsWG + lane] = l_run;
  }
  __syncthreads();
  {
    const int h = tid >> 4;          // head within the group
    const int d0 = 32 * (tid & 15);  // 32 outputs
    const bool has_sink = a.sinks != nullptr && b >= 0;  // a token outside every request: 0, -inf
    const float sk = has_sink ? a.sinks[kHeadsWG * g + h] * kLog2e : -INFINITY;
    float M = sk;
#pragma unroll
    for (int q2 = 0; q2 < 2; ++q2) M = fmaxf(M, ml[q2 * kHeadsWG + h]);
    float cw[2];
    float den = 0.0f;
#pragma unroll
    for (int q2 = 0; q2 < 2; ++q2) {
      const float mw = ml[q2 * kHeadsWG + h];
      cw[q2] = mw == -INFINITY ? 0.0f : exp2f(mw - M);
      den += cw[q2] * ml[64 + q2 * kHeadsWG + h];
    }
    if (has_sink) den += exp2f(sk - M);
    const float inv = den > 0.0f ? 1.0f / den : 0.0f;
    uint16_t* orow = a.out + (static_cast<int64_t>(t) * a.H + kHeadsWG * g + h) * kD + d0;
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      i4 pk;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        uint32_t two[2];
#pragma unroll
        for (int u = 0; u < 2; ++u) {
          const int d = d0 + 8 * v + 2 * j + u;
          float acc = 0.0f;
#pragma unroll
          for (int q2 = 0; q2 < 2; ++q2) acc += cw[q2] * mo[(q2 * kHeadsWG + h) * kD + d];
          two[u] = bf16_rne(acc * inv);
        }
        pk[j] = static_cast<int>(two[0] | (two[1] << 16));
      }
      *reinterpret_cast<i4*>(orow + 8 * v) = pk;
    }
    if (a.lse && (tid & 15) == 0)
      a.lse[static_cast<int64_t>(t) * a.H + kHeadsWG * g + h] = den > 0.0f ? (M + log2f(den)) * kLn2 : -INFINITY;
  }
}

}  // namespace

int launch_attention(const qli_attn_params* p, void* stream) {
  if (p->num_tokens == 0) return QLI_OK;
  AttnArgs a{};
  a.H = p->num_heads;
  a.B = p->batch;
  a.T = p->num_tokens;
  a.topk = p->topk;
  a.window = p->window;
  a.c_rows = p->c_page_rows;
  a.c_bts = p->c_bt_stride;
  a.r_rows = p->window > 0 ? p->r_page_rows : 1;
  a.r_bts = p->window > 0 ? p->r_bt_stride : 1;
  a.G = p->num_heads / kHeadsWG;
  a.c_pages = p->c_num_pages;
  a.r_pages = p->window > 0 ? p->r_num_pages : 0;
  a.c_stride = p->c_page_stride;
  a.r_stride = p->window > 0 ? p->r_page_stride : 0;
  a.zscale = p->scale * kLog2e;
  a.q = static_cast<const uint16_t*>(p->q);
  a.c_cache = static_cast<const char*>(p->c_cache);
  a.c_bt = p->c_block_table;
  a.c_lens = p->c_lens;
  a.r_cache = static_cast<const char*>(p->r_cache);
  a.r_bt = p->r_block_table;
  a.r_lens = p->r_lens;
  a.qsl = p->query_start_loc;
  a.idx = p->indices;
  a.sinks = p->sinks;
  a.out = static_cast<uint16_t*>(p->out);
  a.lse = p->lse;
  a.status = p->status_out;
  hipStream_t st = static_cast<hipStream_t>(stream);
  const int64_t tpad = (static_cast<int64_t>(a.T) + 7) / 8 * 8;
  const int64_t grid = tpad * a.G;
  {
    Stamp s(QLI_KERNEL_ATTN, st);
    hipLaunchKernelGGL(sparse_attn_kernel, dim3(static_cast<unsigned>(grid)), dim3(kAttnThreads), 0, st, a);
  }
  return hipGetLastError() == hipSuccess ? QLI_OK : QLI_ERR_HIP;
}

}  // namespace qli
