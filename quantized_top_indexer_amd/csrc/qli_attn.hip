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
//   2. Four pairs of waves (eight waves, two per SIMD) take every fourth
//      tile of 16 entries; both waves of a pair score every tile of the
//      pair (the 16 heads' logits, queries held in registers) and keep their
//      own online softmax, each for the outputs of half the dims.  A tile's
//      rows go into the pair's LDS buffer twice, row-major (keys: A operand
//      of S^T = K Q^T, 16x16x32 BF16 MFMAs over D = 512) and transposed
//      (values: A operand of O^T = V^T P^T, 16x16x16 BF16 MFMAs).  The S^T
//      accumulator of lane l holds head l % 16 for rows 4 (l / 16) .. + 3,
//      which is exactly the B operand P^T needs, so the weights never leave
//      their lanes.  The rows of two steps ahead are in flight in registers
//      while a step is scored.
//   3. The four pairs' states meet in LDS; each thread writes 16 outputs of
//      one head.
// Keys and values are the same cache entry (one shared latent KV head).
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <algorithm>

#include "qli.h"
#include "qli_internal.h"

namespace qli {
namespace {

constexpr int kD = 512;               // head dim (key and value width)
constexpr int kHeadsWG = 16;          // heads per workgroup
constexpr int kAttnThreads = 512;     // eight waves: four pairs
constexpr int kTile = 16;             // entries per wave tile
constexpr int kMaxEntries = QLI_ATTN_MAX_TOPK + QLI_ATTN_MAX_WINDOW;
constexpr int kWaveLds = 2 * kTile * kD * 2;  // one tile buffer: row-major and transposed copies, 32 KB
constexpr int kPairs = kAttnThreads / 128;   // wave pairs, one tile buffer each
constexpr int kQOff = kPairs * kWaveLds;      // end of the tile buffers
constexpr int kEntOff = kQOff;                // entries (4 bytes each)
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
typedef float f2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf2 __attribute__((ext_vector_type(2)));

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
  // the split kernel: splits per token, blocks of 64 heads, partial states
  // [T][HB][S][64] (m, l) and [T][HB][S][64][D]
  int S, HB;
  float* wml;
  float* wo;
};

__device__ __forceinline__ void flag(const AttnArgs& a, uint32_t bits) {
  if (a.status) atomicOr(a.status, bits);
}

// BF16 of an FP32 value, round to nearest even (finite inputs).
__device__ __forceinline__ uint32_t bf16_rne(float x) {
  const uint32_t u = __float_as_uint(x);
  return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}

// Maximum and sum over the lanes that hold one head (l, l ^ 16, l ^ 32,
// l ^ 48) with the lane swaps of gfx950 (VALU, no LDS round trip): a swap of
// a register with itself across halves (rows) leaves each lane its own value
// in one result and its partner's (lane ^ 32, lane ^ 16) in the other.
__device__ __forceinline__ float wave_max_heads_swap(float x) {
  const auto r32 = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = fmaxf(__uint_as_float(r32[0]), __uint_as_float(r32[1]));
  const auto r16 = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r16[0]), __uint_as_float(r16[1]));
}
__device__ __forceinline__ float wave_sum_heads_swap(float x) {
  const auto r32 = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = __uint_as_float(r32[0]) + __uint_as_float(r32[1]);
  const auto r16 = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r16[0]) + __uint_as_float(r16[1]);
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

// The entries of token t, resolved through both block tables and compacted
// in order into ent (index positions first, then the window), padded with
// copies of the last entry to a multiple of `pad`; returns their count and
// the token's request in *b_out (-1: outside every request).  Called by all
// kAttnThreads threads of the workgroup.  Virtual entry v (index slot v,
// then window position v - topk) belongs to thread v % kAttnThreads, round
// v / kAttnThreads.  Three dependent global round trips: the token's index
// values (with the request search); the request's lengths with the
// block-table entries of the index values; the window's block-table entries.
// The rounds are then compacted in order with wave ballots (scan: 8 words
// per round).
constexpr int kRounds = (kMaxEntries + kAttnThreads - 1) / kAttnThreads;
__device__ int token_entries(const AttnArgs& a, int t, uint32_t* ent, int* misc, uint32_t* scan, int pad,
                             int* b_out) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  // index values (slots past the row read its last slot, unused)
  int c[kRounds];
#pragma unroll
  for (int i = 0; i < kRounds; ++i) {
    const int v = tid + kAttnThreads * i;
    c[i] = a.topk > 0 ? a.idx[static_cast<int64_t>(t) * a.topk + min(v, a.topk - 1)] : -1;
  }
  if (tid == 0) misc[0] = -1;
  __syncthreads();
  for (int i = tid; i < a.B; i += kAttnThreads)
    if (a.qsl[i] <= t && t < a.qsl[i + 1]) misc[0] = i;
  __syncthreads();
  const int b = misc[0];
  *b_out = b;
  int E = 0;
  if (b >= 0) {
    const int q0 = a.qsl[b], q1 = a.qsl[b + 1];
    const int64_t cmax = static_cast<int64_t>(a.c_bts) * a.c_rows, rmax = static_cast<int64_t>(a.r_bts) * a.r_rows;
    const int32_t* crow = a.c_bt + static_cast<int64_t>(b) * a.c_bts;
    // block-table entries of the index values that the table row maps (the
    // length checks come after; other slots read the row's first entry)
    int pgc[kRounds];
#pragma unroll
    for (int i = 0; i < kRounds; ++i) pgc[i] = crow[c[i] >= 0 && c[i] < cmax ? c[i] / a.c_rows : 0];
    // lengths beyond what the request's block-table row can map are cut there
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
    const int nv = a.topk + nwin;
    const int32_t* rrow = a.window > 0 ? a.r_bt + static_cast<int64_t>(b) * a.r_bts : crow;
    int pg[kRounds], row[kRounds];
    bool raw[kRounds];
    uint32_t bad = 0;
#pragma unroll
    for (int i = 0; i < kRounds; ++i) {
      const int v = tid + kAttnThreads * i;
      raw[i] = v >= a.topk;
      if (!raw[i]) {
        if (c[i] >= clen) bad |= QLI_DEV_BAD_INDEX;
        row[i] = c[i] >= 0 && c[i] < clen ? c[i] % a.c_rows : -1;
        pg[i] = pgc[i];
      } else {
        const int pos = v < nv ? static_cast<int>(s0) + (v - a.topk) : -1;
        row[i] = pos >= 0 ? pos % a.r_rows : -1;
        pg[i] = rrow[pos >= 0 ? pos / a.r_rows : 0];
      }
    }
    // compaction, round by round in order
    uint32_t base = 0;
#pragma unroll
    for (int i = 0; i < kRounds; ++i) {
      uint32_t en = kNoEntry;
      if (row[i] >= 0) {
        if (pg[i] < 0 || pg[i] >= (raw[i] ? a.r_pages : a.c_pages)) {
          bad |= QLI_DEV_BAD_PAGE;
        } else {
          en = (raw[i] ? 0x80000000u : 0u) | (static_cast<uint32_t>(pg[i]) << 8) | static_cast<uint32_t>(row[i]);
        }
      }
      const uint64_t m = __ballot(en != kNoEntry);
      const uint32_t within = static_cast<uint32_t>(__popcll(m & ((1ull << lane) - 1ull)));
      if (lane == 0) scan[8 * i + wave] = static_cast<uint32_t>(__popcll(m));
      __syncthreads();
      uint32_t before = base, tot = 0;
#pragma unroll
      for (int w = 0; w < kAttnThreads / 64; ++w) {
        const uint32_t x = scan[8 * i + w];
        before += w < wave ? x : 0u;
        tot += x;
      }
      if (en != kNoEntry) ent[before + within] = en;
      base += tot;
    }
    if (bad) flag(a, bad);
    E = static_cast<int>(base);
  }
  __syncthreads();
  // the last tile is padded with copies of the last entry (scored as absent),
  // so that a wave reads its entries of a tile with vector loads
  if (E > 0 && tid < pad) {
    const uint32_t last = ent[E - 1];
    if (E + tid < (E + pad - 1) / pad * pad) ent[E + tid] = last;
  }
  __syncthreads();
  return E;
}

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
  int* misc = reinterpret_cast<int*>(lds + kMiscOff);
  uint32_t* scan = reinterpret_cast<uint32_t*>(misc + 16);

  // the queries of the workgroup's 16 heads (every wave scores all 16), as
  // B operands of S^T: lane l holds head 16 g + l % 16, dims
  // 32 ks + 8 (l / 16) .. + 7
  bf8 qf[kD / 32];
  {
    const uint16_t* qrow = a.q + (static_cast<int64_t>(t) * a.H + kHeadsWG * g + (lane & 15)) * kD + 8 * (lane >> 4);
#pragma unroll
    for (int ks = 0; ks < kD / 32; ++ks) qf[ks] = __builtin_bit_cast(bf8, *reinterpret_cast<const i4*>(qrow + 32 * ks));
  }

  // 1. request, raw position and the entry list
  int b;
  const int E = token_entries(a, t, ent, misc, scan, kTile, &b);

  // 2. the tiles: wave pair pi = wave / 2 takes tiles pi, pi + 4, ...; both
  // waves of a pair score every tile of the pair (the logits of all 16
  // heads) and each keeps the outputs of half the dims, dims
  // 256 eta .. + 255 (eta = wave % 2), so that its accumulators fit the
  // registers of two waves per SIMD.  Each pair has one LDS tile buffer;
  // each wave stages 8 of a tile's 16 rows.  Two workgroup barriers per
  // step (tiles staged; tiles scored).
  const int pi = wave >> 1, eta = wave & 1;
  const int ntiles = (E + kTile - 1) / kTile;
  const int nsteps = (ntiles + kPairs - 1) / kPairs;
  float m_run = -INFINITY, l_run = 0.0f;
  constexpr int kOT = kD / 2 / 16;  // output tiles of a wave: 16
  f4 o[kOT];
#pragma unroll
  for (int mt = 0; mt < kOT; ++mt) o[mt] = f4{0.0f, 0.0f, 0.0f, 0.0f};
  char* const kbuf = lds + pi * kWaveLds;

  // this wave's 8 rows of tile k (lane: 16 bytes `lane` of each row),
  // issued together (rows past E repeat the last entry, scored as absent)
  auto load = [&](int k, i4 (&rr)[kTile / 2]) {
    const i4 e0 = *reinterpret_cast<const i4*>(ent + kTile * k + 8 * eta);
    const i4 e1 = *reinterpret_cast<const i4*>(ent + kTile * k + 8 * eta + 4);
#pragma unroll
    for (int i = 0; i < kTile / 2; ++i) {
      const uint32_t en = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(i < 4 ? e0[i] : e1[i - 4]));
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
    // two independent accumulator chains (even and odd k-steps) halve the
    // dependent MFMA latency
    f4 sa = {0.0f, 0.0f, 0.0f, 0.0f}, sb = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int ks = 0; ks < kD / 32; ks += 2) {
      const int ch = 4 * ks + (ln >> 4);
      const i4 kv0 = *reinterpret_cast<const i4*>(kt + krm_offset(ln & 15, ch));
      const i4 kv1 = *reinterpret_cast<const i4*>(kt + krm_offset(ln & 15, ch + 4));
      sa = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf8, kv0), qf[ks], sa, 0, 0, 0);
      sb = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf8, kv1), qf[ks + 1], sb, 0, 0, 0);
    }
    const f4 sacc = sa + sb;
    // sacc[i]: head lane % 16, row 4 (lane / 16) + i
    float z[4];
    float tmax = -INFINITY;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      z[i] = 4 * (lane >> 4) + i < n ? sacc[i] * a.zscale : -INFINITY;
      tmax = fmaxf(tmax, z[i]);
    }
    tmax = wave_max_heads_swap(tmax);
    // The weights are taken against a reference maximum m_run that moves
    // only when a head's logits pass it by more than 8 (weights below 2^8,
    // exact as BF16 exponents and harmless in the FP32 sums): the output
    // accumulators are rescaled on those few tiles only (a wave-uniform
    // branch), so the matrix core keeps them the rest of the time.
    const float m_cand = fmaxf(m_run, tmax);
    if (__ballot(m_cand > m_run + 8.0f) != 0) {
      const float alpha = m_cand == -INFINITY ? 1.0f : exp2f(m_run - m_cand);
#pragma unroll
      for (int mt = 0; mt < kOT; ++mt) o[mt] *= alpha;
      l_run *= alpha;
      m_run = m_cand;
    }
    // m_run is finite here (every tile holds a valid entry): z = -inf gives
    // weight 0 through the hardware exponential
    const bf2 w01 = __builtin_convertvector(
        (f2{__builtin_amdgcn_exp2f(z[0] - m_run), __builtin_amdgcn_exp2f(z[1] - m_run)}), bf2);
    const bf2 w23 = __builtin_convertvector(
        (f2{__builtin_amdgcn_exp2f(z[2] - m_run), __builtin_amdgcn_exp2f(z[3] - m_run)}), bf2);
    const uint32_t u01 = __builtin_bit_cast(uint32_t, w01), u23 = __builtin_bit_cast(uint32_t, w23);
    l_run += (__uint_as_float(u01 << 16) + __uint_as_float(u01 & 0xFFFF0000u)) +
             (__uint_as_float(u23 << 16) + __uint_as_float(u23 & 0xFFFF0000u));
    const s4 pv = __builtin_bit_cast(s4, i2{static_cast<int>(u01), static_cast<int>(u23)});
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
      for (int j = 0; j < 8; ++j)
        o[mg + j] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(s4, vv[j]), pv, o[mg + j], 0, 0, 0);
      __builtin_amdgcn_sched_barrier(0);
    }
  };

  {
    // a ring of two register sets: the rows of step s + 2 are loaded while
    // step s is scored.  Every load is issued unconditionally (a tile past
    // the end reads the last tile again), so that the compiler's memory
    // counters stay exact and staging a set waits for that set's loads only.
    i4 r0[kTile / 2], r1[kTile / 2];
    auto step_body = [&](int step, i4 (&rr)[kTile / 2]) {
      const bool live = step < nsteps;  // workgroup-uniform
      const int k = pi + kPairs * step; // this pair's tile of the step
      if (live && k < ntiles) stage(kbuf, rr);
      if (live) __syncthreads();  // the step's tiles are staged
      __builtin_amdgcn_sched_barrier(0);  // the sets' loads stay in issue order
      load(min(k + 2 * kPairs, ntiles - 1), rr);
      __builtin_amdgcn_sched_barrier(0);
      if (live && k < ntiles) score(kbuf, min(kTile, E - kTile * k));
      if (live) __syncthreads();  // the step's tiles are scored: the buffers are free
    };
    if (ntiles > 0) {
      load(min(pi, ntiles - 1), r0);
      __builtin_amdgcn_sched_barrier(0);
      load(min(pi + kPairs, ntiles - 1), r1);
      __builtin_amdgcn_sched_barrier(0);
      for (int step = 0; step < nsteps; step += 2) {
        step_body(step, r0);
        step_body(step + 1, r1);
      }
    }
  }

  // 3. the pairs' states meet in LDS (over the tile buffers)
  l_run = wave_sum_heads_swap(l_run);
  __syncthreads();  // every wave is done with the tile buffers
  float* mo = reinterpret_cast<float*>(lds);  // [pair][head][D]
  float* ml = reinterpret_cast<float*>(lds + kMiscOff + 256);  // [pair][head]: m, then l
  static_assert(kPairs * kHeadsWG * kD * 4 <= kQOff, "pair outputs over the tile buffers");
#pragma unroll
  for (int mt = 0; mt < kOT; ++mt) {
    const int d0 = (kD / 2) * eta + 16 * mt + 4 * (lane >> 4);
    *reinterpret_cast<f4*>(mo + (pi * kHeadsWG + (lane & 15)) * kD + d0) = o[mt];
  }
  if (eta == 0 && lane < 16) {
    ml[pi * kHeadsWG + lane] = m_run;
    ml[kPairs * kHeadsWG + pi * kHeadsWG + lane] = l_run;
  }
  __syncthreads();
  {
    constexpr int kPer = kHeadsWG * kD / kAttnThreads;  // outputs per thread: 16
    const int h = tid / (kD / kPer);                    // head within the group
    const int d0 = kPer * (tid % (kD / kPer));
    const bool has_sink = a.sinks != nullptr && b >= 0;  // a token outside every request: 0, -inf
    const float sk = has_sink ? a.sinks[kHeadsWG * g + h] * kLog2e : -INFINITY;
    float M = sk;
#pragma unroll
    for (int q2 = 0; q2 < kPairs; ++q2) M = fmaxf(M, ml[q2 * kHeadsWG + h]);
    float cw[kPairs];
    float den = 0.0f;
#pragma unroll
    for (int q2 = 0; q2 < kPairs; ++q2) {
      const float mw = ml[q2 * kHeadsWG + h];
      cw[q2] = mw == -INFINITY ? 0.0f : exp2f(mw - M);
      den += cw[q2] * ml[kPairs * kHeadsWG + q2 * kHeadsWG + h];
    }
    if (has_sink) den += exp2f(sk - M);
    const float inv = den > 0.0f ? 1.0f / den : 0.0f;
    uint16_t* orow = a.out + (static_cast<int64_t>(t) * a.H + kHeadsWG * g + h) * kD + d0;
#pragma unroll
    for (int v = 0; v < kPer / 8; ++v) {
      i4 pk;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        uint32_t two[2];
#pragma unroll
        for (int u = 0; u < 2; ++u) {
          const int d = d0 + 8 * v + 2 * j + u;
          float acc = 0.0f;
#pragma unroll
          for (int q2 = 0; q2 < kPairs; ++q2) acc += cw[q2] * mo[(q2 * kHeadsWG + h) * kD + d];
          two[u] = bf16_rne(acc * inv);
        }
        pk[j] = static_cast<int>(two[0] | (two[1] << 16));
      }
      *reinterpret_cast<i4*>(orow + 8 * v) = pk;
    }
    if (a.lse && d0 == 0)
      a.lse[static_cast<int64_t>(t) * a.H + kHeadsWG * g + h] = den > 0.0f ? (M + log2f(den)) * kLn2 : -INFINITY;
  }
}


// ---------------------------------------------------------------------------
// All 64 heads of a block in one workgroup; a token's entries split over S
// workgroups whose partial softmax states meet in a workspace.
//
// Workgroup (token t, head block hb, split s): steps of 32 entries, split s
// taking steps [N s / S, N (s + 1) / S) of the token's N, so each row is
// loaded and staged into LDS once for all 64 heads (the head-group kernel
// above stages every row once per 16 heads).  Eight waves: wave w scores
// half eta = w / 4 of a step (entries 16 eta .. + 15) for head group
// hg = w % 4 and keeps the outputs of dims 256 eta .. + 255 of those 16
// heads; the two waves of a head group trade their logits through LDS, so
// both see all 32 logits of a step and take identical softmax decisions.
// O^T = V^T P^T runs as 16x16x32 MFMAs over the whole step: k slot
// 8 (l / 16) + j of lane l stands for entry 4 (l / 16) + j of the first
// half (j < 4) or of the second (j >= 4), which is where the S^T
// accumulators of the two halves hold their logits.  The step's rows sit
// in LDS twice, row-major (keys) and transposed (values), in two buffers:
// a step is staged while the previous one is scored, one barrier after
// staging and one for the logit exchange.  With S > 1 each workgroup writes
// its softmax state (outputs relative to its maximum, maximum, normalizer)
// to the workspace and a second launch merges a token's states; with S = 1
// the workgroup writes the outputs itself.

constexpr int kStepE = 32;                        // entries per step
constexpr int kSplitBuf = 2 * kStepE * kD * 2;   // one step: keys, then values: 64 KB
constexpr int kSZOff = 2 * kSplitBuf;             // logits exchange: 8 waves x 64 lanes x 16 B
constexpr int kSEntOff = kSZOff + 8 * 64 * 16;
constexpr int kSMiscOff = kSEntOff + kMaxEntries * 4;
constexpr int kSLdsBytes = kSMiscOff + 1024;
constexpr int kMaxSplits = 4;
static_assert(kSLdsBytes <= 160 * 1024, "LDS of one workgroup");
static_assert(kMaxEntries % kStepE == 0, "padded entry lists fit");

// Transposed step layout: the values of dim d for entry quads c and c + 4
// (entries 4c .. 4c + 3 and 16 + 4c .. + 3) share a 16-byte slot; quad half
// h sits at byte 8 (h ^ bit 6 of d).  The slots of eight consecutive dims
// (one MFMA operand load of eight lanes) and of the dims 8 apart written by
// one store instruction fall on distinct LDS banks.
__device__ __forceinline__ int vts_slot(int d, int c) {
  return ((((d >> 3) << 2) + c) << 7) + (((d ^ (d >> 3) ^ c) & 7) << 4);
}

// Row-major step layout: chunk ch (16 B) of row i at chunk ch ^ (i % 16), so
// the 16 rows of one key operand load fall on distinct banks.  That load
// (rows 16 eta + l % 16, chunks 8 k + 4 h + l / 16) is a per-lane base for
// h and the parity of k plus 128 k bytes, an immediate offset.
__device__ __forceinline__ int krs_offset(int i, int ch) { return i * (kD * 2) + ((ch ^ (i & 15)) << 4); }

__global__ __launch_bounds__(kAttnThreads, 1) void sparse_attn_split_kernel(AttnArgs a) {
  __shared__ __attribute__((aligned(16))) char lds[kSLdsBytes];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  // workgroup -> (token, head block, split); the workgroups of a token share
  // i mod 8 (one XCD)
  const int U = a.HB * a.S;
  const int x = blockIdx.x & 7, r = blockIdx.x >> 3;
  const int u = r % U;
  const int t = x + 8 * (r / U);
  if (t >= a.T) return;
  const int hb = u / a.S, s = u % a.S;
  const int hg = wave & 3, eta = wave >> 2;
  const int h = 64 * hb + 16 * hg + (lane & 15);  // this lane's head
  uint32_t* ent = reinterpret_cast<uint32_t*>(lds + kSEntOff);
  int* misc = reinterpret_cast<int*>(lds + kSMiscOff);
  uint32_t* scan = reinterpret_cast<uint32_t*>(misc + 16);
  f4* zx = reinterpret_cast<f4*>(lds + kSZOff);  // [wave][lane]

  // the queries of the wave's 16 heads as B operands of S^T: lane l holds
  // dims 32 ks + 8 (l / 16) .. + 7 of head h
  bf8 qf[kD / 32];
  {
    const uint16_t* qrow = a.q + (static_cast<int64_t>(t) * a.H + h) * kD + 8 * (lane >> 4);
#pragma unroll
    for (int ks = 0; ks < kD / 32; ++ks) qf[ks] = __builtin_bit_cast(bf8, *reinterpret_cast<const i4*>(qrow + 32 * ks));
  }

  int b;
  const int E = token_entries(a, t, ent, misc, scan, kStepE, &b);
  const int N = (E + kStepE - 1) / kStepE;
  const int st0 = static_cast<int>(static_cast<int64_t>(N) * s / a.S);
  const int st1 = static_cast<int>(static_cast<int64_t>(N) * (s + 1) / a.S);
  const int ns = st1 - st0;

  float m_run = -INFINITY, l_run = 0.0f;
  constexpr int kOT = kD / 2 / 16;  // output tiles of a wave: 16
  f4 o[kOT];
#pragma unroll
  for (int mt = 0; mt < kOT; ++mt) o[mt] = f4{0.0f, 0.0f, 0.0f, 0.0f};

  // this wave's 4 rows of step k (entries 32 k + 4 wave .. + 3; lane: bytes
  // 16 lane .. + 15 of each row)
  auto load = [&](int k, i4 (&rr)[4]) {
    const i4 e4 = *reinterpret_cast<const i4*>(ent + kStepE * k + 4 * wave);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const uint32_t en = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(e4[i]));
      const bool raw = (en >> 31) != 0;
      const char* base = raw ? a.r_cache : a.c_cache;
      const int64_t stride = raw ? a.r_stride : a.c_stride;
      const char* row = base + static_cast<int64_t>((en >> 8) & 0x7FFFFFu) * stride + (en & 0xFFu) * (kD * 2);
      rr[i] = *reinterpret_cast<const i4*>(row + 16 * lane);
    }
  };
  // the rows into both copies of a step buffer (quad `wave` of the step)
  auto stage = [&](char* kb, const i4 (&rr)[4]) {
    const int ln = opaque_lane();
#pragma unroll
    for (int i = 0; i < 4; ++i) *reinterpret_cast<i4*>(kb + krs_offset(4 * wave + i, ln)) = rr[i];
    // dims 8 ln + e: slot base 512 ln + 128 c, position (ln ^ c ^ e) % 8
    char* vt = kb + kStepE * kD * 2 + 512 * ln + 128 * (wave & 3) + 8 * ((wave >> 2) ^ ((ln >> 3) & 1));
    const int ls = (ln ^ wave) & 3 | (ln & 4);  // (ln ^ c) % 8
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int w = e >> 1;
      const uint32_t sel = (e & 1) ? 0x07060302u : 0x05040100u;
      i2 hv;
      hv[0] = static_cast<int>(__builtin_amdgcn_perm(static_cast<uint32_t>(rr[1][w]), static_cast<uint32_t>(rr[0][w]), sel));
      hv[1] = static_cast<int>(__builtin_amdgcn_perm(static_cast<uint32_t>(rr[3][w]), static_cast<uint32_t>(rr[2][w]), sel));
      *reinterpret_cast<i2*>(vt + ((ls ^ e) << 4)) = hv;
    }
  };
  // per-lane bases of the operand loads (the rest of each address is an
  // immediate): keys, chunk groups h = 0, 1; values, tiles with mt % 4 = k
  // (8 k + 4 h + g) ^ (i % 16) = 8 (k ^ b) + ((4 h + g) ^ (i % 8)) with
  // b = bit 3 of i, and 8 (k ^ b) = 8 k + 8 b for even k, 8 k - 8 b for odd
  int kbase[2][2], vbase[4];
  {
    const int i = 16 * eta + (lane & 15), g = lane >> 4, j = lane & 15;
    const int bq = 128 * ((i >> 3) & 1);
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int rest = i * (kD * 2) + (((4 * h + g) ^ (i & 7)) << 4);
      kbase[0][h] = rest + bq;
      kbase[1][h] = rest - bq;
    }
    const int lv = (j & 7) ^ (j >> 3) ^ g;
#pragma unroll
    for (int k = 0; k < 4; ++k)
      vbase[k] = kStepE * kD * 2 + 16384 * eta + 512 * (j >> 3) + 128 * g + ((lv ^ (2 * k)) << 4);
  }
  // score step k from buffer kb (holds the logit exchange barrier)
  auto score = [&](const char* kb, int k) {
    f4 sa = {0.0f, 0.0f, 0.0f, 0.0f}, sb = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int ks = 0; ks < kD / 32; ks += 2) {
      const int par = (ks >> 1) & 1;  // parity of k = ks / 2
      const i4 kv0 = *reinterpret_cast<const i4*>(kb + kbase[par][0] + 64 * ks);
      const i4 kv1 = *reinterpret_cast<const i4*>(kb + kbase[par][1] + 64 * ks);
      sa = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf8, kv0), qf[ks], sa, 0, 0, 0);
      sb = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf8, kv1), qf[ks + 1], sb, 0, 0, 0);
    }
    const f4 sacc = sa + sb;
    // sacc[i]: head h, entry 32 k + 16 eta + 4 (lane / 16) + i
    f4 zo;
    const int e0 = kStepE * k + 16 * eta + 4 * (lane >> 4);
#pragma unroll
    for (int i = 0; i < 4; ++i) zo[i] = e0 + i < E ? sacc[i] * a.zscale : -INFINITY;
    zx[wave * 64 + lane] = zo;
    __syncthreads();  // both halves' logits are in LDS
    const f4 zp = zx[(wave ^ 4) * 64 + lane];
    const f4 z0 = eta == 0 ? zo : zp, z1 = eta == 0 ? zp : zo;
    float tmax = -INFINITY;
#pragma unroll
    for (int i = 0; i < 4; ++i) tmax = fmaxf(tmax, fmaxf(z0[i], z1[i]));
    tmax = wave_max_heads_swap(tmax);
    // the reference maximum moves only when a head's logits pass it by more
    // than 8 (weights stay below 2^8); both waves of a head group see the
    // same logits and move it together
    const float m_cand = fmaxf(m_run, tmax);
    if (__ballot(m_cand > m_run + 8.0f) != 0) {
      const float alpha = m_cand == -INFINITY ? 1.0f : exp2f(m_run - m_cand);
#pragma unroll
      for (int mt = 0; mt < kOT; ++mt) o[mt] *= alpha;
      l_run *= alpha;
      m_run = m_cand;
    }
    // m_run is finite here (every step holds a valid entry), so z = -inf
    // gives weight 0 through the hardware exponential; weights below 2^-126
    // of the maximum flush to 0
    i4 pa;
    float psum = 0.0f;
#pragma unroll
    for (int i = 0; i < 4; i += 2) {
      const bf2 w0 = __builtin_convertvector(
          (f2{__builtin_amdgcn_exp2f(z0[i] - m_run), __builtin_amdgcn_exp2f(z0[i + 1] - m_run)}), bf2);
      const bf2 w1 = __builtin_convertvector(
          (f2{__builtin_amdgcn_exp2f(z1[i] - m_run), __builtin_amdgcn_exp2f(z1[i + 1] - m_run)}), bf2);
      const uint32_t u0 = __builtin_bit_cast(uint32_t, w0), u1 = __builtin_bit_cast(uint32_t, w1);
      pa[i / 2] = static_cast<int>(u0);
      pa[2 + i / 2] = static_cast<int>(u1);
      psum += (__uint_as_float(u0 << 16) + __uint_as_float(u0 & 0xFFFF0000u)) +
              (__uint_as_float(u1 << 16) + __uint_as_float(u1 & 0xFFFF0000u));
    }
    l_run += psum;
    const i4 pb = {pa[2], pa[3], pa[0], pa[1]};
    const bf8 PA = __builtin_bit_cast(bf8, pa), PB = __builtin_bit_cast(bf8, pb);
#pragma unroll
    for (int mg = 0; mg < kOT; mg += 8) {  // eight output tiles per group
      i4 vv[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        // dims 256 eta + 16 mt + l % 16 (mt = mg + j): vts_slot written as
        // a base per mt % 4 plus 1024 mt
        const int mt = mg + j;
        vv[j] = *reinterpret_cast<const i4*>(kb + vbase[mt & 3] + 1024 * mt);
      }
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        // bit 6 of the tile's dims says which quad the slot holds first
        const int mt = mg + j;
        o[mt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf8, vv[j]), ((mt >> 2) & 1) ? PB : PA,
                                                        o[mt], 0, 0, 0);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
  };

  if (ns > 0) {
    // a ring of two register sets: the rows of step j + 2 are in flight
    // while step j is scored; loads past the split's last step read that
    // step again, so every load is unconditional
    char* const buf0 = lds;
    char* const buf1 = lds + kSplitBuf;
    i4 r0[4], r1[4];
    load(st0, r0);
    __builtin_amdgcn_sched_barrier(0);
    load(min(st0 + 1, st1 - 1), r1);
    __builtin_amdgcn_sched_barrier(0);
    stage(buf0, r0);
    __builtin_amdgcn_sched_barrier(0);
    load(min(st0 + 2, st1 - 1), r0);
    __builtin_amdgcn_sched_barrier(0);
    auto body = [&](int j, const char* cur, char* nxt, i4 (&rr)[4]) {
      const bool live = j < ns;  // workgroup-uniform
      if (live) __syncthreads();  // step j is staged; the logit buffer is free
      if (live) score(cur, st0 + j);
      if (j + 1 < ns) stage(nxt, rr);
      __builtin_amdgcn_sched_barrier(0);
      load(min(st0 + j + 3, st1 - 1), rr);
      __builtin_amdgcn_sched_barrier(0);
    };
    for (int j = 0; j < ns; j += 2) {
      body(j, buf0, buf1, r1);
      body(j + 1, buf1, buf0, r0);
    }
  }
  l_run = wave_sum_heads_swap(l_run);

  if (a.S > 1) {
    // this split's state for the merge launch: o relative to m_run, m_run, l_run
    const int64_t unit = static_cast<int64_t>(t) * a.HB + hb;
    const int hl = 16 * hg + (lane & 15);  // head within the block
    float* wo = a.wo + ((unit * a.S + s) * 64 + hl) * kD;
#pragma unroll
    for (int mt = 0; mt < kOT; ++mt)
      *reinterpret_cast<f4*>(wo + (kD / 2) * eta + 16 * mt + 4 * (lane >> 4)) = o[mt];
    if (eta == 0 && lane < 16) {
      float* wml = a.wml + ((unit * a.S + s) * 64 + hl) * 2;
      wml[0] = m_run;
      wml[1] = b >= 0 ? l_run : -1.0f;  // -1: the token is outside every request
    }
    return;
  }

  // 3. outputs: lane l holds dims 256 eta + 16 mt + 4 (l / 16) .. + 3 of head h
  const bool has_sink = a.sinks != nullptr && b >= 0;  // a token outside every request: 0, -inf
  const float sk = has_sink ? a.sinks[h] * kLog2e : -INFINITY;
  const float M = fmaxf(m_run, sk);
  const float c = m_run == -INFINITY ? 0.0f : exp2f(m_run - M);
  const float den = c * l_run + (has_sink ? exp2f(sk - M) : 0.0f);
  const float f = den > 0.0f ? c / den : 0.0f;
  uint16_t* orow = a.out + (static_cast<int64_t>(t) * a.H + h) * kD + (kD / 2) * eta + 4 * (lane >> 4);
#pragma unroll
  for (int mt = 0; mt < kOT; ++mt) {
    const i2 pk = {static_cast<int>(bf16_rne(o[mt][0] * f) | (bf16_rne(o[mt][1] * f) << 16)),
                   static_cast<int>(bf16_rne(o[mt][2] * f) | (bf16_rne(o[mt][3] * f) << 16))};
    *reinterpret_cast<i2*>(orow + 16 * mt) = pk;
  }
  if (a.lse && eta == 0 && lane < 16)
    a.lse[static_cast<int64_t>(t) * a.H + h] = den > 0.0f ? (M + log2f(den)) * kLn2 : -INFINITY;
}


// The merge of a token's split states: workgroup i takes (token, head
// block) i / 16 and its heads 4 (i % 16) .. + 3; thread: head tid / 128 of
// those, dims 4 (tid % 128) .. + 3.
__global__ __launch_bounds__(kAttnThreads) void sparse_attn_merge_kernel(AttnArgs a) {
  const int unit = blockIdx.x >> 4;  // t * HB + hb
  const int t = unit / a.HB, hb = unit % a.HB;
  const int tid = threadIdx.x;
  const int hl = 4 * (blockIdx.x & 15) + tid / 128;  // head within the block
  const int h = 64 * hb + hl;
  const int d = 4 * (tid % 128);
  const float* wml = a.wml + (static_cast<int64_t>(unit) * a.S * 64 + hl) * 2;
  const float* wo = a.wo + (static_cast<int64_t>(unit) * a.S * 64 + hl) * kD + d;
  float ms[kMaxSplits], ls[kMaxSplits];
  f4 v[kMaxSplits];
#pragma unroll
  for (int s = 0; s < kMaxSplits; ++s) {
    if (s < a.S) {
      ms[s] = wml[s * 128];
      ls[s] = wml[s * 128 + 1];
      v[s] = *reinterpret_cast<const f4*>(wo + static_cast<int64_t>(s) * 64 * kD);
    }
  }
  // a token outside every request (normalizer -1) has no sink term: out 0,
  // lse -inf (its states hold no entry: maximum -inf, weight 0)
  const bool has_sink = a.sinks != nullptr && ls[0] >= 0.0f;
  const float sk = has_sink ? a.sinks[h] * kLog2e : -INFINITY;
  float M = sk;
#pragma unroll
  for (int s = 0; s < kMaxSplits; ++s)
    if (s < a.S) M = fmaxf(M, ms[s]);
  f4 acc = {0.0f, 0.0f, 0.0f, 0.0f};
  float den = has_sink ? exp2f(sk - M) : 0.0f;
#pragma unroll
  for (int s = 0; s < kMaxSplits; ++s) {
    if (s < a.S) {
      const float c = ms[s] == -INFINITY ? 0.0f : exp2f(ms[s] - M);
      den += c * ls[s];
      acc += v[s] * c;
    }
  }
  const float f = den > 0.0f ? 1.0f / den : 0.0f;
  const i2 pk = {static_cast<int>(bf16_rne(acc[0] * f) | (bf16_rne(acc[1] * f) << 16)),
                 static_cast<int>(bf16_rne(acc[2] * f) | (bf16_rne(acc[3] * f) << 16))};
  *reinterpret_cast<i2*>(a.out + (static_cast<int64_t>(t) * a.H + h) * kD + d) = pk;
  if (a.lse && d == 0) a.lse[static_cast<int64_t>(t) * a.H + h] = den > 0.0f ? (M + log2f(den)) * kLn2 : -INFINITY;
}

}  // namespace

int attention_splits(int64_t tokens, int heads, int topk, int window) {
  if (heads % 64 != 0) return 0;
  const int64_t units = tokens * (heads / 64);
  if (units >= 256) return 1;
  int64_t S = std::min<int64_t>(kMaxSplits, (256 + units - 1) / std::max<int64_t>(units, 1));
  const int64_t steps = (static_cast<int64_t>(topk) + window + kStepE - 1) / kStepE;
  S = std::min(S, std::max<int64_t>(steps, 1));
  return static_cast<int>(std::max<int64_t>(S, 1));
}

int64_t attention_workspace_bytes(int64_t tokens, int heads, int /*topk*/, int /*window*/, int splits) {
  if (splits <= 1 || heads % 64 != 0) return 0;
  const int64_t units = tokens * (heads / 64);
  return units * splits * 64 * 2 * 4 + units * splits * 64 * kD * 4;
}

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
  int S = attention_splits(a.T, a.H, a.topk, a.window);
  if (S == 0) {
    const int64_t grid = tpad * a.G;
    Stamp s(QLI_KERNEL_ATTN, st);
    hipLaunchKernelGGL(sparse_attn_kernel, dim3(static_cast<unsigned>(grid)), dim3(kAttnThreads), 0, st, a);
  } else {
    // as many splits as the workspace holds
    const int64_t ws = p->workspace ? p->workspace_bytes : 0;
    while (S > 1 && attention_workspace_bytes(a.T, a.H, a.topk, a.window, S) > ws) --S;
    a.S = S;
    a.HB = a.H / 64;
    const int64_t units = static_cast<int64_t>(a.T) * a.HB;
    if (S > 1) {
      a.wml = static_cast<float*>(p->workspace);
      a.wo = a.wml + units * S * 64 * 2;
    }
    const int64_t grid = tpad * a.HB * S;
    {
      Stamp s(QLI_KERNEL_ATTN_SPLIT, st);
      hipLaunchKernelGGL(sparse_attn_split_kernel, dim3(static_cast<unsigned>(grid)), dim3(kAttnThreads), 0, st, a);
    }
    if (S > 1) {
      Stamp s(QLI_KERNEL_ATTN_MERGE, st);
      hipLaunchKernelGGL(sparse_attn_merge_kernel, dim3(static_cast<unsigned>(units * 16)), dim3(kAttnThreads), 0, st, a);
    }
  }
  return hipGetLastError() == hipSuccess ? QLI_OK : QLI_ERR_HIP;
}

}  // namespace qli
