// Internal declarations shared by the host API and the kernel launcher.
#pragma once

#include <stddef.h>
#include <stdint.h>

#include "qli.h"

namespace qli {

// Carve-up of the caller's workspace for slices of `tokens` query tokens
// (T below): a call is processed slice by slice, each slice reusing the
// whole workspace, so its size is bounded by the slice, not by the call.
//   keys   [T, ncap]    u32 order-preserving score keys by slot (0 = not eligible)
//   bkeys  [T, nbcap]   u32 block-max keys (source mode)
//   plan   header (group counts, work units), groups [2][T] x 32 B, ustart [2][T+1]:
//          the two work lists the plan kernel builds for the persistent score kernel
//   wgs    [kMaxScoreWGs] x 64 B: each score workgroup's list, first item and range
//   tokv   [T, 2]       per token: visible compressed count (written by the plan), and
//                       the launch's epoch where the token met an out-of-contract page
//   slots  [T, cand_in_blocks] sorted unique visible incoming block ids (consumer)
//   srow   [T, cand_in_blocks] page*page_rows + row of each slot block (consumer)
//   ncount [T]          eligible positions per token (consumer)
struct WsLayout {
  int64_t tokens = 0;  // query tokens per slice
  int64_t ncap = 0;
  int64_t nbcap = 0;
  size_t keys_off = 0;
  size_t bkeys_off = 0;
  size_t plan_off = 0;
  size_t groups_off = 0;
  size_t ustart_off = 0;
  size_t wgs_off = 0;
  size_t tokv_off = 0;
  size_t slots_off = 0;
  size_t srow_off = 0;
  size_t ncount_off = 0;
  size_t total = 0;
};

constexpr int kChunk = 256;       // score slots per work item
constexpr int kGroupTokens = 4;   // tokens of one request sharing a K tile (plain/source)
constexpr int kMaxScoreWGs = 2048;  // score grid cap (two workgroups per CU)
constexpr int kWgStartBytes = 64;

inline size_t align256(size_t x) { return (x + 255) & ~static_cast<size_t>(255); }

// Default budget of a slice's workspace: the call is cut into slices of as
// many tokens as fit in it (at least one token per slice).
constexpr int64_t kSliceBudgetBytes = int64_t(4) << 30;

inline WsLayout ws_layout(const qli_params* p, int64_t slice_tokens) {
  WsLayout w;
  w.tokens = slice_tokens;
  const size_t T = static_cast<size_t>(slice_tokens);
  if (p->mode == QLI_MODE_CONSUMER)
    w.ncap = static_cast<int64_t>(p->cand_in_blocks) * 8;
  else
    w.ncap = (static_cast<int64_t>(p->max_k_len) + kChunk - 1) / kChunk * kChunk;
  size_t off = 0;
  w.keys_off = off;
  off = align256(off + T * static_cast<size_t>(w.ncap) * 4);
  if (p->mode == QLI_MODE_SOURCE) {
    // covers every block id below max_k_len and every 8-slot group below ncap
    const int64_t nb = (static_cast<int64_t>(p->max_k_len) + 7) / 8;
    w.nbcap = ((nb > w.ncap / 8 ? nb : w.ncap / 8) + 63) / 64 * 64;
    w.bkeys_off = off;
    off = align256(off + T * static_cast<size_t>(w.nbcap) * 4);
  }
  w.plan_off = off;
  off = align256(off + 256);
  w.groups_off = off;
  off = align256(off + 2 * T * 32);
  w.ustart_off = off;
  off = align256(off + 2 * (T + 1) * 4);
  w.wgs_off = off;
  off = align256(off + static_cast<size_t>(kMaxScoreWGs) * kWgStartBytes);
  w.tokv_off = off;
  off = align256(off + T * 8);
  if (p->mode == QLI_MODE_CONSUMER) {
    const size_t cb = static_cast<size_t>(p->cand_in_blocks);
    w.slots_off = off;
    off = align256(off + T * cb * 4);
    w.srow_off = off;
    off = align256(off + T * cb * 4);
    w.ncount_off = off;
    off = align256(off + T * 4);
  }
  w.total = off;
  return w;
}

// The layout of the largest slice (at most num_tokens, at least one token)
// whose workspace fits in `bytes`; tokens = 0 when not even one token fits.
inline WsLayout slice_layout(const qli_params* p, size_t bytes) {
  const int64_t T = p->num_tokens;
  if (T <= 0 || ws_layout(p, T).total <= bytes) return ws_layout(p, T > 0 ? T : 0);
  if (ws_layout(p, 1).total > bytes) return WsLayout{};
  int64_t lo = 1, hi = T;  // ws_layout(lo) fits, ws_layout(hi) does not
  while (hi - lo > 1) {
    const int64_t mid = lo + (hi - lo) / 2;
    if (ws_layout(p, mid).total <= bytes) lo = mid;
    else hi = mid;
  }
  return ws_layout(p, lo);
}

// The workspace qli_workspace_bytes() recommends: the whole call when it
// fits in kSliceBudgetBytes, otherwise the largest slice that does.
inline WsLayout default_layout(const qli_params* p) {
  const WsLayout full = ws_layout(p, p->num_tokens);
  if (full.total <= static_cast<size_t>(kSliceBudgetBytes)) return full;
  const WsLayout w = slice_layout(p, static_cast<size_t>(kSliceBudgetBytes));
  return w.tokens > 0 ? w : ws_layout(p, 1);
}

// Enqueue the kernels (arguments already validated), slice by slice of
// w.tokens query tokens.  timed: record the optional timing events (when
// the timing facility is on).
int launch(const qli_params* p, const WsLayout& w, void* stream, bool timed);

// Device address of the library's static scratch array on the current
// device (looked up once per device); a qli_status.
int static_scratch(void** ptr);

int timing_enable(int on);
int timing_read(double* ms, int64_t* count, int reset);

// While timing is enabled, records a HIP event on `stream` at construction
// and another at destruction, queued for timing_read() under `kernel`.
class Stamp {
 public:
  Stamp(int kernel, void* stream, bool enabled = true);
  ~Stamp();
  Stamp(const Stamp&) = delete;
  Stamp& operator=(const Stamp&) = delete;

 private:
  int kernel_;
  void* st_;
  void* start_ = nullptr;
  void* stop_ = nullptr;
};

// Compute units and XCDs of the current device (cached per device).
int cu_count();
int xcd_count();

// Enqueue the quantization / K-write kernels (arguments already validated).
int launch_quantize(const qli_quant_params* p, void* stream);
int launch_write_k(const qli_kwrite_params* p, void* stream);
int launch_attention(const qli_attn_params* p, void* stream);
// Workgroups over which a token's entries are split when heads are a
// multiple of 64 (0: the head-group kernel runs; 1: no split).
int attention_splits(int64_t tokens, int heads, int topk, int window);
// Workspace bytes of a call with `splits` splits (0 for splits <= 1).
int64_t attention_workspace_bytes(int64_t tokens, int heads, int topk, int window, int splits);

}  // namespace qli
