// Workspace of the Top-k pipeline (internal; see topk.hip).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "csa2.h"

namespace csa2 {

constexpr int kTopkBins = 4096;                        // top-digit histogram (12 bits)
constexpr int kTopkCandCap = 8192;                     // keys buffered from the threshold bin
constexpr int kTopkLdsWords = 262144 / 32;            // bitmaps kept in LDS up to this many words
constexpr int kTopkFilterSlots = 8192;                 // slots per filter workgroup
constexpr int kTopkFilterWgMax = CSA2_TOPK_NMAX / kTopkFilterSlots;  // filter workgroups per sequence

// Per-sequence regions of one workspace.  hist must be zero when a Top-k
// call starts; the call leaves it zero.  Filter workgroup w of a sequence
// owns candidate slots [w * kTopkCandCap / nw, (w + 1) * kTopkCandCap / nw)
// of its sequence's buffer (nw = the sequence's filter workgroups) and
// writes how many candidates it found (possibly more than it could keep).
struct TopkWs {
  uint32_t* hist;     // [n_seq][kTopkBins]
  uint32_t* wcnt;     // [n_seq][kTopkFilterWgMax] candidates found per filter workgroup
  uint32_t* bits;     // [n_seq][words_cap] selection bitmap of the filter pass
  uint32_t* tie;      // [n_seq][words_cap] tie bitmap (inputs longer than kTopkLdsWords * 32)
  uint2* cand;        // [n_seq][kTopkCandCap] (key, slot)
  uint32_t* bound;    // [n_seq][kPoolTiles] per-tile key bounds left by bounded pool scoring
  int64_t words_cap;
};

// Order-preserving key of a score; NaN and -inf (non-candidates) map to 0,
// -0 and +0 map to the same key.
__device__ __forceinline__ uint32_t order_key(float f) {
  uint32_t u = __builtin_bit_cast(uint32_t, f);
  if ((u & 0x7FFFFFFFu) == 0) u = 0;
  if ((u & 0x7FFFFFFFu) > 0x7F800000u) return 0;  // NaN
  if (u == 0xFF800000u) return 0;                  // -inf
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// A row's threshold estimate of the many-row selection: an order key kept
// in entry kThresholdSlot of the row's wcnt row (kNoEstimate: none).
constexpr uint32_t kNoEstimate = 0xFFFFFFFFu;
constexpr int kThresholdSlot = kTopkFilterWgMax - 1;

// The smallest score whose order key is >= lo, for a threshold key lo that
// is 0, a key of a non-NaN score, or kNoEstimate: key(x) >= lo and
// key(x) != 0 hold exactly when x >= key_threshold(lo) (-0 and +0 share a
// key and compare equal; lo = 0 admits every score but NaN and -inf; the
// NaN for kNoEstimate admits none).
__device__ __forceinline__ float key_threshold(uint32_t lo) {
  if (lo == 0) return -__FLT_MAX__;
  return __builtin_bit_cast(float, (lo & 0x80000000u) ? (lo & 0x7FFFFFFFu) : ~lo);
}

// Candidates of many rows filtered while they are scored (a prefill chunk's
// selection, rows of at most kTopkRowsMax slots): per row and block of
// kCandBlock slots, the (score bits, slot) pairs of the block's scores at
// or above the row's threshold, in no particular order, and how many there
// were (more than kCandCap: the block's list is incomplete).
constexpr int kCandBlock = 512;
constexpr int kCandCap = 256;
struct PrefillCandOut {
  const uint32_t* thr = nullptr;  // threshold key of row i at thr[i * thr_stride]
  int64_t thr_stride = 0;
  uint2* cand = nullptr;          // [n_rows][n_blocks][kCandCap]
  uint32_t* cnt = nullptr;        // [n_rows][n_blocks]
  uint32_t* flags = nullptr;      // [ceil(n_rows / 32)]: bit i of word b = row 32b + i left to the full selection
  int32_t n_blocks = 0;           // ceil(n / kCandBlock)
};

// Inputs of at most this many slots per sequence are selected by one
// workgroup per sequence with the scores held in registers, unless a
// histogram was produced upstream.
constexpr int64_t kTopkRowsMax = 65536;

size_t topk_workspace_bytes(int64_t n, int32_t n_seq);
TopkWs topk_ws_carve(void* ws, int64_t n, int32_t n_seq);
// hist_ready: ws.hist already holds the histogram of these scores (written by
// the indexer-score kernel), so the histogram pass is skipped.  gids: if not
// NULL, [n_seq][n] ids emitted in place of the slots (inputs of at most
// kTopkRowsMax slots, no pool, no ready histogram).
csa2_status topk_launch(const float* scores, int64_t n, const int32_t* lens, int32_t len_div, int32_t k,
                        const int32_t* pool, int32_t n_pool, int32_t blk, int32_t* out, const TopkWs& ws,
                        bool hist_ready, int32_t n_seq, hipStream_t stream, const int32_t* gids = nullptr);

// A prefill chunk's selection filtered while it is scored (see topk.hip).
bool prefill_filter_applies(int64_t n, int32_t n_rows, int32_t k);
csa2_status prefill_select_launch(int stage, const float* scores, int64_t n, const int32_t* lens, int32_t k,
                                  int32_t* out, const TopkWs& ws, const PrefillCandOut& co, int32_t n_rows,
                                  hipStream_t stream);

// Pool slots of a hierarchical layer selected after scoring that left
// ws.bound (index_score_launch with tile_bound = ws.bound); n <= 16,384.
constexpr int64_t kPoolSelectMax = 16384;
constexpr int kPoolTiles = kPoolSelectMax / 128;  // 128-slot tiles with a bound each
csa2_status pool_select_launch(const float* scores, int64_t n, int32_t k, const int32_t* pool, int32_t n_pool,
                               int32_t blk, const TopkWs& ws, int32_t* out, int32_t n_seq, hipStream_t stream);

// A hierarchical layer's pool selection (scores of the pool's positions +
// Top-k; csa2_pool_select and the scheduler's pool layers).
struct PoolSelectWs {
  int64_t n;       // slots per sequence, n_pool * blk
  float* scores;   // [n_seq][n]
  TopkWs tw;
  size_t bytes;
};
PoolSelectWs pool_select_ws(int32_t n_pool, int32_t blk, int32_t n_seq, void* base);
csa2_status pool_select_path(const uint16_t* q, const float* w, const uint16_t* keys, int64_t key_cap,
                             const int32_t* lens, const int32_t* pool, int32_t n_pool, int32_t blk, int32_t k,
                             int32_t* out, float* scores, const TopkWs& tw, int32_t n_seq, hipStream_t stream);

// A flat Full layer's selection (scores + Top-k) and its workspace
// (csa2_flat_select; the scheduler's flat layers).
struct FlatSelectWs {
  int64_t local_groups;  // > 0: per-workgroup candidates (ceil(key_cap / 8192) groups)
  int64_t n_scores;      // scores per sequence: local_groups * k, or key_cap
  float* scores;         // [n_seq][n_scores]
  int32_t* cand;         // [n_seq][n_scores] candidate positions (local mode)
  TopkWs tw;
  size_t bytes;
};
FlatSelectWs flat_select_ws(int64_t key_cap, int32_t k, int32_t n_seq, void* base);
csa2_status flat_select_launch(const uint16_t* q, const float* w, const uint16_t* keys, int64_t key_cap,
                               const int32_t* lens, int32_t k, int32_t* out, const FlatSelectWs& f, int32_t n_seq,
                               hipStream_t stream);

}  // namespace csa2
