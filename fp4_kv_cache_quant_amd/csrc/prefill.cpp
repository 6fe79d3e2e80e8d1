// Prefill chunk of an encoder layer group over compressed entries: the
// indexer entry point of the chunk and the layer-table driver.  Semantics
// are documented in include/csa2.h.
//
// [P1 "Compressed Sparse Attention 2 (CSA2)"]: encoder layers run CSA2 at
// compression ratio 2 in groups of one Full and five Reuse layers; [P3]:
// the encoder merges adjacent positions.  Citation keys: [P1] "DeepSeek AI
// Released DeepSeek-V4.1-Flash with 1M Context, FP4 KV Cache, and
// Cross-Layer Attention Reuse"; [P3] "DeepSeek-V4.1 Flash: Pushing the
// Limits of KV Cache Compression".
#include <hip/hip_runtime.h>

#include <string>

#include "common.hpp"
#include "topk_ws.hpp"

namespace csa2 {

csa2_status prefill_score_launch(const uint16_t*, const float*, const uint16_t*, int64_t, int64_t, int32_t,
                                 int32_t, float*, int32_t*, int32_t*, int32_t, hipStream_t);
csa2_status prefill_filter_launch(int, const uint16_t*, const float*, const uint16_t*, int64_t, int64_t, int32_t,
                                  int32_t, float*, int32_t*, int32_t*, int32_t, const PrefillCandOut&, hipStream_t);
size_t attn_workspace_bytes(int32_t, int32_t, int32_t);
csa2_status attn_launch(const uint16_t*, int32_t, const csa2_fp4_kv&, int32_t, const int32_t*, int32_t,
                        const void*, int, int64_t, const int32_t*, int32_t, const void*, const int32_t*, float,
                        float*, void*, hipStream_t);
csa2_status check_kv(const csa2_fp4_kv& kv, const char* who);

namespace {

constexpr size_t kAlign = 256;
inline size_t align_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

// The selection of a chunk's queries (csa2_prefill_select and the Full /
// Reindex layers of csa2_prefill_chunk).  Workspace: scores [n_q][n] f32
// | Top-k workspace | when the selection is filtered while scoring
// (prefill_filter_applies): candidate lists [n_q][blocks][kCandCap] (score
// bits, entry), their counts [n_q][blocks] u32 and the flags of the query
// blocks to rescore [ceil(n_q / 32)] u32 (blocks = ceil(n / kCandBlock)).
struct SelectWs {
  float* scores;
  void* topk;
  bool filtered;
  PrefillCandOut co;
  size_t bytes;
};

SelectWs select_ws_layout(int64_t n_entries, int32_t n_q, int32_t k, uintptr_t p) {
  size_t off = 0;
  SelectWs w{};
  w.scores = reinterpret_cast<float*>(p + off);
  off += align_up((size_t)n_q * (size_t)n_entries * sizeof(float));
  w.topk = reinterpret_cast<void*>(p + off);
  off += align_up(topk_workspace_bytes(n_entries, n_q));
  w.filtered = prefill_filter_applies(n_entries, n_q, k);
  if (w.filtered) {
    const int32_t blocks = (int32_t)((n_entries + kCandBlock - 1) / kCandBlock);
    w.co.n_blocks = blocks;
    w.co.cand = reinterpret_cast<uint2*>(p + off);
    off += align_up((size_t)n_q * blocks * kCandCap * sizeof(uint2));
    w.co.cnt = reinterpret_cast<uint32_t*>(p + off);
    off += align_up((size_t)n_q * blocks * sizeof(uint32_t));
    w.co.flags = reinterpret_cast<uint32_t*>(p + off);
    off += align_up((size_t)(n_q + 31) / 32 * sizeof(uint32_t));
  }
  w.bytes = off;
  return w;
}

// Each query's Top-k of its scores over its visible entries into idx, and
// the visible counts into n_vis (win_len / win: the chunk's window lengths,
// or null).  Filtered: sampled scores -> thresholds -> candidates ->
// selection among them; the rows that selection cannot take are scored
// again in full (their whole query blocks) and selected over all entries.
csa2_status select_run(const SelectWs& w, const uint16_t* q, const float* wq, const uint16_t* keys,
                       int64_t n_entries, int64_t t0, int32_t ratio, int32_t n_q, int32_t k, int32_t* idx,
                       int32_t* n_vis, int32_t* win_len, int32_t win, hipStream_t stream) {
  const TopkWs tw = topk_ws_carve(w.topk, n_entries, n_q);
  csa2_status st = CSA2_OK;
  if (w.filtered) {
    PrefillCandOut co = w.co;
    co.thr = tw.wcnt + kThresholdSlot;
    co.thr_stride = kTopkFilterWgMax;
    for (int stage = 0; stage < 3 && st == CSA2_OK; ++stage) {
      st = prefill_filter_launch(stage, q, wq, keys, n_entries, t0, ratio, n_q, w.scores, n_vis, win_len, win, co,
                                 stream);
      if (st == CSA2_OK)
        st = prefill_select_launch(stage, w.scores, n_entries, n_vis, k, idx, tw, co, n_q, stream);
    }
    return st;
  }
  st = prefill_score_launch(q, wq, keys, n_entries, t0, ratio, n_q, w.scores, n_vis, win_len, win, stream);
  if (st == CSA2_OK) st = topk_launch(w.scores, n_entries, n_vis, 1, k, nullptr, 0, 1, idx, tw, false, n_q, stream);
  return st;
}

// Workspace of a chunk: the selection's | n_vis [n_q] | win_len [n_q] |
// attention workspace.
struct PrefillWs {
  SelectWs sel;
  int32_t* n_vis;
  int32_t* win_len;
  void* attn;
  size_t bytes;
};

PrefillWs prefill_ws_layout(const csa2_prefill_desc& d, void* base) {
  const uintptr_t p = reinterpret_cast<uintptr_t>(base);
  PrefillWs w{};
  w.sel = select_ws_layout(d.n_entries, d.n_q, d.topk, p);
  size_t off = w.sel.bytes;
  w.n_vis = reinterpret_cast<int32_t*>(p + off);
  off += align_up((size_t)d.n_q * sizeof(int32_t));
  w.win_len = reinterpret_cast<int32_t*>(p + off);
  off += align_up((size_t)d.n_q * sizeof(int32_t));
  w.attn = reinterpret_cast<void*>(p + off);
  off += align_up(attn_workspace_bytes(d.n_q, d.topk, d.swa));
  w.bytes = off;
  return w;
}

csa2_status check_prefill_desc(const csa2_prefill_desc* d) {
  CSA2_REQUIRE(d && d->layers && d->n_layers >= 1, CSA2_EINVAL, "csa2_prefill: null descriptor or empty table");
  CSA2_REQUIRE(d->n_q >= 1 && d->n_q <= 65535, CSA2_ESHAPE, "csa2_prefill: n_q must be in [1, 65535]");
  CSA2_REQUIRE(d->n_entries >= 1 && d->n_entries <= CSA2_TOPK_NMAX, CSA2_ESHAPE,
               "csa2_prefill: n_entries must be in [1, 1048576]");
  CSA2_REQUIRE(d->ratio >= 1, CSA2_EINVAL, "csa2_prefill: ratio must be >= 1");
  CSA2_REQUIRE(d->topk >= 1 && d->topk <= CSA2_TOPK_MAX, CSA2_ESHAPE, "csa2_prefill: topk must be in [1, 2048]");
  CSA2_REQUIRE(d->swa >= 0 && d->swa <= 4096 && (int64_t)d->topk + d->swa <= 8192, CSA2_ESHAPE,
               "csa2_prefill: need swa <= 4096 and topk + swa <= 8192");
  CSA2_REQUIRE(d->t0 >= (int64_t)d->swa - 1 && d->t0 >= 0, CSA2_ESHAPE,
               "csa2_prefill: t0 must be >= swa - 1 (every window lies inside the context)");
  bool seen_full = false, seen_sel = false;
  for (int l = 0; l < d->n_layers; ++l) {
    const csa2_layer& L = d->layers[l];
    CSA2_REQUIRE(L.kv_id >= 0, CSA2_EMODE, "csa2_prefill: negative kv_id");
    if (L.mode == CSA2_FULL) {
      CSA2_REQUIRE(!L.hierarchical, CSA2_EMODE, "csa2_prefill: hierarchical selection is a decode-only mode");
      seen_full = seen_sel = true;
    } else if (L.mode == CSA2_REINDEX) {
      CSA2_REQUIRE(seen_full, CSA2_EMODE, "csa2_prefill: Reindex layer without an earlier Full layer");
      seen_sel = true;
    } else if (L.mode == CSA2_REUSE) {
      CSA2_REQUIRE(seen_sel, CSA2_EMODE, "csa2_prefill: Reuse layer without an earlier Full/Reindex layer");
    } else {
      CSA2_REQUIRE(false, CSA2_EMODE, "csa2_prefill: unknown layer mode");
    }
  }
  return CSA2_OK;
}

}  // namespace
}  // namespace csa2

using namespace csa2;

extern "C" {

csa2_status csa2_prefill_index_score(const uint16_t* q, const float* w, const uint16_t* keys, int64_t n_entries,
                                     int64_t t0, int32_t ratio, int32_t n_q, float* scores, int32_t* n_vis,
                                     void* stream) {
  clear_error();
  CSA2_REQUIRE(n_q >= 0 && n_q <= 2097120, CSA2_ESHAPE, "csa2_prefill_index_score: n_q must be in [0, 2097120]");
  if (n_q == 0) return CSA2_OK;
  CSA2_REQUIRE(q && keys && scores && n_vis, CSA2_EINVAL, "csa2_prefill_index_score: null pointer");
  CSA2_REQUIRE(n_entries >= 1 && n_entries <= (int64_t(1) << 30), CSA2_ESHAPE,
               "csa2_prefill_index_score: n_entries must be in [1, 2^30]");
  CSA2_REQUIRE(ratio >= 1 && t0 >= 0, CSA2_EINVAL, "csa2_prefill_index_score: need ratio >= 1 and t0 >= 0");
  const uintptr_t a = reinterpret_cast<uintptr_t>(q) | reinterpret_cast<uintptr_t>(keys) |
                      reinterpret_cast<uintptr_t>(scores);
  CSA2_REQUIRE((a & 15) == 0, CSA2_EINVAL, "csa2_prefill_index_score: q, keys, scores must be 16-byte aligned");
  return prefill_score_launch(q, w, keys, n_entries, t0, ratio, n_q, scores, n_vis, nullptr, 0, as_stream(stream));
}

size_t csa2_prefill_select_workspace_size(int64_t n_entries, int32_t n_q, int32_t k) {
  clear_error();
  if (n_q < 1 || n_q > 65535 || n_entries < 1 || n_entries > CSA2_TOPK_NMAX || k < 1 || k > CSA2_TOPK_MAX) {
    set_error("csa2_prefill_select_workspace_size: need 1 <= n_q <= 65535, 1 <= n_entries <= 1048576, 1 <= k <= 2048");
    return 0;
  }
  return select_ws_layout(n_entries, n_q, k, 0).bytes;
}

csa2_status csa2_prefill_select(const uint16_t* q, const float* w, const uint16_t* keys, int64_t n_entries, int64_t t0,
                                int32_t ratio, int32_t n_q, int32_t k, int32_t* idx, int32_t* n_vis, void* ws,
                                size_t ws_bytes, void* stream) {
  clear_error();
  CSA2_REQUIRE(n_q >= 1 && n_q <= 65535 && n_entries >= 1 && n_entries <= CSA2_TOPK_NMAX && k >= 1 &&
                   k <= CSA2_TOPK_MAX,
               CSA2_ESHAPE, "csa2_prefill_select: need 1 <= n_q <= 65535, 1 <= n_entries <= 1048576, 1 <= k <= 2048");
  CSA2_REQUIRE(ratio >= 1 && t0 >= 0, CSA2_EINVAL, "csa2_prefill_select: need ratio >= 1 and t0 >= 0");
  CSA2_REQUIRE(q && keys && idx && n_vis && ws, CSA2_EINVAL, "csa2_prefill_select: null pointer");
  CSA2_REQUIRE(((reinterpret_cast<uintptr_t>(q) | reinterpret_cast<uintptr_t>(keys)) & 15) == 0, CSA2_EINVAL,
               "csa2_prefill_select: q and keys must be 16-byte aligned");
  CSA2_REQUIRE((reinterpret_cast<uintptr_t>(ws) & (kAlign - 1)) == 0, CSA2_EINVAL,
               "csa2_prefill_select: workspace must be 256-byte aligned");
  const SelectWs sw = select_ws_layout(n_entries, n_q, k, reinterpret_cast<uintptr_t>(ws));
  CSA2_REQUIRE(ws_bytes >= sw.bytes, CSA2_ECAPACITY, "csa2_prefill_select: workspace too small");
  return select_run(sw, q, w, keys, n_entries, t0, ratio, n_q, k, idx, n_vis, nullptr, 0, as_stream(stream));
}

size_t csa2_prefill_workspace_size(const csa2_prefill_desc* desc) {
  clear_error();
  if (check_prefill_desc(desc) != CSA2_OK) return 0;
  return prefill_ws_layout(*desc, nullptr).bytes;
}

csa2_status csa2_prefill_chunk(const csa2_prefill_desc* desc, const csa2_prefill_io* io, void* ws,
                               size_t ws_bytes, void* stream_v) {
  clear_error();
  csa2_status st = check_prefill_desc(desc);
  if (st != CSA2_OK) return st;
  const csa2_prefill_desc& d = *desc;
  CSA2_REQUIRE(io && ws, CSA2_EINVAL, "csa2_prefill_chunk: null io or workspace");
  CSA2_REQUIRE((reinterpret_cast<uintptr_t>(ws) & (kAlign - 1)) == 0, CSA2_EINVAL,
               "csa2_prefill_chunk: workspace must be 256-byte aligned");
  const PrefillWs w = prefill_ws_layout(d, ws);
  CSA2_REQUIRE(ws_bytes >= w.bytes, CSA2_ECAPACITY, "csa2_prefill_chunk: workspace too small");
  CSA2_REQUIRE(io->n_kv >= 1 && io->kv && io->entry_k && io->main_q && io->swa && io->out && io->idx,
               CSA2_EINVAL, "csa2_prefill_chunk: null pointer in io");
  CSA2_REQUIRE((reinterpret_cast<uintptr_t>(io->entry_k) & 15) == 0, CSA2_EINVAL,
               "csa2_prefill_chunk: entry_k must be 16-byte aligned");
  for (int i = 0; i < io->n_kv; ++i) {
    st = check_kv(io->kv[i], "csa2_prefill_chunk");
    if (st != CSA2_OK) return st;
    CSA2_REQUIRE((reinterpret_cast<uintptr_t>(io->kv[i].codes) & 15) == 0 &&
                     (reinterpret_cast<uintptr_t>(io->kv[i].scales) & 7) == 0,
                 CSA2_EINVAL, "csa2_prefill_chunk: codes need 16-byte and scales 8-byte alignment");
    CSA2_REQUIRE(io->kv[i].n_seq >= 1 && io->kv[i].cap >= d.n_entries, CSA2_ESHAPE,
                 "csa2_prefill_chunk: kv tensor " + std::to_string(i) + " must hold n_entries rows");
  }
  for (int l = 0; l < d.n_layers; ++l) {
    const csa2_layer& L = d.layers[l];
    CSA2_REQUIRE(L.kv_id < io->n_kv, CSA2_EMODE,
                 "csa2_prefill_chunk: layer " + std::to_string(l) + " names a missing kv tensor");
    CSA2_REQUIRE(L.mode == CSA2_REUSE || (io->idx_q && io->idx_q[l] && io->idx[l]), CSA2_EINVAL,
                 "csa2_prefill_chunk: missing indexer Q or index output for layer " + std::to_string(l));
    CSA2_REQUIRE(io->main_q[l] && io->swa[l] && io->out[l], CSA2_EINVAL,
                 "csa2_prefill_chunk: missing main Q / SWA / out for layer " + std::to_string(l));
    const uintptr_t a = reinterpret_cast<uintptr_t>(io->main_q[l]) | reinterpret_cast<uintptr_t>(io->swa[l]) |
                        reinterpret_cast<uintptr_t>(io->out[l]) |
                        (L.mode == CSA2_REUSE ? 0 : reinterpret_cast<uintptr_t>(io->idx_q[l]));
    CSA2_REQUIRE((a & 15) == 0, CSA2_EINVAL,
                 "csa2_prefill_chunk: Q, SWA and out of layer " + std::to_string(l) + " must be 16-byte aligned");
  }

  const hipStream_t stream = as_stream(stream_v);
  const int32_t* cur = nullptr;
  for (int l = 0; l < d.n_layers; ++l) {
    const csa2_layer& L = d.layers[l];
    if (L.mode != CSA2_REUSE) {
      // Full and Reindex both score every visible entry with their own Q.
      st = select_run(w.sel, io->idx_q[l], io->idx_w ? io->idx_w[l] : nullptr, io->entry_k, d.n_entries, d.t0,
                      d.ratio, d.n_q, d.topk, io->idx[l], w.n_vis, w.win_len, d.swa, stream);
      if (st != CSA2_OK) return st;
      cur = io->idx[l];
    }
    // Query i's window rows start at row i of the layer's SWA buffer (bf16,
    // converted to f16 in the attention kernel's registers).
    st = attn_launch(io->main_q[l], d.n_q, io->kv[L.kv_id], d.n_q, cur, d.topk, io->swa[l], kWinBf16, 1, w.win_len,
                     d.swa, nullptr, nullptr, d.sm_scale, io->out[l], w.attn, stream);
    if (st != CSA2_OK) return st;
  }
  return CSA2_OK;
}

}  // extern "C"
