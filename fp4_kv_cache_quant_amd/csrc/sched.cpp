// Layer-group scheduler: walks a static Full / Reindex / Reuse table and
// enqueues one decode step ([P1 "Compressed Sparse Attention 2 (CSA2)"]:
// each CSA2 layer is statically assigned one of three modes; the decoder's
// Full layer builds a pool of up to 2,048 blocks of 8 that later Reindex
// layers rescore).  All buffers are allocated once at create, so a step
// enqueues kernels only and can be captured in a HIP graph.
//
// Citation key: [P1] "DeepSeek AI Released DeepSeek-V4.1-Flash with 1M
// Context, FP4 KV Cache, and Cross-Layer Attention Reuse".
#include <hip/hip_runtime.h>

#include <algorithm>
#include <string>
#include <vector>

#include "common.hpp"
#include "topk_ws.hpp"

namespace csa2 {
csa2_status quant_append_launch(const uint16_t*, const csa2_fp4_kv&, int32_t*, int32_t*, hipStream_t);
csa2_status index_score_launch(const uint16_t*, const float*, const uint16_t*, int64_t, const int32_t*,
                               int32_t, const int32_t*, int32_t, int32_t, float*, int64_t, int32_t,
                               uint32_t*, hipStream_t, uint32_t* bound_inv = nullptr, int32_t bound_k = 0);
int64_t flat_local_groups(int64_t key_cap, int32_t k, int32_t n_seq);
size_t attn_workspace_bytes(int32_t, int32_t, int32_t);
csa2_status attn_launch(const uint16_t*, int32_t, const csa2_fp4_kv&, int32_t, const int32_t*, int32_t,
                        const void*, int, int64_t, const int32_t*, int32_t, const void*, const int32_t*, float,
                        float*, void*, hipStream_t);
csa2_status append_keys_launch(const uint16_t*, uint16_t*, int64_t, uint16_t*, int64_t, int32_t, const int32_t*,
                               int32_t*, int32_t, hipStream_t);
csa2_status check_kv(const csa2_fp4_kv& kv, const char* who);
}  // namespace csa2

using namespace csa2;

struct csa2_sched {
  csa2_sched_desc desc{};
  std::vector<csa2_layer> layers;
  std::vector<int> idx_buf_of_layer;  // buffer each layer attends with
  std::vector<int> full_of_layer;     // Reindex: the Full layer it rescores (else -1)
  int n_idx_bufs = 0;
  bool any_hier = false, any_flat = false;
  int device = 0;
  int32_t* idx_bufs = nullptr;  // [n_idx_bufs][n_seq][topk]
  int32_t* pool = nullptr;      // [n_seq][pool_blocks]
  float* scores = nullptr;      // [n_seq][scores_n]
  int64_t scores_n = 0;
  // Flat selection with per-workgroup Top-k candidates (flat_local_groups:
  // local_groups * topk per sequence, scores in `scores`, positions here),
  // then one selection over them; 0: every score written and selected.
  int64_t local_groups = 0;
  int32_t* cand_slot = nullptr;  // [n_seq][local_groups * topk]
  void* attn_ws = nullptr;
  size_t attn_ws_bytes = 0;
  void* topk_ws = nullptr;      // Top-k workspace (histogram, counters, bitmap, candidates)
  size_t topk_ws_bytes = 0;
  TopkWs tw{};
  int32_t* err = nullptr;
};

namespace {

void free_sched(csa2_sched* s) {
  if (!s) return;
  hipFree(s->idx_bufs);
  hipFree(s->pool);
  hipFree(s->scores);
  hipFree(s->cand_slot);
  hipFree(s->attn_ws);
  hipFree(s->topk_ws);
  hipFree(s->err);
  delete s;
}

csa2_status validate_table(const csa2_sched_desc& d) {
  CSA2_REQUIRE(d.n_layers >= 1 && d.layers, CSA2_EMODE, "csa2_sched_create: empty layer table");
  bool seen_full = false, seen_sel = false;
  for (int l = 0; l < d.n_layers; ++l) {
    const csa2_layer& L = d.layers[l];
    CSA2_REQUIRE(L.kv_id >= 0, CSA2_EMODE, "csa2_sched_create: negative kv_id in layer " + std::to_string(l));
    switch (L.mode) {
      case CSA2_FULL:
        seen_full = seen_sel = true;
        break;
      case CSA2_REINDEX:
        CSA2_REQUIRE(seen_full, CSA2_EMODE,
                     "csa2_sched_create: Reindex layer " + std::to_string(l) + " has no earlier Full layer");
        seen_sel = true;
        break;
      case CSA2_REUSE:
        CSA2_REQUIRE(seen_sel, CSA2_EMODE,
                     "csa2_sched_create: Reuse layer " + std::to_string(l) + " has no earlier Full/Reindex layer");
        break;
      default:
        CSA2_REQUIRE(false, CSA2_EMODE, "csa2_sched_create: unknown mode in layer " + std::to_string(l));
    }
  }
  return CSA2_OK;
}

template <typename T>
csa2_status dev_alloc(T** p, size_t bytes) {
  if (bytes == 0) bytes = 256;
  if (hipMalloc(reinterpret_cast<void**>(p), bytes) != hipSuccess) {
    hipGetLastError();
    set_error("csa2_sched_create: device allocation of " + std::to_string(bytes) + " bytes failed");
    return CSA2_ENOMEM;
  }
  return CSA2_OK;
}

}  // namespace

extern "C" {

csa2_status csa2_sched_create(const csa2_sched_desc* desc, csa2_sched** out) {
  clear_error();
  CSA2_REQUIRE(desc && out, CSA2_EINVAL, "csa2_sched_create: null pointer");
  *out = nullptr;
  const csa2_sched_desc& d = *desc;
  csa2_status st = validate_table(d);
  if (st != CSA2_OK) return st;
  CSA2_REQUIRE(d.n_seq >= 1 && d.n_seq <= 65535, CSA2_ESHAPE, "csa2_sched_create: n_seq must be in [1, 65535]");
  CSA2_REQUIRE(d.key_cap >= 1 && d.topk >= 1 && d.topk <= CSA2_TOPK_MAX, CSA2_ESHAPE,
               "csa2_sched_create: bad key_cap / topk");
  CSA2_REQUIRE(d.swa_max >= 0 && d.swa_max <= 4096 && d.topk + d.swa_max <= 8192, CSA2_ESHAPE,
               "csa2_sched_create: bad swa_max");
  CSA2_REQUIRE(d.swa_fp8 == 0 || d.swa_fp8 == 1, CSA2_EINVAL, "csa2_sched_create: swa_fp8 must be 0 or 1");

  csa2_sched* s = new csa2_sched();
  s->desc = d;
  s->layers.assign(d.layers, d.layers + d.n_layers);
  s->desc.layers = s->layers.data();
  hipGetDevice(&s->device);

  int last_sel = -1, last_full = -1;
  for (int l = 0; l < d.n_layers; ++l) {
    const csa2_layer& L = s->layers[l];
    int full = -1;
    if (L.mode == CSA2_FULL) {
      last_sel = s->n_idx_bufs++;
      last_full = l;
      (L.hierarchical ? s->any_hier : s->any_flat) = true;
    } else if (L.mode == CSA2_REINDEX) {
      last_sel = s->n_idx_bufs++;
      full = last_full;
      if (!s->layers[last_full].hierarchical) s->any_flat = true;
    }
    s->idx_buf_of_layer.push_back(last_sel);
    s->full_of_layer.push_back(full);
  }
  if (s->any_hier) {
    if (!(d.blk >= 1 && d.pool_blocks >= 1 && d.blk_cap >= 1 && d.blk_cap <= CSA2_TOPK_NMAX &&
          (int64_t)d.pool_blocks * d.blk <= CSA2_TOPK_NMAX && d.pool_blocks <= CSA2_TOPK_MAX &&
          d.blk_cap * d.blk >= d.key_cap)) {
      free_sched(s);
      set_error("csa2_sched_create: hierarchical layers need 1 <= pool_blocks <= 2048, blk >= 1, "
                "pool_blocks*blk <= 1048576, blk_cap*blk >= key_cap and blk_cap <= 1048576");
      return CSA2_ESHAPE;
    }
    s->scores_n = std::max<int64_t>(d.blk_cap, (int64_t)d.pool_blocks * d.blk);
  }
  if (s->any_flat) {
    if (d.key_cap > CSA2_TOPK_NMAX) {
      free_sched(s);
      set_error("csa2_sched_create: flat selection supports key_cap <= 1048576");
      return CSA2_ESHAPE;
    }
    s->scores_n = std::max<int64_t>(s->scores_n, d.key_cap);
    s->local_groups = flat_local_groups(d.key_cap, d.topk, d.n_seq);
  }
  s->attn_ws_bytes = attn_workspace_bytes(d.n_seq, d.topk, d.swa_max);
  s->topk_ws_bytes = topk_workspace_bytes(s->scores_n, d.n_seq);
  const size_t n = (size_t)d.n_seq;
  if ((st = dev_alloc(&s->idx_bufs, (size_t)s->n_idx_bufs * n * d.topk * sizeof(int32_t))) != CSA2_OK ||
      (st = dev_alloc(&s->pool, s->any_hier ? n * d.pool_blocks * sizeof(int32_t) : 0)) != CSA2_OK ||
      (st = dev_alloc(&s->scores, n * (size_t)s->scores_n * sizeof(float))) != CSA2_OK ||
      (st = dev_alloc(&s->cand_slot, n * (size_t)(s->local_groups * d.topk) * sizeof(int32_t))) != CSA2_OK ||
      (st = dev_alloc(&s->attn_ws, s->attn_ws_bytes)) != CSA2_OK ||
      (st = dev_alloc(&s->topk_ws, s->topk_ws_bytes)) != CSA2_OK ||
      (st = dev_alloc(&s->err, sizeof(int32_t))) != CSA2_OK) {
    free_sched(s);
    return st;
  }
  s->tw = topk_ws_carve(s->topk_ws, s->scores_n, d.n_seq);
  if (hipMemset(s->err, 0, sizeof(int32_t)) != hipSuccess ||
      hipMemset(s->topk_ws, 0, s->topk_ws_bytes) != hipSuccess ||
      hipMemset(s->idx_bufs, 0xFF, (size_t)s->n_idx_bufs * n * d.topk * sizeof(int32_t)) != hipSuccess) {
    free_sched(s);
    set_error("csa2_sched_create: hipMemset failed");
    return CSA2_EHIP;
  }
  *out = s;
  return CSA2_OK;
}

csa2_status csa2_sched_decode_step(csa2_sched* s, const csa2_step_io* io, void* stream_v) {
  clear_error();
  CSA2_REQUIRE(s && io, CSA2_EINVAL, "csa2_sched_decode_step: null pointer");
  int cur = -1;
  CSA2_REQUIRE(hipGetDevice(&cur) == hipSuccess && cur == s->device, CSA2_EINVAL,
               "csa2_sched_decode_step: the current device is not the one the scheduler was created on");
  const csa2_sched_desc& d = s->desc;
  const hipStream_t stream = as_stream(stream_v);
  CSA2_REQUIRE(io->n_kv >= 1 && io->kv, CSA2_EINVAL, "csa2_sched_decode_step: no main-KV tensors");
  CSA2_REQUIRE(io->lens && io->idx_k && io->main_q && io->swa && io->swa_len && io->out, CSA2_EINVAL,
               "csa2_sched_decode_step: null pointer in io");
  CSA2_REQUIRE(!s->any_hier || io->blk_k, CSA2_EINVAL, "csa2_sched_decode_step: hierarchical table needs blk_k");
  // The kernels read keys, queries, window rows and the appended row, and
  // write the outputs, in 16-byte pieces (FP4 scales in 8-byte pieces).
  auto a16 = [](const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15) == 0; };
  CSA2_REQUIRE(a16(io->idx_k) && a16(io->blk_k) && a16(io->new_row), CSA2_EINVAL,
               "csa2_sched_decode_step: idx_k, blk_k and new_row must be 16-byte aligned");
  for (int i = 0; i < io->n_kv; ++i) {
    csa2_status st = check_kv(io->kv[i], "csa2_sched_decode_step");
    if (st != CSA2_OK) return st;
    CSA2_REQUIRE(a16(io->kv[i].codes) && (reinterpret_cast<uintptr_t>(io->kv[i].scales) & 7) == 0, CSA2_EINVAL,
                 "csa2_sched_decode_step: kv codes need 16-byte and scales 8-byte alignment");
    CSA2_REQUIRE(io->kv[i].n_seq == d.n_seq && io->kv[i].cap <= d.key_cap, CSA2_ESHAPE,
                 "csa2_sched_decode_step: kv tensor " + std::to_string(i) +
                     " must hold n_seq sequences and cap <= key_cap");
  }
  for (int l = 0; l < d.n_layers; ++l) {
    const csa2_layer& L = s->layers[l];
    CSA2_REQUIRE(L.kv_id < io->n_kv, CSA2_EMODE,
                 "csa2_sched_decode_step: layer " + std::to_string(l) + " names a missing kv tensor");
    CSA2_REQUIRE(L.mode == CSA2_REUSE || (io->idx_q && io->idx_q[l]), CSA2_EINVAL,
                 "csa2_sched_decode_step: missing indexer Q for layer " + std::to_string(l));
    CSA2_REQUIRE(io->main_q[l] && io->swa[l] && io->out[l], CSA2_EINVAL,
                 "csa2_sched_decode_step: missing main Q / SWA / out for layer " + std::to_string(l));
    CSA2_REQUIRE(!io->layer_idx_k || !io->layer_idx_k[l] || (L.mode == CSA2_FULL && !L.hierarchical), CSA2_EINVAL,
                 "csa2_sched_decode_step: layer_idx_k entry " + std::to_string(l) +
                     " must be NULL (only flat Full layers own indexer K)");
    CSA2_REQUIRE(!io->new_swa_row || (io->new_swa_row[l] && a16(io->new_swa_row[l])), CSA2_EINVAL,
                 "csa2_sched_decode_step: new_swa_row entry " + std::to_string(l) +
                     " must be a 16-byte aligned row block");
    CSA2_REQUIRE(a16(io->main_q[l]) && a16(io->swa[l]) && a16(io->out[l]) &&
                     (L.mode == CSA2_REUSE || a16(io->idx_q[l])) && (!io->layer_idx_k || a16(io->layer_idx_k[l])),
                 CSA2_EINVAL,
                 "csa2_sched_decode_step: main Q, SWA, out, indexer Q and K of layer " + std::to_string(l) +
                     " must be 16-byte aligned");
  }
  if (io->new_idx_k) {
    // The appended position's indexer key, and its block's key: before the
    // latent append, which advances lens.
    csa2_status st = append_keys_launch(io->new_idx_k, io->idx_k, d.key_cap, s->any_hier ? io->blk_k : nullptr,
                                        d.blk_cap, d.blk, io->lens, s->err, d.n_seq, stream);
    if (st != CSA2_OK) return st;
  }
  if (io->new_row) {
    CSA2_REQUIRE(io->append_kv >= 0 && io->append_kv < io->n_kv, CSA2_EINVAL,
                 "csa2_sched_decode_step: append_kv out of range");
    csa2_status st = quant_append_launch(io->new_row, io->kv[io->append_kv], io->lens, s->err, stream);
    if (st != CSA2_OK) return st;
  }

  const size_t idx_stride = (size_t)d.n_seq * d.topk;
  for (int l = 0; l < d.n_layers; ++l) {
    const csa2_layer& L = s->layers[l];
    int32_t* idx = s->idx_bufs + idx_stride * s->idx_buf_of_layer[l];
    // Indexer K of this layer's Full layer (itself, or the one a Reindex
    // follows); Reuse layers read no keys.
    const int32_t full = L.mode == CSA2_FULL ? l : s->full_of_layer[l];
    const uint16_t* keys = (full >= 0 && io->layer_idx_k && io->layer_idx_k[full]) ? io->layer_idx_k[full] : io->idx_k;
    const float* w = io->idx_w ? io->idx_w[l] : nullptr;
    csa2_status st = CSA2_OK;
    bool use_pool = false;
    if (L.mode == CSA2_FULL && L.hierarchical) {
      // Blocks: flat scores of block keys (with their histogram), keep pool_blocks of them.
      st = index_score_launch(io->idx_q[l], w, io->blk_k, d.blk_cap, io->lens, d.blk, nullptr, 0, 1,
                              s->scores, d.blk_cap, d.n_seq, s->tw.hist, stream);
      if (st == CSA2_OK)
        st = topk_launch(s->scores, d.blk_cap, io->lens, d.blk, d.pool_blocks, nullptr, 0, 1, s->pool, s->tw,
                         true, d.n_seq, stream);
      use_pool = true;
    } else if (L.mode == CSA2_REINDEX) {
      use_pool = s->layers[s->full_of_layer[l]].hierarchical != 0;
    }
    if (st == CSA2_OK && L.mode != CSA2_REUSE) {
      // Up to kTopkRowsMax slots the selection reads the scores once in
      // registers (no histogram from the score kernel); longer inputs get the
      // histogram fused into the scoring pass.
      if (use_pool) {
        st = pool_select_path(io->idx_q[l], w, keys, d.key_cap, io->lens, s->pool, d.pool_blocks, d.blk, d.topk,
                              idx, s->scores, s->tw, d.n_seq, stream);
      } else {
        // Flat: all positions (csa2_flat_select's path, on the scheduler's buffers).
        FlatSelectWs f{};
        f.local_groups = s->local_groups;
        f.n_scores = s->local_groups ? s->local_groups * d.topk : d.key_cap;
        f.scores = s->scores;
        f.cand = s->cand_slot;
        f.tw = s->tw;
        st = flat_select_launch(io->idx_q[l], w, keys, d.key_cap, io->lens, d.topk, idx, f, d.n_seq, stream);
      }
    }
    if (st == CSA2_OK)
      st = attn_launch(io->main_q[l], d.n_seq, io->kv[L.kv_id], 1, idx, d.topk, io->swa[l],
                       d.swa_fp8 ? kWinE4m3 : kWinBf16, d.swa_max, io->swa_len, d.swa_max,
                       io->new_swa_row ? io->new_swa_row[l] : nullptr, io->lens, d.sm_scale, io->out[l],
                       s->attn_ws, stream);
    if (st != CSA2_OK) return st;
  }
  return CSA2_OK;
}

const int32_t* csa2_sched_indices(const csa2_sched* s, int32_t layer) {
  if (!s || layer < 0 || layer >= s->desc.n_layers) return nullptr;
  return s->idx_bufs + (size_t)s->desc.n_seq * s->desc.topk * s->idx_buf_of_layer[layer];
}

const int32_t* csa2_sched_pool(const csa2_sched* s) { return (s && s->any_hier) ? s->pool : nullptr; }

csa2_status csa2_sched_check(csa2_sched* s, int32_t* flags, void* stream_v) {
  clear_error();
  CSA2_REQUIRE(s && flags, CSA2_EINVAL, "csa2_sched_check: null pointer");
  int cur = -1;
  CSA2_REQUIRE(hipGetDevice(&cur) == hipSuccess && cur == s->device, CSA2_EINVAL,
               "csa2_sched_check: the current device is not the one the scheduler was created on");
  // Read and clear in order on the stream the steps ran on: the read sees
  // every step enqueued there before, and the clear cannot overtake a flag
  // that one of them raises.
  const hipStream_t stream = as_stream(stream_v);
  int32_t h = 0;
  if (hipMemcpyAsync(&h, s->err, sizeof h, hipMemcpyDeviceToHost, stream) != hipSuccess ||
      hipMemsetAsync(s->err, 0, sizeof h, stream) != hipSuccess || hipStreamSynchronize(stream) != hipSuccess) {
    set_error(std::string("csa2_sched_check: ") + hipGetErrorString(hipGetLastError()));
    return CSA2_EHIP;
  }
  *flags = h;
  return CSA2_OK;
}

void csa2_sched_destroy(csa2_sched* s) { free_sched(s); }

}  // extern "C"
