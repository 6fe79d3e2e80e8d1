// C ABI of libcsa2: argument validation, error reporting, dispatch to the
// kernel launchers.  Semantics of every entry point are documented in
// include/csa2.h.
#include <hip/hip_runtime.h>

#include <string>

#include "common.hpp"
#include "topk_ws.hpp"

namespace csa2 {

csa2_status quant_rows_launch(const uint16_t*, int64_t, uint8_t*, uint8_t*, hipStream_t);
csa2_status quant_append_launch(const uint16_t*, const csa2_fp4_kv&, int32_t*, int32_t*, hipStream_t);
csa2_status quant_fp8_launch(const uint16_t*, int64_t, uint8_t*, hipStream_t);
csa2_status block_keys_launch(const uint16_t*, int64_t, const int32_t*, int32_t, uint16_t*, int64_t, int32_t,
                              hipStream_t);
csa2_status append_keys_launch(const uint16_t*, uint16_t*, int64_t, uint16_t*, int64_t, int32_t, const int32_t*,
                               int32_t*, int32_t, hipStream_t);
csa2_status index_score_launch(const uint16_t*, const float*, const uint16_t*, int64_t, const int32_t*,
                               int32_t, const int32_t*, int32_t, int32_t, float*, int64_t, int32_t,
                               uint32_t*, hipStream_t, uint32_t* bound_inv = nullptr, int32_t bound_k = 0);
int64_t flat_local_groups(int64_t key_cap, int32_t k, int32_t n_seq);
csa2_status index_score_local_launch(const uint16_t*, const float*, const uint16_t*, int64_t, const int32_t*, int32_t,
                                     float*, int32_t*, int32_t, hipStream_t);
size_t attn_workspace_bytes(int32_t, int32_t, int32_t);
csa2_status attn_scratch(void** ptr, size_t* bytes);
csa2_status attn_launch(const uint16_t*, int32_t, const csa2_fp4_kv&, int32_t, const int32_t*, int32_t,
                        const void*, int, int64_t, const int32_t*, int32_t, const void*, const int32_t*, float,
                        float*, void*, hipStream_t);
csa2_status attn_partial_launch(const uint16_t*, int32_t, const csa2_fp4_kv&, int32_t, const int32_t*, int32_t,
                                const void*, int, int64_t, const int32_t*, int32_t, float, float*, float*, void*,
                                hipStream_t);
csa2_status attn_merge_launch(const float*, const float*, int32_t, int32_t, float*, hipStream_t);

namespace {
thread_local std::string g_error;
}

void set_error(const std::string& msg) { g_error = msg; }
void clear_error() { g_error.clear(); }

csa2_status launch_status(const char* what) {
  const hipError_t e = hipGetLastError();
  if (e == hipSuccess) return CSA2_OK;
  set_error(std::string(what) + ": " + hipGetErrorString(e));
  return CSA2_EHIP;
}

// Checks shared by the standalone calls and the scheduler.
csa2_status check_kv(const csa2_fp4_kv& kv, const char* who) {
  CSA2_REQUIRE(kv.codes && kv.scales, CSA2_EINVAL, std::string(who) + ": null FP4 cache pointer");
  CSA2_REQUIRE(kv.cap > 0 && kv.n_seq >= 0, CSA2_ESHAPE, std::string(who) + ": bad FP4 cache shape");
  CSA2_REQUIRE(kv.cap < (int64_t(1) << 31), CSA2_ESHAPE,
               std::string(who) + ": cache capacity must be below 2^31 rows");
  return CSA2_OK;
}

csa2_status check_index_score(const uint16_t* q, const uint16_t* keys, int64_t key_cap,
                              const int32_t* lens, int32_t len_div, const int32_t* pool, int32_t n_pool,
                              int32_t blk, const float* scores, int64_t n_out, int32_t n_seq) {
  CSA2_REQUIRE(n_seq >= 0 && n_seq <= 65535, CSA2_ESHAPE, "csa2_index_score: n_seq must be in [0, 65535]");
  if (n_seq == 0) return CSA2_OK;
  CSA2_REQUIRE(q && keys && lens && scores, CSA2_EINVAL, "csa2_index_score: null pointer");
  CSA2_REQUIRE(key_cap > 0 && n_out >= 0, CSA2_ESHAPE, "csa2_index_score: bad key_cap / n_out");
  if (pool) {
    CSA2_REQUIRE(n_pool > 0 && blk > 0, CSA2_ESHAPE, "csa2_index_score: bad n_pool / blk");
    CSA2_REQUIRE(n_out == (int64_t)n_pool * blk, CSA2_ESHAPE,
                 "csa2_index_score: pool mode needs n_out == n_pool * blk");
  } else {
    CSA2_REQUIRE(len_div > 0, CSA2_EINVAL, "csa2_index_score: len_div must be positive");
    CSA2_REQUIRE(n_out <= key_cap, CSA2_ESHAPE, "csa2_index_score: n_out exceeds key_cap");
  }
  CSA2_REQUIRE((reinterpret_cast<uintptr_t>(q) & 15) == 0 && (reinterpret_cast<uintptr_t>(keys) & 15) == 0,
               CSA2_EINVAL, "csa2_index_score: q and keys must be 16-byte aligned");
  return CSA2_OK;
}

// ------------------------------------------------------------ flat select
// Workspace of a flat selection: scores (or the per-workgroup candidates'
// scores) | candidate positions | Top-k workspace, 256-byte aligned parts.
FlatSelectWs flat_select_ws(int64_t key_cap, int32_t k, int32_t n_seq, void* base) {
  auto up = [](size_t x) { return (x + 255) / 256 * 256; };
  FlatSelectWs f{};
  f.local_groups = flat_local_groups(key_cap, k, n_seq);
  f.n_scores = f.local_groups ? f.local_groups * k : key_cap;
  char* p = reinterpret_cast<char*>(base);
  size_t off = 0;
  f.scores = reinterpret_cast<float*>(p + off);
  off += up((size_t)n_seq * f.n_scores * sizeof(float));
  f.cand = reinterpret_cast<int32_t*>(p + off);
  off += up(f.local_groups ? (size_t)n_seq * f.n_scores * sizeof(int32_t) : 0);
  f.tw = base ? topk_ws_carve(p + off, f.n_scores, n_seq) : TopkWs{};
  off += topk_workspace_bytes(f.n_scores, n_seq);
  f.bytes = off;
  return f;
}

csa2_status flat_select_launch(const uint16_t* q, const float* w, const uint16_t* keys, int64_t key_cap,
                               const int32_t* lens, int32_t k, int32_t* out, const FlatSelectWs& f, int32_t n_seq,
                               hipStream_t stream) {
  if (f.local_groups > 0) {
    // Each scoring workgroup keeps the Top-k of its positions; the Top-k of
    // those candidates (ids = their positions) is the sequence's.
    csa2_status st = index_score_local_launch(q, w, keys, key_cap, lens, k, f.scores, f.cand, n_seq, stream);
    if (st != CSA2_OK) return st;
    return topk_launch(f.scores, f.n_scores, nullptr, 1, k, nullptr, 0, 1, out, f.tw, false, n_seq, stream, f.cand);
  }
  // Up to kTopkRowsMax positions the selection reads the scores once in
  // registers (no histogram from the score kernel); longer inputs get the
  // histogram fused into the scoring pass.
  const bool fused = key_cap > kTopkRowsMax;
  csa2_status st = index_score_launch(q, w, keys, key_cap, lens, 1, nullptr, 0, 1, f.scores, key_cap, n_seq,
                                      fused ? f.tw.hist : nullptr, stream);
  if (st != CSA2_OK) return st;
  return topk_launch(f.scores, key_cap, lens, 1, k, nullptr, 0, 1, out, f.tw, fused, n_seq, stream);
}

// ------------------------------------------------------------ pool select
// Workspace of a pool selection: scores [n_seq][n_pool * blk] | Top-k
// workspace, 256-byte aligned parts.
PoolSelectWs pool_select_ws(int32_t n_pool, int32_t blk, int32_t n_seq, void* base) {
  auto up = [](size_t x) { return (x + 255) / 256 * 256; };
  PoolSelectWs f{};
  f.n = (int64_t)n_pool * blk;
  char* p = reinterpret_cast<char*>(base);
  f.scores = reinterpret_cast<float*>(p);
  const size_t off = up((size_t)n_seq * f.n * sizeof(float));
  f.tw = base ? topk_ws_carve(p + off, f.n, n_seq) : TopkWs{};
  f.bytes = off + topk_workspace_bytes(f.n, n_seq);
  return f;
}

csa2_status pool_select_path(const uint16_t* q, const float* w, const uint16_t* keys, int64_t key_cap,
                             const int32_t* lens, const int32_t* pool, int32_t n_pool, int32_t blk, int32_t k,
                             int32_t* out, float* scores, const TopkWs& tw, int32_t n_seq, hipStream_t stream) {
  const int64_t n = (int64_t)n_pool * blk;
  if (n <= kPoolSelectMax) {
    // Scoring leaves a lower bound of each sequence's k-th key; the
    // selection takes the keys above it into LDS.
    csa2_status st = index_score_launch(q, w, keys, key_cap, lens, 1, pool, n_pool, blk, scores, n, n_seq, nullptr,
                                        stream, tw.bound, k);
    if (st != CSA2_OK) return st;
    return pool_select_launch(scores, n, k, pool, n_pool, blk, tw, out, n_seq, stream);
  }
  const bool fused = n > kTopkRowsMax;
  csa2_status st = index_score_launch(q, w, keys, key_cap, lens, 1, pool, n_pool, blk, scores, n, n_seq,
                                      fused ? tw.hist : nullptr, stream);
  if (st != CSA2_OK) return st;
  return topk_launch(scores, n, nullptr, 1, k, pool, n_pool, blk, out, tw, fused, n_seq, stream);
}

csa2_status check_topk(const float* scores, int64_t n, int32_t len_div, int32_t k, const int32_t* pool,
                       int32_t n_pool, int32_t blk, const int32_t* out, const void* ws, size_t ws_bytes,
                       int32_t n_seq) {
  CSA2_REQUIRE(n_seq >= 0 && n_seq <= 65535, CSA2_ESHAPE, "csa2_topk: n_seq must be in [0, 65535]");
  if (n_seq == 0) return CSA2_OK;
  CSA2_REQUIRE(scores && out && ws, CSA2_EINVAL, "csa2_topk: null pointer");
  CSA2_REQUIRE((reinterpret_cast<uintptr_t>(ws) & 15) == 0, CSA2_EINVAL, "csa2_topk: ws must be 16-byte aligned");
  CSA2_REQUIRE(k >= 1 && k <= CSA2_TOPK_MAX, CSA2_ESHAPE, "csa2_topk: k must be in [1, 2048]");
  CSA2_REQUIRE(n >= 0 && n <= CSA2_TOPK_NMAX, CSA2_ESHAPE, "csa2_topk: n must be in [0, 1048576]");
  CSA2_REQUIRE(len_div > 0, CSA2_EINVAL, "csa2_topk: len_div must be positive");
  if (pool) {
    CSA2_REQUIRE(n_pool > 0 && n_pool <= CSA2_TOPK_MAX && blk > 0 && n == (int64_t)n_pool * blk, CSA2_ESHAPE,
                 "csa2_topk: pool mode needs n == n_pool * blk and n_pool <= 2048");
  }
  CSA2_REQUIRE(ws_bytes >= topk_workspace_bytes(n, n_seq), CSA2_ECAPACITY, "csa2_topk: workspace too small");
  return CSA2_OK;
}

csa2_status check_attn(const uint16_t* q, int32_t n_q, const csa2_fp4_kv* kv, int32_t q_per_seq,
                       const int32_t* idx, int32_t k_idx, const void* swa, int64_t swa_q_stride_rows,
                       const int32_t* swa_len, int32_t swa_max, const float* out, const void* ws,
                       size_t ws_bytes) {
  CSA2_REQUIRE(n_q >= 0 && n_q <= 65535, CSA2_ESHAPE, "csa2_sparse_attn: n_q must be in [0, 65535]");
  if (n_q == 0) return CSA2_OK;
  CSA2_REQUIRE(q && kv && swa_len && out, CSA2_EINVAL, "csa2_sparse_attn: null pointer");
  CSA2_REQUIRE(k_idx >= 0 && swa_max >= 0 && k_idx + swa_max >= 1, CSA2_ESHAPE,
               "csa2_sparse_attn: need k_idx + swa_max >= 1");
  CSA2_REQUIRE(k_idx == 0 || idx, CSA2_EINVAL, "csa2_sparse_attn: null idx");
  CSA2_REQUIRE(swa_max == 0 || swa, CSA2_EINVAL, "csa2_sparse_attn: null swa");
  CSA2_REQUIRE(swa_max == 0 || swa_q_stride_rows >= 0, CSA2_EINVAL,
               "csa2_sparse_attn: swa_q_stride_rows must be >= 0");
  CSA2_REQUIRE(swa_max <= 4096 && (int64_t)k_idx + swa_max <= 128 * 64, CSA2_ESHAPE,
               "csa2_sparse_attn: k_idx + swa_max must be <= 8192 and swa_max <= 4096");
  CSA2_REQUIRE(q_per_seq >= 1, CSA2_EINVAL, "csa2_sparse_attn: q_per_seq must be >= 1");
  csa2_status st = check_kv(*kv, "csa2_sparse_attn");
  if (st != CSA2_OK) return st;
  CSA2_REQUIRE((n_q + q_per_seq - 1) / q_per_seq <= kv->n_seq, CSA2_ESHAPE,
               "csa2_sparse_attn: queries address more cache sequences than kv.n_seq");
  const size_t need = attn_workspace_bytes(n_q, k_idx, swa_max);
  CSA2_REQUIRE(need == 0 || ws, CSA2_EINVAL, "csa2_sparse_attn: null workspace");
  CSA2_REQUIRE(ws_bytes >= need, CSA2_ECAPACITY, "csa2_sparse_attn: workspace too small");
  const uintptr_t a = reinterpret_cast<uintptr_t>(q) | reinterpret_cast<uintptr_t>(kv->codes) |
                      reinterpret_cast<uintptr_t>(swa) | reinterpret_cast<uintptr_t>(out) |
                      reinterpret_cast<uintptr_t>(ws);
  CSA2_REQUIRE((a & 15) == 0 && (reinterpret_cast<uintptr_t>(kv->scales) & 7) == 0, CSA2_EINVAL,
               "csa2_sparse_attn: q, codes, swa, out, ws need 16-byte and scales 8-byte alignment");
  return CSA2_OK;
}

}  // namespace csa2

using namespace csa2;

extern "C" {

const char* csa2_last_error(void) { return g_error.c_str(); }

int32_t csa2_abi_version(void) { return 7; }

csa2_status csa2_quant_rows(const uint16_t* src, int64_t n_rows, uint8_t* codes, uint8_t* scales,
                            void* stream) {
  clear_error();
  CSA2_REQUIRE(n_rows >= 0, CSA2_ESHAPE, "csa2_quant_rows: negative n_rows");
  if (n_rows == 0) return CSA2_OK;
  CSA2_REQUIRE(src && codes && scales, CSA2_EINVAL, "csa2_quant_rows: null pointer");
  CSA2_REQUIRE((reinterpret_cast<uintptr_t>(src) & 15) == 0 && (reinterpret_cast<uintptr_t>(codes) & 3) == 0,
               CSA2_EINVAL, "csa2_quant_rows: src needs 16-byte and codes 4-byte alignment");
  return quant_rows_launch(src, n_rows, codes, scales, as_stream(stream));
}

csa2_status csa2_quant_append(const uint16_t* src, csa2_fp4_kv kv, int32_t* lens, int32_t* err_flag,
                              void* stream) {
  clear_error();
  CSA2_REQUIRE(kv.n_seq >= 0 && kv.n_seq <= 65535, CSA2_ESHAPE, "csa2_quant_append: bad n_seq");
  if (kv.n_seq == 0) return CSA2_OK;
  csa2_status st = check_kv(kv, "csa2_quant_append");
  if (st != CSA2_OK) return st;
  CSA2_REQUIRE(src && lens, CSA2_EINVAL, "csa2_quant_append: null pointer");
  CSA2_REQUIRE((reinterpret_cast<uintptr_t>(src) & 15) == 0 && (reinterpret_cast<uintptr_t>(kv.codes) & 3) == 0,
               CSA2_EINVAL, "csa2_quant_append: src needs 16-byte and codes 4-byte alignment");
  return quant_append_launch(src, kv, lens, err_flag, as_stream(stream));
}

csa2_status csa2_index_score(const uint16_t* q, const float* w, const uint16_t* keys, int64_t key_cap,
                             const int32_t* lens, int32_t len_div, const int32_t* pool, int32_t n_pool,
                             int32_t blk, float* scores, int64_t n_out, int32_t n_seq, void* stream) {
  clear_error();
  csa2_status st = check_index_score(q, keys, key_cap, lens, len_div, pool, n_pool, blk, scores, n_out, n_seq);
  if (st != CSA2_OK || n_seq == 0) return st;
  return index_score_launch(q, w, keys, key_cap, lens, len_div, pool, n_pool, blk, scores, n_out, n_seq,
                            nullptr, as_stream(stream));
}

size_t csa2_flat_select_workspace_size(int64_t key_cap, int32_t k, int32_t n_seq) {
  if (key_cap <= 0 || key_cap > CSA2_TOPK_NMAX || k < 1 || k > CSA2_TOPK_MAX || n_seq <= 0 || n_seq > 65535)
    return 0;
  return flat_select_ws(key_cap, k, n_seq, nullptr).bytes;
}

csa2_status csa2_flat_select(const uint16_t* q, const float* w, const uint16_t* keys, int64_t key_cap,
                             const int32_t* lens, int32_t k, int32_t* out, void* ws, size_t ws_bytes, int32_t n_seq,
                             void* stream) {
  clear_error();
  CSA2_REQUIRE(n_seq >= 0 && n_seq <= 65535, CSA2_ESHAPE, "csa2_flat_select: n_seq must be in [0, 65535]");
  if (n_seq == 0) return CSA2_OK;
  CSA2_REQUIRE(q && keys && lens && out && ws, CSA2_EINVAL, "csa2_flat_select: null pointer");
  CSA2_REQUIRE(key_cap >= 1 && key_cap <= CSA2_TOPK_NMAX, CSA2_ESHAPE, "csa2_flat_select: key_cap must be in [1, 1048576]");
  CSA2_REQUIRE(k >= 1 && k <= CSA2_TOPK_MAX, CSA2_ESHAPE, "csa2_flat_select: k must be in [1, 2048]");
  CSA2_REQUIRE((reinterpret_cast<uintptr_t>(q) & 15) == 0 && (reinterpret_cast<uintptr_t>(keys) & 15) == 0 &&
                   (reinterpret_cast<uintptr_t>(ws) & 255) == 0,
               CSA2_EINVAL, "csa2_flat_select: q and keys need 16-byte, ws 256-byte alignment");
  const FlatSelectWs f = flat_select_ws(key_cap, k, n_seq, ws);
  CSA2_REQUIRE(ws_bytes >= f.bytes, CSA2_ECAPACITY, "csa2_flat_select: workspace too small");
  return flat_select_launch(q, w, keys, key_cap, lens, k, out, f, n_seq, as_stream(stream));
}

size_t csa2_pool_select_workspace_size(int32_t n_pool, int32_t blk, int32_t n_seq) {
  if (n_pool < 1 || n_pool > CSA2_TOPK_MAX || blk < 1 || (int64_t)n_pool * blk > CSA2_TOPK_NMAX || n_seq <= 0 ||
      n_seq > 65535)
    return 0;
  return pool_select_ws(n_pool, blk, n_seq, nullptr).bytes;
}

csa2_status csa2_pool_select(const uint16_t* q, const float* w, const uint16_t* keys, int64_t key_cap,
                             const int32_t* lens, const int32_t* pool, int32_t n_pool, int32_t blk, int32_t k,
                             int32_t* out, void* ws, size_t ws_bytes, int32_t n_seq, void* stream) {
  clear_error();
  CSA2_REQUIRE(n_seq >= 0 && n_seq <= 65535, CSA2_ESHAPE, "csa2_pool_select: n_seq must be in [0, 65535]");
  if (n_seq == 0) return CSA2_OK;
  CSA2_REQUIRE(q && keys && lens && pool && out && ws, CSA2_EINVAL, "csa2_pool_select: null pointer");
  CSA2_REQUIRE(key_cap >= 1, CSA2_ESHAPE, "csa2_pool_select: key_cap must be >= 1");
  CSA2_REQUIRE(n_pool >= 1 && n_pool <= CSA2_TOPK_MAX && blk >= 1 && (int64_t)n_pool * blk <= CSA2_TOPK_NMAX,
               CSA2_ESHAPE, "csa2_pool_select: need 1 <= n_pool <= 2048 and n_pool * blk <= 1048576");
  CSA2_REQUIRE(k >= 1 && k <= CSA2_TOPK_MAX, CSA2_ESHAPE, "csa2_pool_select: k must be in [1, 2048]");
  CSA2_REQUIRE((reinterpret_cast<uintptr_t>(q) & 15) == 0 && (reinterpret_cast<uintptr_t>(keys) & 15) == 0 &&
                   (reinterpret_cast<uintptr_t>(ws) & 255) == 0,
               CSA2_EINVAL, "csa2_pool_select: q and keys need 16-byte, ws 256-byte alignment");
  const PoolSelectWs f = pool_select_ws(n_pool, blk, n_seq, ws);
  CSA2_REQUIRE(ws_bytes >= f.bytes, CSA2_ECAPACITY, "csa2_pool_select: workspace too small");
  return pool_select_path(q, w, keys, key_cap, lens, pool, n_pool, blk, k, out, f.scores, f.tw, n_seq,
                          as_stream(stream));
}

size_t csa2_topk_workspace_size(int64_t n, int32_t n_seq) {
  if (n < 0 || n_seq <= 0 || n > CSA2_TOPK_NMAX) return 0;
  return topk_workspace_bytes(n, n_seq);
}

csa2_status csa2_topk(const float* scores, int64_t n, const int32_t* lens, int32_t len_div, int32_t k,
                      const int32_t* pool, int32_t n_pool, int32_t blk, int32_t* out, void* ws,
                      size_t ws_bytes, int32_t n_seq, void* stream) {
  clear_error();
  csa2_status st = check_topk(scores, n, len_div, k, pool, n_pool, blk, out, ws, ws_bytes, n_seq);
  if (st != CSA2_OK || n_seq == 0) return st;
  return topk_launch(scores, n, lens, len_div, k, pool, n_pool, blk, out, topk_ws_carve(ws, n, n_seq), false,
                     n_seq, as_stream(stream));
}

size_t csa2_sparse_attn_workspace_size(int32_t n_q, int32_t k_idx, int32_t swa_max) {
  if (n_q <= 0 || k_idx < 0 || swa_max < 0 || k_idx + swa_max < 1) return 0;
  return attn_workspace_bytes(n_q, k_idx, swa_max);
}

csa2_status csa2_sparse_attn(const uint16_t* q, int32_t n_q, const csa2_fp4_kv* kv, int32_t q_per_seq,
                             const int32_t* idx, int32_t k_idx, const uint16_t* swa,
                             int64_t swa_q_stride_rows, const int32_t* swa_len, int32_t swa_max,
                             float sm_scale, float* out, void* ws, size_t ws_bytes, void* stream) {
  clear_error();
  csa2_status st = check_attn(q, n_q, kv, q_per_seq, idx, k_idx, swa, swa_q_stride_rows, swa_len, swa_max, out, ws,
                              ws_bytes);
  if (st != CSA2_OK || n_q == 0) return st;
  return attn_launch(q, n_q, *kv, q_per_seq, idx, k_idx, swa, kWinBf16, swa_q_stride_rows, swa_len, swa_max,
                     nullptr, nullptr, sm_scale, out, ws, as_stream(stream));
}

csa2_status csa2_sparse_attn_partial(const uint16_t* q, int32_t n_q, const csa2_fp4_kv* kv, int32_t q_per_seq,
                                     const int32_t* idx, int32_t k_idx, const uint16_t* swa,
                                     int64_t swa_q_stride_rows, const int32_t* swa_len, int32_t swa_max,
                                     float sm_scale, float* out_o, float* out_ml, void* ws, size_t ws_bytes,
                                     void* stream) {
  clear_error();
  csa2_status st = check_attn(q, n_q, kv, q_per_seq, idx, k_idx, swa, swa_q_stride_rows, swa_len, swa_max, out_o,
                              ws, ws_bytes);
  if (st != CSA2_OK || n_q == 0) return st;
  CSA2_REQUIRE(out_ml, CSA2_EINVAL, "csa2_sparse_attn_partial: null out_ml");
  CSA2_REQUIRE((reinterpret_cast<uintptr_t>(out_ml) & 7) == 0, CSA2_EINVAL,
               "csa2_sparse_attn_partial: out_ml needs 8-byte alignment");
  return attn_partial_launch(q, n_q, *kv, q_per_seq, idx, k_idx, swa, kWinBf16, swa_q_stride_rows, swa_len,
                             swa_max, sm_scale, out_o, out_ml, ws, as_stream(stream));
}

csa2_status csa2_attn_merge(const float* parts_o, const float* parts_ml, int32_t n_parts, int32_t n_q, float* out,
                            void* stream) {
  clear_error();
  CSA2_REQUIRE(n_q >= 0 && n_q <= 65535, CSA2_ESHAPE, "csa2_attn_merge: n_q must be in [0, 65535]");
  CSA2_REQUIRE(n_parts >= 1, CSA2_ESHAPE, "csa2_attn_merge: n_parts must be >= 1");
  if (n_q == 0) return CSA2_OK;
  CSA2_REQUIRE(parts_o && parts_ml && out, CSA2_EINVAL, "csa2_attn_merge: null pointer");
  CSA2_REQUIRE(((reinterpret_cast<uintptr_t>(parts_o) | reinterpret_cast<uintptr_t>(out)) & 15) == 0 &&
                   (reinterpret_cast<uintptr_t>(parts_ml) & 7) == 0,
               CSA2_EINVAL, "csa2_attn_merge: parts_o and out need 16-byte, parts_ml 8-byte alignment");
  return attn_merge_launch(parts_o, parts_ml, n_parts, n_q, out, as_stream(stream));
}

csa2_status csa2_sparse_attn_noalloc(const uint16_t* q, int32_t n_q, const csa2_fp4_kv* kv, int32_t q_per_seq,
                                     const int32_t* idx, int32_t k_idx, const uint16_t* swa,
                                     int64_t swa_q_stride_rows, const int32_t* swa_len, int32_t swa_max,
                                     float sm_scale, float* out, void* stream) {
  clear_error();
  void* ws = nullptr;
  size_t ws_bytes = 0;
  if (n_q > 0) {
    csa2_status st = attn_scratch(&ws, &ws_bytes);
    if (st != CSA2_OK) return st;
    const size_t need = attn_workspace_bytes(n_q, k_idx, swa_max);
    CSA2_REQUIRE(need <= ws_bytes, CSA2_ECAPACITY,
                 "csa2_sparse_attn_noalloc: this call needs " + std::to_string(need) +
                     " bytes of split partials; the static scratch holds " + std::to_string(ws_bytes) +
                     " (use csa2_sparse_attn with a workspace)");
  }
  csa2_status st = check_attn(q, n_q, kv, q_per_seq, idx, k_idx, swa, swa_q_stride_rows, swa_len, swa_max, out, ws,
                              ws_bytes);
  if (st != CSA2_OK || n_q == 0) return st;
  return attn_launch(q, n_q, *kv, q_per_seq, idx, k_idx, swa, kWinBf16, swa_q_stride_rows, swa_len, swa_max,
                     nullptr, nullptr, sm_scale, out, ws, as_stream(stream));
}

csa2_status csa2_sparse_attn_f8w(const uint16_t* q, int32_t n_q, const csa2_fp4_kv* kv, int32_t q_per_seq,
                                 const int32_t* idx, int32_t k_idx, const uint8_t* swa,
                                 int64_t swa_q_stride_rows, const int32_t* swa_len, int32_t swa_max,
                                 float sm_scale, float* out, void* ws, size_t ws_bytes, void* stream) {
  clear_error();
  csa2_status st = check_attn(q, n_q, kv, q_per_seq, idx, k_idx, swa, swa_q_stride_rows, swa_len, swa_max, out, ws,
                              ws_bytes);
  if (st != CSA2_OK || n_q == 0) return st;
  return attn_launch(q, n_q, *kv, q_per_seq, idx, k_idx, swa, kWinE4m3, swa_q_stride_rows, swa_len, swa_max,
                     nullptr, nullptr, sm_scale, out, ws, as_stream(stream));
}

csa2_status csa2_block_keys(const uint16_t* idx_k, int64_t key_cap, const int32_t* lens, int32_t blk,
                            uint16_t* blk_k, int64_t blk_cap, int32_t n_seq, void* stream) {
  clear_error();
  CSA2_REQUIRE(n_seq >= 0 && n_seq <= 65535, CSA2_ESHAPE, "csa2_block_keys: n_seq must be in [0, 65535]");
  if (n_seq == 0) return CSA2_OK;
  CSA2_REQUIRE(idx_k && lens && blk_k, CSA2_EINVAL, "csa2_block_keys: null pointer");
  CSA2_REQUIRE(key_cap >= 1 && blk >= 1 && blk_cap >= 1 && blk_cap * blk >= key_cap, CSA2_ESHAPE,
               "csa2_block_keys: need blk >= 1 and blk_cap * blk >= key_cap");
  return block_keys_launch(idx_k, key_cap, lens, blk, blk_k, blk_cap, n_seq, as_stream(stream));
}

csa2_status csa2_append_index_keys(const uint16_t* new_k, uint16_t* idx_k, int64_t key_cap, uint16_t* blk_k,
                                   int64_t blk_cap, int32_t blk, const int32_t* lens, int32_t* err_flag,
                                   int32_t n_seq, void* stream) {
  clear_error();
  CSA2_REQUIRE(n_seq >= 0 && n_seq <= 65535, CSA2_ESHAPE, "csa2_append_index_keys: n_seq must be in [0, 65535]");
  if (n_seq == 0) return CSA2_OK;
  CSA2_REQUIRE(new_k && idx_k && lens, CSA2_EINVAL, "csa2_append_index_keys: null pointer");
  CSA2_REQUIRE(key_cap >= 1 && (!blk_k || (blk >= 1 && blk_cap >= 1)), CSA2_ESHAPE,
               "csa2_append_index_keys: bad key_cap / blk / blk_cap");
  return append_keys_launch(new_k, idx_k, key_cap, blk_k, blk_cap, blk, lens, err_flag, n_seq, as_stream(stream));
}

csa2_status csa2_quant_fp8_rows(const uint16_t* src, int64_t n_rows, uint8_t* dst, void* stream) {
  clear_error();
  CSA2_REQUIRE(n_rows >= 0, CSA2_ESHAPE, "csa2_quant_fp8_rows: negative n_rows");
  if (n_rows == 0) return CSA2_OK;
  CSA2_REQUIRE(src && dst, CSA2_EINVAL, "csa2_quant_fp8_rows: null pointer");
  CSA2_REQUIRE((reinterpret_cast<uintptr_t>(src) & 15) == 0 && (reinterpret_cast<uintptr_t>(dst) & 7) == 0,
               CSA2_EINVAL, "csa2_quant_fp8_rows: src must be 16-byte and dst 8-byte aligned");
  return quant_fp8_launch(src, n_rows, dst, as_stream(stream));
}

}  // extern "C"
