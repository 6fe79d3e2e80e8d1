// Step (b): indexer scoring, score(k) = sum_h w_h * max(0, q_h . k) over the
// 8 indexer heads (the pages name indexer Q/K scoring without a formula;
// this per-head ReLU sum is the reading documented in csa2.h).
//
// The 8-head x 64-dim query against a stream of 64-dim keys is a small dense
// contraction, so it runs on MFMA: one v_mfma_f32_16x16x32_bf16 pair per 16
// keys, A = the query (rows 0..7 = heads, rows 8..15 zero), B = 16 keys.
// Lane (n = l%16, g = l/16) loads 32 contiguous bytes of key n (dims
// 16g..16g+15) and the query lanes hold the same dims, so the k-slot -> dim
// map is consistent on both operands.  The output lane holds heads
// 4g..4g+3 of key n; lanes g = 0, 1 hold the real heads, and one exchange
// (xor 16) adds heads 0..3 (lo) and 4..7 (hi).  Integer-valued bf16 inputs
// give products and fp32 sums that are exact, so scores are exact.
//
// The kernel is a pure HBM stream (128 bytes per key); each wavefront
// issues all its key loads before its MFMAs to keep many bytes in flight.
#include "common.hpp"

namespace csa2 {
namespace {

constexpr int kTilesPerWave = 8;                       // 16 keys per tile
constexpr int kKeysPerWG = 4 * kTilesPerWave * 16;     // 512 keys, 4 wavefronts

// Weighted ReLU sum of four heads, ((w0 r0 + w1 r1) + w2 r2) + w3 r3, every
// product and sum rounded on its own (no fused multiply-add).
__device__ __forceinline__ float relu_wsum4(const f32x4& acc, const float* wh) {
#pragma clang fp contract(off)
  float part = wh[0] * fmaxf(acc[0], 0.f);
#pragma unroll
  for (int r = 1; r < 4; ++r) part = part + wh[r] * fmaxf(acc[r], 0.f);
  return part;
}

template <bool kPool, bool kWeights>
__global__ __launch_bounds__(256) void index_score_kernel(
    const uint16_t* __restrict__ q, const float* __restrict__ w, const uint16_t* __restrict__ keys,
    int64_t key_cap, const int32_t* __restrict__ lens, int32_t len_div,
    const int32_t* __restrict__ pool, int32_t n_pool, int32_t blk, float* __restrict__ scores,
    int64_t n_out) {
  const int b = blockIdx.y;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int n = lane & 15, g = lane >> 4;
  const int64_t L = lens[b];
  int64_t n_valid = n_out;
  if (!kPool) n_valid = min(n_out, (L + len_div - 1) / len_div);

  // Query operand: row n = head n (n < 8), dims 16g + 8t + i for step t.
  bf16x8 qa[2];
  {
    u32x4 v0 = {0, 0, 0, 0}, v1 = {0, 0, 0, 0};
    if (n < 8) {
      const u32x4* qp = reinterpret_cast<const u32x4*>(q + ((int64_t)b * 8 + n) * 64 + 16 * g);
      v0 = qp[0];
      v1 = qp[1];
    }
    qa[0] = as_bf16x8(v0);
    qa[1] = as_bf16x8(v1);
  }
  float wh[4] = {1.f, 1.f, 1.f, 1.f};
  if (kWeights && g < 2) {
#pragma unroll
    for (int r = 0; r < 4; ++r) wh[r] = w[(int64_t)b * 8 + 4 * g + r];
  }

  const int64_t base = (int64_t)blockIdx.x * kKeysPerWG + (int64_t)wave * (kTilesPerWave * 16);
  const uint16_t* kb = keys + (int64_t)b * key_cap * 64;

  u32x4 kv[kTilesPerWave][2];
  bool valid[kTilesPerWave];
#pragma unroll
  for (int t = 0; t < kTilesPerWave; ++t) {
    const int64_t slot = base + t * 16 + n;
    int64_t row = slot;
    bool ok = slot < n_valid;
    if (kPool && ok) {
      const int32_t blk_id = pool[(int64_t)b * n_pool + slot / blk];
      row = (int64_t)blk_id * blk + slot % blk;
      ok = blk_id >= 0 && row < L && row < key_cap;
    }
    valid[t] = ok;
    if (ok) {
      const u32x4* kp = reinterpret_cast<const u32x4*>(kb + row * 64 + 16 * g);
      kv[t][0] = __builtin_nontemporal_load(kp);
      kv[t][1] = __builtin_nontemporal_load(kp + 1);
    } else {
      kv[t][0] = u32x4{0, 0, 0, 0};
      kv[t][1] = u32x4{0, 0, 0, 0};
    }
  }

  float* sb = scores + (int64_t)b * n_out;
#pragma unroll
  for (int t = 0; t < kTilesPerWave; ++t) {
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
    acc = mfma16x16x32(qa[0], as_bf16x8(kv[t][0]), acc);
    acc = mfma16x16x32(qa[1], as_bf16x8(kv[t][1]), acc);
    // acc[r] = q_{4g+r} . key n.
    const float part = relu_wsum4(acc, wh);
    const float other = __shfl_xor(part, 16);
    const int64_t slot = base + t * 16 + n;
    if (g == 0 && slot < n_out) sb[slot] = valid[t] ? part + other : kNegInf;
  }
}

template <bool kPool, bool kWeights>
void launch_one(dim3 grid, hipStream_t stream, const uint16_t* q, const float* w, const uint16_t* keys,
                int64_t key_cap, const int32_t* lens, int32_t len_div, const int32_t* pool,
                int32_t n_pool, int32_t blk, float* scores, int64_t n_out) {
  hipLaunchKernelGGL((index_score_kernel<kPool, kWeights>), grid, dim3(256), 0, stream, q, w, keys,
                     key_cap, lens, len_div, pool, n_pool, blk, scores, n_out);
}

}  // namespace

csa2_status index_score_launch(const uint16_t* q, const float* w, const uint16_t* keys, int64_t key_cap,
                               const int32_t* lens, int32_t len_div, const int32_t* pool,
                               int32_t n_pool, int32_t blk, float* scores, int64_t n_out, int32_t n_seq,
                               hipStream_t stream) {
  if (n_seq == 0 || n_out == 0) return CSA2_OK;
  const int64_t wgs = (n_out + kKeysPerWG - 1) / kKeysPerWG;
  CSA2_REQUIRE(wgs <= 0x7FFFFFFF && n_seq <= 65535, CSA2_ESHAPE, "csa2_index_score: grid too large");
  const dim3 grid((uint32_t)wgs, (uint32_t)n_seq);
  if (pool) {
    if (w) launch_one<true, true>(grid, stream, q, w, keys, key_cap, lens, 1, pool, n_pool, blk, scores, n_out);
    else launch_one<true, false>(grid, stream, q, w, keys, key_cap, lens, 1, pool, n_pool, blk, scores, n_out);
  } else {
    if (w) launch_one<false, true>(grid, stream, q, w, keys, key_cap, lens, len_div, pool, 0, 1, scores, n_out);
    else launch_one<false, false>(grid, stream, q, w, keys, key_cap, lens, len_div, pool, 0, 1, scores, n_out);
  }
  return launch_status("csa2_index_score");
}

}  // namespace csa2
