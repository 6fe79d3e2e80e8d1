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
#include <algorithm>

#include "common.hpp"
#include "topk_ws.hpp"

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

// kHist: also add the scores' top key digits into a per-sequence histogram
// (ghist [n_seq][4096]) for the Top-k that follows.
template <bool kPool, bool kWeights, bool kHist>
__global__ __launch_bounds__(256) void index_score_kernel(
    const uint16_t* __restrict__ q, const float* __restrict__ w, const uint16_t* __restrict__ keys,
    int64_t key_cap, const int32_t* __restrict__ lens, int32_t len_div,
    const int32_t* __restrict__ pool, int32_t n_pool, int32_t blk, float* __restrict__ scores,
    int64_t n_out, uint32_t* __restrict__ ghist) {
  __shared__ uint32_t hist[kHist ? kTopkBins : 1];
  const int b = blockIdx.y;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int n = lane & 15, g = lane >> 4;
  const int64_t L = lens[b];
  if (kHist) {
    for (int i = threadIdx.x; i < kTopkBins; i += 256) hist[i] = 0;
    __syncthreads();
  }
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

  const uint16_t* kb = keys + (int64_t)b * key_cap * 64;
  float* sb = scores + (int64_t)b * n_out;
  // Grid-stride over chunks of kKeysPerWG keys (one histogram flush per workgroup).
  for (int64_t chunk = blockIdx.x; chunk * kKeysPerWG < n_out; chunk += gridDim.x) {
    const int64_t base = chunk * kKeysPerWG + (int64_t)wave * (kTilesPerWave * 16);
    u32x4 kv[kTilesPerWave][2];
    bool valid[kTilesPerWave];
#pragma unroll
    for (int t = 0; t < kTilesPerWave; ++t) {
      const int64_t slot = base + t * 16 + n;
      int64_t row = slot;
      bool ok = slot < n_valid;
      if (kPool && ok) {
        const int32_t blk_id = pool[(int64_t)b * n_pool + slot / blk];  // slot < n_out = n_pool * blk
        row = (int64_t)blk_id * blk + slot % blk;
        ok = blk_id >= 0 && row < L && row < key_cap;
      }
      valid[t] = ok;
      // Unconditional load of a clamped row (an invalid slot reads row 0 and
      // is masked below), so the wavefront's loads are all in flight together.
      const u32x4* kp = reinterpret_cast<const u32x4*>(kb + (ok ? row : 0) * 64 + 16 * g);
      kv[t][0] = __builtin_nontemporal_load(kp);
      kv[t][1] = __builtin_nontemporal_load(kp + 1);
    }
#pragma unroll
    for (int t = 0; t < kTilesPerWave; ++t) {
      if (!valid[t]) kv[t][0] = kv[t][1] = u32x4{0, 0, 0, 0};
      f32x4 acc = {0.f, 0.f, 0.f, 0.f};
      acc = mfma16x16x32(qa[0], as_bf16x8(kv[t][0]), acc);
      acc = mfma16x16x32(qa[1], as_bf16x8(kv[t][1]), acc);
      // acc[r] = q_{4g+r} . key n.
      const float part = relu_wsum4(acc, wh);
      const float other = __shfl_xor(part, 16);
      const int64_t slot = base + t * 16 + n;
      if (g == 0 && slot < n_out) {
        const float score = part + other;
        sb[slot] = valid[t] ? score : kNegInf;
        const uint32_t key = order_key(score);
        if (kHist && valid[t] && key) atomicAdd(&hist[key >> 20], 1u);
      }
    }
  }
  if (kHist) {
    __syncthreads();
    uint32_t* gh = ghist + (int64_t)b * kTopkBins;
    for (int i = threadIdx.x; i < kTopkBins; i += 256)
      if (hist[i]) atomicAdd(&gh[i], hist[i]);
  }
}

template <bool kPool, bool kWeights>
void launch_one(dim3 grid, hipStream_t stream, const uint16_t* q, const float* w, const uint16_t* keys,
                int64_t key_cap, const int32_t* lens, int32_t len_div, const int32_t* pool,
                int32_t n_pool, int32_t blk, float* scores, int64_t n_out, uint32_t* ghist) {
  if (ghist)
    hipLaunchKernelGGL((index_score_kernel<kPool, kWeights, true>), grid, dim3(256), 0, stream, q, w, keys,
                       key_cap, lens, len_div, pool, n_pool, blk, scores, n_out, ghist);
  else
    hipLaunchKernelGGL((index_score_kernel<kPool, kWeights, false>), grid, dim3(256), 0, stream, q, w, keys,
                       key_cap, lens, len_div, pool, n_pool, blk, scores, n_out, ghist);
}

}  // namespace

csa2_status index_score_launch(const uint16_t* q, const float* w, const uint16_t* keys, int64_t key_cap,
                               const int32_t* lens, int32_t len_div, const int32_t* pool,
                               int32_t n_pool, int32_t blk, float* scores, int64_t n_out, int32_t n_seq,
                               uint32_t* ghist, hipStream_t stream) {
  if (n_seq == 0 || n_out == 0) return CSA2_OK;
  // About two workgroups per CU in total; each loops over chunks of 512
  // keys, so a fused histogram is flushed by few workgroups (its hot bins
  // see one global atomic per workgroup).
  const int64_t chunks = (n_out + kKeysPerWG - 1) / kKeysPerWG;
  const int64_t per_seq = std::max<int64_t>(1, std::min<int64_t>(chunks, (512 + n_seq - 1) / n_seq));
  CSA2_REQUIRE(n_seq <= 65535, CSA2_ESHAPE, "csa2_index_score: grid too large");
  const dim3 grid((uint32_t)per_seq, (uint32_t)n_seq);
  if (pool) {
    if (w) launch_one<true, true>(grid, stream, q, w, keys, key_cap, lens, 1, pool, n_pool, blk, scores, n_out, ghist);
    else launch_one<true, false>(grid, stream, q, w, keys, key_cap, lens, 1, pool, n_pool, blk, scores, n_out, ghist);
  } else {
    if (w) launch_one<false, true>(grid, stream, q, w, keys, key_cap, lens, len_div, pool, 0, 1, scores, n_out, ghist);
    else launch_one<false, false>(grid, stream, q, w, keys, key_cap, lens, len_div, pool, 0, 1, scores, n_out, ghist);
  }
  return launch_status("csa2_index_score");
}

}  // namespace csa2
