// Step (c): Top-k selection per sequence, ties to the lower slot, output in
// ascending id order ([P1 "Compressed Sparse Attention 2 (CSA2)"]: a fresh
// Top-512, and the hierarchical indexer's pool of 2,048 blocks).
//
// One 1024-thread workgroup per sequence.  Scores are mapped to an
// order-preserving 32-bit key (0 = not a candidate) and the exact k-th key T
// is found by a radix select over digits of 12, 12 and 8 bits:
//   pass 1  LDS histogram of the top 12 bits over all candidates;
//   pass 2  keys above the threshold bin go straight into a selection
//           bitmap, keys inside it are buffered in LDS;
//   then the two low digits are resolved from the buffer (or, if the bin
//   holds more keys than the buffer, by further passes over the scores).
// Keys above T are selected; of the keys equal to T, the ones with the
// lowest slots are taken through a prefix count over a tie bitmap.  A final
// prefix count over the selection bitmap writes ids in ascending order.
// Everything is integer work on the keys, so the result is exact and
// independent of thread timing.
//
// Citation key: [P1] "DeepSeek AI Released DeepSeek-V4.1-Flash with 1M
// Context, FP4 KV Cache, and Cross-Layer Attention Reuse".
#include "common.hpp"

namespace csa2 {
namespace {

constexpr int kThreads = 1024;
constexpr int kWaves = kThreads / 64;
constexpr int kBins = 4096;
constexpr int kCandCap = 4096;
constexpr int kMaxWords = CSA2_TOPK_NMAX / 32;

struct TopkSmem {
  uint32_t hist[kBins];
  uint32_t sel[kMaxWords];
  uint32_t tie[kMaxWords];
  uint32_t cand_key[kCandCap];
  uint32_t cand_slot[kCandCap];
  uint32_t wave_sum[kWaves];
  uint32_t n_cand;
  uint32_t found_bin;
  uint32_t found_above;
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

// Exclusive prefix sum over the workgroup in thread order; *total gets the sum.
__device__ __forceinline__ uint32_t block_exclusive_scan(uint32_t v, TopkSmem& sm, uint32_t* total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  uint32_t x = v;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const uint32_t y = __shfl_up(x, d);
    if (lane >= d) x += y;
  }
  if (lane == 63) sm.wave_sum[wave] = x;
  __syncthreads();
  uint32_t before = 0, all = 0;
#pragma unroll
  for (int i = 0; i < kWaves; ++i) {
    const uint32_t s = sm.wave_sum[i];
    before += (i < wave) ? s : 0u;
    all += s;
  }
  __syncthreads();
  *total = all;
  return before + x - v;
}

// Over hist[0..nbins), find the largest bin B with (count of bins >= B) >= need.
// Writes B and the count of bins > B to sm.found_bin / sm.found_above.
// Requires 1 <= need <= total count.
__device__ void find_threshold_bin(TopkSmem& sm, int nbins, uint32_t need) {
  const int per = (nbins + kThreads - 1) / kThreads;
  const int t = threadIdx.x;
  // Thread t owns bins [hi - per, hi) with hi = nbins - t*per (top bins first).
  const int hi = nbins - t * per;
  const int lo = hi - per > 0 ? hi - per : 0;
  uint32_t mine = 0;
  for (int i = lo; i < hi; ++i) mine += sm.hist[i];
  uint32_t total;
  const uint32_t above = block_exclusive_scan(hi > 0 ? mine : 0u, sm, &total);
  if (hi > 0 && above < need && above + mine >= need) {
    uint32_t acc = above;
    for (int i = hi - 1; i >= lo; --i) {
      if (acc + sm.hist[i] >= need) {
        sm.found_bin = (uint32_t)i;
        sm.found_above = acc;
        break;
      }
      acc += sm.hist[i];
    }
  }
  __syncthreads();
}

__global__ __launch_bounds__(kThreads) void topk_kernel(const float* __restrict__ scores, int64_t n,
                                                        const int32_t* __restrict__ lens, int32_t len_div,
                                                        int32_t k, const int32_t* __restrict__ pool,
                                                        int32_t n_pool, int32_t blk,
                                                        int32_t* __restrict__ out) {
  extern __shared__ __attribute__((aligned(16))) unsigned char smem_raw[];
  TopkSmem& sm = *reinterpret_cast<TopkSmem*>(smem_raw);
  const int b = blockIdx.x;
  const int tid = threadIdx.x;
  int64_t nv = n;
  if (lens) {
    const int64_t L = lens[b];
    nv = min(n, L > 0 ? (L + len_div - 1) / len_div : 0);
  }
  const int nvalid = (int)nv;
  const int words = (nvalid + 31) / 32;
  const float* sc = scores + (int64_t)b * n;

  for (int i = tid; i < kBins; i += kThreads) sm.hist[i] = 0;
  for (int i = tid; i < words; i += kThreads) {
    sm.sel[i] = 0;
    sm.tie[i] = 0;
  }
  if (tid == 0) sm.n_cand = 0;
  __syncthreads();

  // Pass 1: histogram of the top digit.
  for (int i = tid; i < nvalid; i += kThreads) {
    const uint32_t key = order_key(sc[i]);
    if (key) atomicAdd(&sm.hist[key >> 20], 1u);
  }
  __syncthreads();

  uint32_t total = 0;
  {
    uint32_t mine = 0;
    for (int i = tid; i < kBins; i += kThreads) mine += sm.hist[i];
    block_exclusive_scan(mine, sm, &total);
  }
  const uint32_t kk = (uint32_t)k;
  uint32_t T = 0;       // selected: key > T, plus the first `ties` keys == T
  uint32_t ties = 0;

  if (total <= kk) {
    for (int i = tid; i < nvalid; i += kThreads)
      if (order_key(sc[i])) atomicOr(&sm.sel[i >> 5], 1u << (i & 31));
  } else {
    find_threshold_bin(sm, kBins, kk);
    const uint32_t b1 = sm.found_bin;
    const uint32_t need1 = kk - sm.found_above;
    const uint32_t in_bin = sm.hist[b1];
    __syncthreads();

    // Pass 2: keys above bin b1 are selected; keys in it are buffered.
    for (int i = tid; i < nvalid; i += kThreads) {
      const uint32_t key = order_key(sc[i]);
      const uint32_t d = key >> 20;
      if (!key) continue;
      if (d > b1) {
        atomicOr(&sm.sel[i >> 5], 1u << (i & 31));
      } else if (d == b1 && in_bin <= (uint32_t)kCandCap) {
        const uint32_t p = atomicAdd(&sm.n_cand, 1u);
        sm.cand_key[p] = key;
        sm.cand_slot[p] = (uint32_t)i;
      }
    }
    for (int i = tid; i < kBins; i += kThreads) sm.hist[i] = 0;
    __syncthreads();

    const bool buffered = in_bin <= (uint32_t)kCandCap;
    const int nc = (int)in_bin;
    // Digit 2: bits 19..8 among keys of bin b1.
    if (buffered) {
      for (int c = tid; c < nc; c += kThreads) atomicAdd(&sm.hist[(sm.cand_key[c] >> 8) & 0xFFFu], 1u);
    } else {
      for (int i = tid; i < nvalid; i += kThreads) {
        const uint32_t key = order_key(sc[i]);
        if (key && (key >> 20) == b1) atomicAdd(&sm.hist[(key >> 8) & 0xFFFu], 1u);
      }
    }
    __syncthreads();
    find_threshold_bin(sm, kBins, need1);
    const uint32_t b2 = sm.found_bin;
    const uint32_t need2 = need1 - sm.found_above;
    for (int i = tid; i < 256; i += kThreads) sm.hist[i] = 0;
    __syncthreads();
    const uint32_t pre2 = (b1 << 12) | b2;
    // Digit 3: bits 7..0 among keys with the first two digits.
    if (buffered) {
      for (int c = tid; c < nc; c += kThreads) {
        const uint32_t key = sm.cand_key[c];
        if ((key >> 8) == pre2) atomicAdd(&sm.hist[key & 0xFFu], 1u);
      }
    } else {
      for (int i = tid; i < nvalid; i += kThreads) {
        const uint32_t key = order_key(sc[i]);
        if (key && (key >> 8) == pre2) atomicAdd(&sm.hist[key & 0xFFu], 1u);
      }
    }
    __syncthreads();
    find_threshold_bin(sm, 256, need2);
    T = (pre2 << 8) | sm.found_bin;
    ties = need2 - sm.found_above;

    // Keys of bin b1 above T are selected, keys equal to T are tie candidates.
    if (buffered) {
      for (int c = tid; c < nc; c += kThreads) {
        const uint32_t key = sm.cand_key[c], i = sm.cand_slot[c];
        if (key > T) atomicOr(&sm.sel[i >> 5], 1u << (i & 31));
        else if (key == T) atomicOr(&sm.tie[i >> 5], 1u << (i & 31));
      }
    } else {
      for (int i = tid; i < nvalid; i += kThreads) {
        const uint32_t key = order_key(sc[i]);
        if ((key >> 20) != b1) continue;
        if (key > T) atomicOr(&sm.sel[i >> 5], 1u << (i & 31));
        else if (key == T) atomicOr(&sm.tie[i >> 5], 1u << (i & 31));
      }
    }
    __syncthreads();
  }

  // Each thread owns a contiguous run of bitmap words.
  const int per = (words + kThreads - 1) / kThreads;
  const int w0 = min(words, tid * per), w1 = min(words, w0 + per);

  if (ties > 0) {
    uint32_t cnt = 0;
    for (int w = w0; w < w1; ++w) cnt += __popc(sm.tie[w]);
    uint32_t dummy;
    uint32_t rank = block_exclusive_scan(cnt, sm, &dummy);
    for (int w = w0; w < w1 && rank < ties; ++w) {
      uint32_t x = sm.tie[w];
      const uint32_t pc = __popc(x);
      if (rank + pc <= ties) {
        sm.sel[w] |= x;
      } else {
        uint32_t keep = 0;
        for (uint32_t m = rank; m < ties; ++m) {
          keep |= x & (0u - x);
          x &= x - 1;
        }
        sm.sel[w] |= keep;
      }
      rank += pc;
    }
    __syncthreads();
  }

  // Ordered output.
  uint32_t cnt = 0;
  for (int w = w0; w < w1; ++w) cnt += __popc(sm.sel[w]);
  uint32_t n_sel;
  uint32_t pos = block_exclusive_scan(cnt, sm, &n_sel);
  int32_t* ob = out + (int64_t)b * k;
  for (int w = w0; w < w1; ++w) {
    uint32_t x = sm.sel[w];
    while (x) {
      const int bit = __ffs(x) - 1;
      x &= x - 1;
      const int64_t slot = (int64_t)w * 32 + bit;
      int64_t id = slot;
      if (pool) id = (int64_t)pool[(int64_t)b * n_pool + slot / blk] * blk + slot % blk;
      if (pos < kk) ob[pos] = (int32_t)id;
      ++pos;
    }
  }
  for (uint32_t i = n_sel + tid; i < kk; i += kThreads) ob[i] = -1;
}

}  // namespace

csa2_status topk_launch(const float* scores, int64_t n, const int32_t* lens, int32_t len_div, int32_t k,
                        const int32_t* pool, int32_t n_pool, int32_t blk, int32_t* out, int32_t n_seq,
                        hipStream_t stream) {
  if (n_seq == 0) return CSA2_OK;
  static bool attr_set = false;
  if (!attr_set) {
    if (hipFuncSetAttribute(reinterpret_cast<const void*>(topk_kernel),
                            hipFuncAttributeMaxDynamicSharedMemorySize,
                            (int)sizeof(TopkSmem)) != hipSuccess)
      return launch_status("csa2_topk (shared memory attribute)");
    attr_set = true;
  }
  hipLaunchKernelGGL(topk_kernel, dim3(n_seq), dim3(kThreads), sizeof(TopkSmem), stream, scores, n,
                     lens, len_div, k, pool, n_pool, blk, out);
  return launch_status("csa2_topk");
}

}  // namespace csa2
