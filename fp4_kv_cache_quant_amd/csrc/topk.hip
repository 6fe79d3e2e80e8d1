// Step (c): Top-k selection per sequence, ties to the lower slot, output in
// ascending id order ([P1 "Compressed Sparse Attention 2 (CSA2)"]: a fresh
// Top-512, and the hierarchical indexer's pool of 2,048 blocks).
//
// Scores map to an order-preserving 32-bit key (0 = not a candidate).  The
// exact k-th key T is found by a radix select over digits of 12, 12 and 8
// bits, spread over up to three kernels so that the full-length passes run
// on many workgroups:
//   histogram  per-sequence counts of the top 12 key bits (global atomics of
//              per-workgroup LDS histograms; the indexer-score kernel can
//              produce it as a by-product, then this kernel is skipped);
//   filter     (long inputs) every workgroup reads the histogram, finds the
//              threshold bin b1, writes a selection bitmap of the keys above
//              b1 and the keys inside b1 to its own region of a candidate
//              buffer;
//   final      one workgroup per sequence resolves the two low digits among
//              the candidates, takes keys above T and the lowest-slot keys
//              equal to T (prefix count over a tie bitmap), and writes the
//              ids in ascending order from a prefix count over the bitmap.
//              For short inputs it does the filter pass itself.
// If the threshold bin holds more keys than the candidate buffer, the final
// kernel resolves the low digits with passes over the scores instead.
// Inputs of at most 65,536 slots with no histogram given take one kernel,
// rows: a workgroup per sequence holds the scores in registers, estimates
// the threshold's top digit from a sample, and selects exactly among the
// keys at or above it (or, if the estimate fails, runs the three digit
// passes over all keys).
// Score loads use clamped, unconditional addresses so that a thread's batch
// of loads is in flight together (a conditional load waits on its own).
// All of it is integer work on the keys: exact and independent of timing.
//
// Citation key: [P1] "DeepSeek AI Released DeepSeek-V4.1-Flash with 1M
// Context, FP4 KV Cache, and Cross-Layer Attention Reuse".
#include <algorithm>

#include "common.hpp"
#include "topk_ws.hpp"
#include "select_dev.hpp"

namespace csa2 {
namespace {

constexpr int kFinalThreads = 1024;
constexpr int kFinalWaves = kFinalThreads / 64;
constexpr int kPassThreads = 256;
constexpr int kBatch = 8;                         // slots per thread loaded together
constexpr int kHistSlots = kPassThreads * 16;     // slots per histogram workgroup
constexpr int kFilterSlots = kTopkFilterSlots;     // slots per filter workgroup
static_assert(kFilterSlots == kPassThreads * 32, "filter: 32 slots per thread");
constexpr int kDirectMax = 32768;                 // final kernel filters inputs up to this length itself
constexpr size_t kCandBytes = kTopkCandCap * sizeof(uint2);  // candidate buffer per sequence

__device__ __forceinline__ int64_t valid_slots(int64_t n, const int32_t* lens, int32_t len_div, int b) {
  if (!lens) return n;
  const int64_t L = lens[b];
  return min(n, L > 0 ? (L + len_div - 1) / len_div : 0);
}

// hist[bin] += 1 for every lane with `active`, one LDS atomic per distinct
// bin of the wavefront: cheap when the wavefront's keys share few bins.
// Called by all lanes of the wavefront.
__device__ __forceinline__ void wave_hist_add_grouped(uint32_t* hist, uint32_t bin, bool active) {
  uint64_t pending = __ballot(active);
  while (pending) {
    const int leader = __ffsll((unsigned long long)pending) - 1;
    const uint32_t lb = (uint32_t)__builtin_amdgcn_readlane((int)bin, leader);
    const uint64_t same = __ballot(active && bin == lb);
    if (lane_id() == leader) atomicAdd(&hist[lb], (uint32_t)__popcll(same));
    pending &= ~same;
    active = active && bin != lb;
  }
}

// Threshold state every filter/final workgroup derives from the histogram.
struct Threshold {
  uint32_t total;   // candidates
  uint32_t b1;      // threshold bin of the top digit (valid if total > k)
  uint32_t need1;   // keys still to take from bin b1
  uint32_t in_bin;  // keys in bin b1
};

template <int NT>
__device__ Threshold load_threshold(const uint32_t* __restrict__ ghist, uint32_t* hist, uint32_t* wave_sum,
                                    uint32_t* found, uint32_t k) {
  constexpr int kPer = kTopkBins / NT;
  uint32_t v[kPer];
#pragma unroll
  for (int j = 0; j < kPer; ++j) v[j] = ghist[threadIdx.x + NT * j];  // all loads in flight together
  uint32_t mine = 0;
#pragma unroll
  for (int j = 0; j < kPer; ++j) {
    hist[threadIdx.x + NT * j] = v[j];
    mine += v[j];
  }
  Threshold th;
  block_exclusive_scan<NT>(mine, wave_sum, &th.total);  // syncs: hist complete
  th.b1 = th.need1 = th.in_bin = 0;
  if (th.total > k) {
    find_threshold_bin<NT>(hist, kTopkBins, k, wave_sum, found);
    th.b1 = found[0];
    th.need1 = k - found[1];
    th.in_bin = hist[th.b1];
  }
  return th;
}

// ---------------------------------------------------------------- kernels
__global__ __launch_bounds__(kPassThreads) void topk_hist_kernel(const float* __restrict__ scores, int64_t n,
                                                                 const int32_t* __restrict__ lens,
                                                                 int32_t len_div, uint32_t* __restrict__ ghist) {
  __shared__ uint32_t hist[kTopkBins];
  const int b = blockIdx.y;
  const int64_t nv = valid_slots(n, lens, len_div, b);
  const int64_t s0 = (int64_t)blockIdx.x * kHistSlots;
  if (s0 >= nv) return;
  for (int i = threadIdx.x; i < kTopkBins; i += kPassThreads) hist[i] = 0;
  __syncthreads();
  const float* sc = scores + (int64_t)b * n;
  for (int j0 = 0; j0 < kHistSlots / kPassThreads; j0 += kBatch) {
    uint32_t key[kBatch];
    float v[kBatch];
#pragma unroll
    for (int j = 0; j < kBatch; ++j) v[j] = sc[min(s0 + (j0 + j) * kPassThreads + threadIdx.x, nv - 1)];
#pragma unroll
    for (int j = 0; j < kBatch; ++j) {
      const int64_t i = s0 + (j0 + j) * kPassThreads + threadIdx.x;
      key[j] = i < nv ? order_key(v[j]) : 0u;
      if (key[j]) atomicAdd(&hist[key[j] >> 20], 1u);
    }
  }
  __syncthreads();
  uint32_t* gh = ghist + (int64_t)b * kTopkBins;
  for (int i = threadIdx.x; i < kTopkBins; i += kPassThreads)
    if (hist[i]) atomicAdd(&gh[i], hist[i]);
}

__global__ __launch_bounds__(kPassThreads) void topk_filter_kernel(const float* __restrict__ scores, int64_t n,
                                                                   const int32_t* __restrict__ lens,
                                                                   int32_t len_div, int32_t k, TopkWs ws) {
  constexpr int kPer = kFilterSlots / kPassThreads;  // slots per thread
  __shared__ uint32_t hist[kTopkBins];
  __shared__ uint32_t wave_sum[kPassThreads / 64];
  __shared__ uint32_t found[2];
  const int b = blockIdx.y;
  const int64_t nv = valid_slots(n, lens, len_div, b);
  const int64_t s0 = (int64_t)blockIdx.x * kFilterSlots;
  if (s0 >= nv) return;
  const float* sc = scores + (int64_t)b * n + s0;
  const int nloc = (int)min<int64_t>(nv - s0, kFilterSlots);  // valid slots of this workgroup
  // All of this thread's slots are loaded up front (clamped addresses).
  float v[kPer];
#pragma unroll
  for (int j = 0; j < kPer; ++j) v[j] = sc[min(j * kPassThreads + (int)threadIdx.x, nloc - 1)];
  const Threshold th = load_threshold<kPassThreads>(ws.hist + (int64_t)b * kTopkBins, hist, wave_sum, found,
                                                    (uint32_t)k);
  const bool all = th.total <= (uint32_t)k;
  const bool buffered = th.in_bin <= (uint32_t)kTopkCandCap;
  uint32_t* bits = ws.bits + (int64_t)b * ws.words_cap;
  uint32_t key[kPer];
  uint32_t mine = 0;
  uint32_t* wbits = bits + (s0 >> 5);
#pragma unroll
  for (int j = 0; j < kPer; ++j) {
    const int il = j * kPassThreads + (int)threadIdx.x;  // slot within the workgroup
    key[j] = il < nloc ? order_key(v[j]) : 0u;
    const uint32_t d = key[j] >> 20;
    const uint64_t mask = __ballot(key[j] != 0 && (all || d > th.b1));
    // The wavefront's 64 slots are 64-aligned: lanes 0 and 32 write the two
    // words (every word of the valid range is written exactly once).
    const int w = (il - lane_id()) >> 5;  // word of lanes 0..31; lanes 32..63 use w + 1
    if (lane_id() == 0 && (w << 5) < nloc) wbits[w] = (uint32_t)mask;
    if (lane_id() == 32 && ((w + 1) << 5) < nloc) wbits[w + 1] = (uint32_t)(mask >> 32);
    mine += (key[j] != 0 && d == th.b1) ? 1u : 0u;
  }
  if (all || !buffered) return;
  // Candidates of bin b1 go to this workgroup's own region of the
  // sequence's buffer, positions from a prefix count (no global counter);
  // the count found is written even when the region is too small, and the
  // final pass then rescans the scores instead.
  uint32_t m;
  uint32_t pos = block_exclusive_scan<kPassThreads>(mine, wave_sum, &m);
  const uint32_t per_wg = kTopkCandCap / gridDim.x;
  if (threadIdx.x == 0) ws.wcnt[(int64_t)b * kTopkFilterWgMax + blockIdx.x] = m;
  uint2* gc = ws.cand + (int64_t)b * kTopkCandCap + (int64_t)blockIdx.x * per_wg;
#pragma unroll
  for (int j = 0; j < kPer; ++j) {
    if (key[j] != 0 && (key[j] >> 20) == th.b1) {
      if (pos < per_wg) gc[pos] = make_uint2(key[j], (uint32_t)(s0 + j * kPassThreads + threadIdx.x));
      ++pos;
    }
  }
}

// Many rows of at most kTopkRowsMax slots (a prefill chunk: one row per
// query): the single-workgroup selection would stream each row through one
// CU.  Instead topk_sample_kernel takes each row's threshold estimate from
// kSamples sampled slots (one workgroup per row), and every filter
// workgroup of the row (8,192 slots each) writes the keys at or above it
// to its own region of the row's candidate buffer, with their count.  When the estimate cannot be taken the threshold and the counts
// are kNoEstimate; topk_rows_kernel then selects among the candidates, or
// runs its full passes over the row when an estimate is missing, a region
// overflowed, or the candidates are fewer than k or more than it can hold.
// The row's threshold is kept in the last entry of its wcnt row, which
// filters of at most kTopkRowsMax slots never use.
constexpr int kSamples = 1024;
static_assert(kTopkRowsMax / kTopkFilterSlots < kThresholdSlot, "threshold slot unused by the filter regions");
// Slots of the wcnt rows no filter region uses (at most 8 per row here):
// entry i of the list of rows left to the fallback sits in row i's
// kFallbackSlot; row 0 also holds the list's length and the fallback
// workgroups' claim counter (both zeroed by topk_sample_kernel).
constexpr int kFallbackSlot = kTopkFilterWgMax - 2;
constexpr int kCountSlot = kTopkFilterWgMax - 3;
constexpr int kClaimSlot = kTopkFilterWgMax - 4;
static_assert(kTopkRowsMax / kTopkFilterSlots < kClaimSlot, "list slots unused by the filter regions");

// Sampled slot i of a row of n >= 1,024 slots (i < kSamples): 64 runs of 16
// contiguous slots, one at the start of each 64th of the row (a
// wavefront's samples are four runs: few cache lines per load).
__device__ __forceinline__ int sample_slot(int i, int64_t n) {
  return (i >> 4) * (int)(n >> 6) + (i & 15);
}

__global__ __launch_bounds__(kPassThreads) void topk_sample_kernel(const float* __restrict__ scores, int64_t n,
                                                                   const int32_t* __restrict__ lens,
                                                                   int32_t len_div, int32_t k, TopkWs ws) {
  constexpr int kSmpPer = kSamples / kPassThreads;  // samples per thread
  __shared__ uint32_t hist[kTopkBins];
  __shared__ uint32_t wave_sum[kPassThreads / 64];
  __shared__ uint32_t found[2];
  __shared__ uint32_t n_smp, n_bin, thr_key;
  __shared__ uint32_t bin_keys[kSamples];
  const int tid = threadIdx.x;
  const int b = blockIdx.x;
  const int nv = (int)valid_slots(n, lens, len_div, b);
  const float* sc = scores + (int64_t)b * n;
  const uint32_t kk = (uint32_t)k;
  float sv[kSmpPer];
#pragma unroll
  for (int j = 0; j < kSmpPer; ++j) sv[j] = sc[min(sample_slot(tid + kPassThreads * j, n), (int)n - 1)];
  for (int i = tid; i < kTopkBins; i += kPassThreads) hist[i] = 0;
  if (tid == 0) n_smp = n_bin = 0;
  __syncthreads();
  // The estimate: the r-th largest sampled key, r about twice the samples
  // that k keys would give -- found as the top-digit bin B where the
  // samples counted from the top reach r, then the exact key among the
  // samples of that bin.
  const int r = (int)(((int64_t)2 * kk * kSamples + nv - 1) / max(nv, 1)) + 8;
  uint32_t lo = kNoEstimate;
  if (nv >= 4 * (int)kk && r <= kSamples / 4) {  // uniform over the workgroup
    uint32_t key[kSmpPer];
    uint32_t mine = 0;
#pragma unroll
    for (int j = 0; j < kSmpPer; ++j) {
      key[j] = sample_slot(tid + kPassThreads * j, n) < nv ? order_key(sv[j]) : 0u;
      if (key[j]) {
        atomicAdd(&hist[key[j] >> 20], 1u);
        ++mine;
      }
    }
    const uint32_t wave_n = (uint32_t)wave_inclusive_scan(mine);
    if (lane_id() == 63 && wave_n) atomicAdd(&n_smp, wave_n);
    __syncthreads();
    if (n_smp >= (uint32_t)r) {
      find_threshold_bin<kPassThreads>(hist, kTopkBins, (uint32_t)r, wave_sum, found);
      const uint32_t bin = found[0], need = (uint32_t)r - found[1];  // 1 <= need <= samples in the bin
#pragma unroll
      for (int j = 0; j < kSmpPer; ++j)
        if (key[j] && (key[j] >> 20) == bin) bin_keys[atomicAdd(&n_bin, 1u)] = key[j];
      __syncthreads();
      const uint32_t m = n_bin;
      for (uint32_t i = tid; i < m; i += kPassThreads) {
        const uint32_t v = bin_keys[i];
        uint32_t gt = 0, ge = 0;
        for (uint32_t t = 0; t < m; ++t) {
          const uint32_t u = bin_keys[t];
          gt += u > v ? 1u : 0u;
          ge += u >= v ? 1u : 0u;
        }
        if (gt < need && ge >= need) thr_key = v;  // the need-th largest (equal keys write the same value)
      }
      __syncthreads();
      lo = thr_key;
    }
  }
  if (tid == 0) ws.wcnt[(int64_t)b * kTopkFilterWgMax + kThresholdSlot] = lo;
  if (b == 0 && tid == 0) ws.wcnt[kCountSlot] = ws.wcnt[kClaimSlot] = 0u;
}

// kVec: rows start 16-byte aligned (n % 4 == 0, aligned scores), so each
// thread loads runs of four slots; slot of register j: s0 + 4 * (j / 4 *
// NT + tid) + j % 4 (else s0 + j * NT + tid).
template <bool kVec>
__global__ __launch_bounds__(kPassThreads) void topk_sample_filter_kernel(const float* __restrict__ scores,
                                                                          int64_t n,
                                                                          const int32_t* __restrict__ lens,
                                                                          int32_t len_div, TopkWs ws) {
  constexpr int kPer = kFilterSlots / kPassThreads;  // slots per thread
  __shared__ uint32_t wave_sum[kPassThreads / 64];
  const int tid = threadIdx.x;
  const int b = blockIdx.y;
  const int s0 = blockIdx.x * kFilterSlots;
  // Loads are clamped to the row (n slots), not to the visible part, so
  // that they need no value from memory; visibility applies afterwards.
  const int nrow = min((int)n - s0, kFilterSlots);
  const float* sc = scores + (int64_t)b * n;
  uint32_t* wrow = ws.wcnt + (int64_t)b * kTopkFilterWgMax;
  auto slot_of = [&](int j) {
    return kVec ? 4 * ((j >> 2) * kPassThreads + tid) + (j & 3) : j * kPassThreads + tid;
  };
  float v[kPer];
  if constexpr (kVec) {
    const int last = (nrow - 1) >> 2;  // last 16-byte group of the row
#pragma unroll
    for (int j = 0; j < kPer / 4; ++j) {
      const f32x4 x = reinterpret_cast<const f32x4*>(sc + s0)[min(j * kPassThreads + tid, last)];
      v[4 * j] = x[0], v[4 * j + 1] = x[1], v[4 * j + 2] = x[2], v[4 * j + 3] = x[3];
    }
  } else {
#pragma unroll
    for (int j = 0; j < kPer; ++j) v[j] = sc[s0 + min(slot_of(j), nrow - 1)];
  }
  const int nv = (int)valid_slots(n, lens, len_div, b);
  const int nloc = min(max(nv - s0, 0), kFilterSlots);  // valid slots of this workgroup
  const uint32_t lo = wrow[kThresholdSlot];
  // A slot is a candidate when its key is nonzero and >= lo, i.e. when its
  // score is >= the float whose key lo is (one compare per slot; NaN
  // compares false).  No early return on a missing estimate: its threshold
  // is a NaN, which nothing passes.
  const float t = key_threshold(lo);
  uint32_t cnt = 0;
#pragma unroll
  for (int j = 0; j < kPer; ++j) cnt += (v[j] >= t && slot_of(j) < nloc) ? 1u : 0u;
  uint32_t total;
  uint32_t pos = block_exclusive_scan<kPassThreads>(cnt, wave_sum, &total);
  const uint32_t per_wg = kTopkCandCap / gridDim.x;
  if (tid == 0) wrow[blockIdx.x] = lo == kNoEstimate ? kNoEstimate : total;
  uint2* gc = ws.cand + (int64_t)b * kTopkCandCap + (int64_t)blockIdx.x * per_wg;
#pragma unroll
  for (int j = 0; j < kPer; ++j) {
    if (v[j] >= t && slot_of(j) < nloc) {
      if (pos < per_wg) gc[pos] = make_uint2(order_key(v[j]), (uint32_t)(s0 + slot_of(j)));
      ++pos;
    }
  }
}

// Words w0 + kG*kQc*r + i (i < kG*kQc) of a bitmap: kQc groups of kG words
// (kG = 4: 16-byte loads) of round r of a thread's run, loaded together
// (clamped to the last group, which exists), words at or past w1 read as 0.
template <int kG, int kQc>
__device__ __forceinline__ void load_round(const uint32_t* bm, int q0, int r, int qmax, int w0, int w1,
                                           uint32_t (&wv)[kG * kQc]) {
#pragma unroll
  for (int j = 0; j < kQc; ++j) {
    const int q = min(q0 + kQc * r + j, qmax);
    if constexpr (kG == 4) {
      const u32x4 v = reinterpret_cast<const u32x4*>(bm)[q];
      wv[4 * j] = v[0], wv[4 * j + 1] = v[1], wv[4 * j + 2] = v[2], wv[4 * j + 3] = v[3];
    } else {
      wv[j] = bm[q];
    }
  }
#pragma unroll
  for (int i = 0; i < kG * kQc; ++i)
    if (w0 + kG * kQc * r + i >= w1) wv[i] = 0u;
}

// Selection bitmap sel (and, if ties > 0, the tie bitmap tie: keys equal to
// the threshold) of one sequence, in LDS -> the ids in ascending order.
// Every thread owns a contiguous run of words; one scan gives, per run, the
// selected and the tie bits before it.  The lowest `ties` tie bits join the
// selection, so a run's first output position is (selected before) +
// min(ties before, ties).  -1 pads the row to k.  fin_sum: 2 * NT / 64
// words used by nothing else; the caller has synchronised after its last
// write of sel / tie.  Called by all NT threads of the workgroup.
template <int NT = kFinalThreads>
__device__ void finish_output_lds(const uint32_t* sel, const uint32_t* tie, int words, uint32_t ties, uint32_t kk,
                                  const int32_t* pool_lds, int32_t blk, uint32_t* fin_sum,
                                  int32_t* __restrict__ ob, const int32_t* __restrict__ gid = nullptr) {
  const int tid = threadIdx.x;
  const int per = (words + NT - 1) / NT;
  const int w0 = min(words, tid * per), w1 = min(words, w0 + per);
  uint2 cnt = make_uint2(0u, 0u);
  for (int w = w0; w < w1; ++w) {
    cnt.x += __popc(sel[w]);
    if (ties > 0) cnt.y += __popc(tie[w]);
  }
  uint2 tot;
  const uint2 before = block_exclusive_scan2_once<NT>(cnt, fin_sum, &tot);
  uint32_t pos = before.x + min(before.y, ties);
  uint32_t trank = before.y;  // tie bits before the current word
  for (int w = w0; w < w1; ++w) {
    uint32_t x = sel[w];
    if (ties > 0 && trank < ties) {
      uint32_t t = tie[w];
      const uint32_t pc = __popc(t);
      if (trank + pc <= ties) {
        x |= t;
      } else {
        for (uint32_t m = trank; m < ties; ++m) {
          x |= t & (0u - t);
          t &= t - 1;
        }
      }
      trank += pc;
    }
    while (x) {
      const int bit = __ffs(x) - 1;
      x &= x - 1;
      const int64_t slot = (int64_t)w * 32 + bit;
      int64_t id = slot;
      if (pool_lds) id = (int64_t)pool_lds[slot / blk] * blk + slot % blk;
      if (gid) id = gid[slot];
      if (pos < kk) ob[pos] = (int32_t)id;
      ++pos;
    }
  }
  const uint32_t n_sel = tot.x + min(tot.y, ties);
  for (uint32_t i = n_sel + tid; i < kk; i += NT) ob[i] = -1;
}

// Words w0 + 16*r + i (i < 16) of a global bitmap: four 16-byte groups of
// round r of a thread's run, loaded together (clamped to the last group,
// which exists), words at or past w1 read as 0.
__device__ __forceinline__ void load_round(const uint32_t* bm, int q0, int r, int qmax, int w0, int w1,
                                           uint32_t (&wv)[16]) {
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const u32x4 v = reinterpret_cast<const u32x4*>(bm)[min(q0 + 4 * r + j, qmax)];
    wv[4 * j] = v[0], wv[4 * j + 1] = v[1], wv[4 * j + 2] = v[2], wv[4 * j + 3] = v[3];
  }
#pragma unroll
  for (int i = 0; i < 16; ++i)
    if (w0 + 16 * r + i >= w1) wv[i] = 0u;
}

// The same for bitmaps in global memory (16-byte aligned; inputs longer
// than the LDS bitmaps), last written by other threads of this workgroup
// before a barrier or by an earlier kernel.  Every thread owns a contiguous
// run of 16-byte groups, read in rounds of four groups whose loads are in
// flight together: a prefix count over the tie words adds the lowest `ties`
// tie slots to the thread's own sel words, then a prefix count over the sel
// words gives each thread the output position of its ids.
__device__ void finish_output_global(uint32_t* sel, const uint32_t* tie, int words, uint32_t ties, uint32_t kk,
                                     const int32_t* pool_lds, int32_t blk, uint32_t* wave_sum,
                                     int32_t* __restrict__ ob) {
  const int tid = threadIdx.x;
  const int nq = (words + 3) / 4;
  const int perq = (nq + kFinalThreads - 1) / kFinalThreads;
  const int rounds = (perq + 3) / 4;
  const int q0 = min(nq, tid * perq);
  const int qmax = max(nq - 1, 0);
  const int w0 = 4 * q0, w1 = min(words, 4 * (q0 + perq));  // this thread's words
  uint32_t wv[16];
  if (ties > 0) {
    uint32_t cnt = 0;
#pragma unroll 1
    for (int r = 0; r < rounds; ++r) {
      load_round(tie, q0, r, qmax, w0, w1, wv);
#pragma unroll
      for (int i = 0; i < 16; ++i) cnt += __popc(wv[i]);
    }
    uint32_t dummy;
    uint32_t rank = block_exclusive_scan<kFinalThreads>(cnt, wave_sum, &dummy);
#pragma unroll 1
    for (int r = 0; r < rounds && rank < ties; ++r) {
      load_round(tie, q0, r, qmax, w0, w1, wv);
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        uint32_t x = wv[i];
        const uint32_t pc = __popc(x);
        if (rank < ties && x) {
          uint32_t keep = x;
          if (rank + pc > ties) {
            keep = 0;
            for (uint32_t m = rank; m < ties; ++m) {
              keep |= x & (0u - x);
              x &= x - 1;
            }
          }
          sel[w0 + 16 * r + i] |= keep;  // the thread's own word
        }
        rank += pc;
      }
    }
  }
  uint32_t cnt = 0;
#pragma unroll 1
  for (int r = 0; r < rounds; ++r) {
    load_round(sel, q0, r, qmax, w0, w1, wv);
#pragma unroll
    for (int i = 0; i < 16; ++i) cnt += __popc(wv[i]);
  }
  uint32_t n_sel;
  uint32_t pos = block_exclusive_scan<kFinalThreads>(cnt, wave_sum, &n_sel);
#pragma unroll 1
  for (int r = 0; r < rounds && pos < kk; ++r) {
    load_round(sel, q0, r, qmax, w0, w1, wv);
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      uint32_t x = wv[i];
      while (x) {
        const int bit = __ffs(x) - 1;
        x &= x - 1;
        const int64_t slot = (int64_t)(w0 + 16 * r + i) * 32 + bit;
        int64_t id = slot;
        if (pool_lds) id = (int64_t)pool_lds[slot / blk] * blk + slot % blk;
        if (pos < kk) ob[pos] = (int32_t)id;
        ++pos;
      }
    }
  }
  for (uint32_t i = n_sel + tid; i < kk; i += kFinalThreads) ob[i] = -1;
}

struct FinalSmem {
  int32_t pool[CSA2_TOPK_MAX];  // the sequence's pool block ids (pool mode)
  uint32_t hist[kTopkBins];
  uint32_t sel[kTopkLdsWords];
  uint32_t tie[kTopkLdsWords];
  uint32_t cand_key[kTopkCandCap];
  uint32_t cand_slot[kTopkCandCap];
  uint32_t wc_off[kTopkFilterWgMax];  // first LDS candidate of each filter workgroup
  uint32_t wc_cnt[kTopkFilterWgMax];  // its candidate count
  uint32_t wave_sum[kFinalWaves];
  uint32_t fin_sum[2 * kFinalWaves];  // the output scan's own
  uint32_t found[2];
};

// kGlobal: the selection and tie bitmaps stay in global memory (inputs of
// more than kTopkLdsWords * 32 slots): the filter pass's bitmap is marked in
// place and the tie bitmap is cleared here first.
template <bool kGlobal>
__global__ __launch_bounds__(kFinalThreads) void topk_final_kernel(const float* __restrict__ scores, int64_t n,
                                                                   const int32_t* __restrict__ lens,
                                                                   int32_t len_div, int32_t k,
                                                                   const int32_t* __restrict__ pool,
                                                                   int32_t n_pool, int32_t blk, TopkWs ws,
                                                                   int32_t* __restrict__ out) {
  extern __shared__ __attribute__((aligned(16))) unsigned char smem_raw[];
  FinalSmem& sm = *reinterpret_cast<FinalSmem*>(smem_raw);
  const int b = blockIdx.x;
  const int tid = threadIdx.x;
  const int nvalid = (int)valid_slots(n, lens, len_div, b);
  const int words = (nvalid + 31) / 32;
  const bool direct = !kGlobal && n <= kDirectMax;  // kGlobal inputs are longer
  const float* sc = scores + (int64_t)b * n;
  const uint32_t kk = (uint32_t)k;
  uint32_t* gh = ws.hist + (int64_t)b * kTopkBins;

  // Direct path: this thread's scores are loaded first (clamped), overlapping
  // the histogram and pool loads.
  constexpr int kPerDirect = kDirectMax / kFinalThreads;
  float dv[kPerDirect];
  if (direct) {
#pragma unroll
    for (int j = 0; j < kPerDirect; ++j) dv[j] = sc[min(j * kFinalThreads + tid, max(nvalid - 1, 0))];
  }
  if (pool) {  // staged for the id mapping at the end (n_pool <= CSA2_TOPK_MAX)
    const int32_t* pb = pool + (int64_t)b * n_pool;
    int32_t pv[CSA2_TOPK_MAX / kFinalThreads];
#pragma unroll
    for (int j = 0; j < CSA2_TOPK_MAX / kFinalThreads; ++j) pv[j] = pb[min(tid + kFinalThreads * j, n_pool - 1)];
#pragma unroll
    for (int j = 0; j < CSA2_TOPK_MAX / kFinalThreads; ++j)
      if (tid + kFinalThreads * j < n_pool) sm.pool[tid + kFinalThreads * j] = pv[j];
  }
  const Threshold th = load_threshold<kFinalThreads>(gh, sm.hist, sm.wave_sum, sm.found, kk);
  // The global histogram is consumed: leave it zero for the next call.
  for (int i = tid; i < kTopkBins; i += kFinalThreads) gh[i] = 0;

  const bool all = th.total <= kk;
  bool buffered = th.in_bin <= (uint32_t)kTopkCandCap;
  uint32_t* sel = kGlobal ? ws.bits + (int64_t)b * ws.words_cap : sm.sel;
  uint32_t* tie = kGlobal ? ws.tie + (int64_t)b * ws.words_cap : sm.tie;
  for (int i = tid; i < words; i += kFinalThreads) tie[i] = 0u;
  if (direct) {
    // Filter pass in this workgroup (scores already loaded).
    constexpr int kPer = kPerDirect;
    for (int i = tid; i < words; i += kFinalThreads) sm.sel[i] = 0;
    __syncthreads();
    uint32_t key[kPer];
    uint32_t mine = 0;
#pragma unroll
    for (int j = 0; j < kPer; ++j) {
      const int i = j * kFinalThreads + tid;
      key[j] = i < nvalid ? order_key(dv[j]) : 0u;
      const uint32_t d = key[j] >> 20;
      const uint64_t mask = __ballot(key[j] != 0 && (all || d > th.b1));
      const int w = (i - lane_id()) >> 5;
      if (lane_id() == 0 && (uint32_t)mask) sm.sel[w] = (uint32_t)mask;
      if (lane_id() == 32 && (uint32_t)(mask >> 32)) sm.sel[w + 1] = (uint32_t)(mask >> 32);
      mine += (key[j] != 0 && d == th.b1) ? 1u : 0u;
    }
    if (!all && buffered) {
      uint32_t dummy;
      uint32_t pos = block_exclusive_scan<kFinalThreads>(mine, sm.wave_sum, &dummy);
#pragma unroll
      for (int j = 0; j < kPer; ++j) {
        if (key[j] != 0 && (key[j] >> 20) == th.b1) {
          sm.cand_key[pos] = key[j];
          sm.cand_slot[pos] = (uint32_t)(j * kFinalThreads + tid);
          ++pos;
        }
      }
    }
  } else {
    // Bitmap (into LDS unless kGlobal) and candidates of the filter pass;
    // clamped loads, all in flight together.
    if (!kGlobal) {
      const uint32_t* gb = ws.bits + (int64_t)b * ws.words_cap;
      constexpr int kWordsPer = kTopkLdsWords / kFinalThreads;
      uint32_t wv[kWordsPer];
#pragma unroll
      for (int j = 0; j < kWordsPer; ++j) wv[j] = gb[min(tid + kFinalThreads * j, max(words - 1, 0))];
#pragma unroll
      for (int j = 0; j < kWordsPer; ++j)
        if (tid + kFinalThreads * j < words) sm.sel[tid + kFinalThreads * j] = wv[j];
    }
    if (!all && buffered) {
      // Candidates of the filter pass: filter workgroup w kept up to per_wg
      // of them in its own region.  Their counts' prefix sum places them in
      // LDS (eight threads per workgroup region); if a region overflowed, or
      // the counts do not add up to the histogram's, the scores are rescanned.
      const int nw = (int)((n + kFilterSlots - 1) / kFilterSlots);
      const int nwv = (nvalid + kFilterSlots - 1) / kFilterSlots;
      const uint32_t per_wg = kTopkCandCap / nw;
      const uint32_t c = tid < nwv ? ws.wcnt[(int64_t)b * kTopkFilterWgMax + tid] : 0u;
      uint32_t total;
      const uint32_t off = block_exclusive_scan<kFinalThreads>(c, sm.wave_sum, &total);
      if (tid < nwv) {
        sm.wc_off[tid] = off;
        sm.wc_cnt[tid] = c;
      }
      buffered = __syncthreads_or(c > per_wg) == 0 && total == th.in_bin;
      if (buffered) {
        const int w = tid >> 3;
        if (w < nwv) {
          const uint32_t cw = sm.wc_cnt[w], ow = sm.wc_off[w];
          const uint2* gc = ws.cand + (int64_t)b * kTopkCandCap + (int64_t)w * per_wg;
          // 64 candidates of the region per pass, eight loads per thread in
          // flight together (clamped to the region's last candidate).
          for (uint32_t i0 = 0; i0 < cw; i0 += 64) {
            uint2 v[8];
#pragma unroll
            for (int r = 0; r < 8; ++r) v[r] = gc[min(i0 + (tid & 7) + 8 * r, cw - 1)];
#pragma unroll
            for (int r = 0; r < 8; ++r) {
              const uint32_t i = i0 + (tid & 7) + 8 * r;
              if (i < cw) {
                sm.cand_key[ow + i] = v[r].x;
                sm.cand_slot[ow + i] = v[r].y;
              }
            }
          }
        }
      }
    }
  }
  __syncthreads();

  uint32_t ties = 0;
  if (!all) {
    const int nc = (int)th.in_bin;
    const int nc_round = (nc + kFinalThreads - 1) / kFinalThreads * kFinalThreads;
    for (int i = tid; i < kTopkBins; i += kFinalThreads) sm.hist[i] = 0;
    __syncthreads();
    // Digit 2: bits 19..8 among the keys of bin b1.
    if (buffered) {
      for (int c = tid; c < nc; c += kFinalThreads) atomicAdd(&sm.hist[(sm.cand_key[c] >> 8) & 0xFFFu], 1u);
    } else {
      for (int i = tid; i < nvalid; i += kFinalThreads) {
        const uint32_t key = order_key(sc[i]);
        if (key && (key >> 20) == th.b1) atomicAdd(&sm.hist[(key >> 8) & 0xFFFu], 1u);
      }
    }
    __syncthreads();
    find_threshold_bin<kFinalThreads>(sm.hist, kTopkBins, th.need1, sm.wave_sum, sm.found);
    const uint32_t b2 = sm.found[0];
    const uint32_t need2 = th.need1 - sm.found[1];
    for (int i = tid; i < 256; i += kFinalThreads) sm.hist[i] = 0;
    __syncthreads();
    const uint32_t pre2 = (th.b1 << 12) | b2;
    // Digit 3: bits 7..0 among keys with the first two digits (integer-valued
    // scores share their low bits: group the atomics per wavefront).
    if (buffered) {
      for (int c = tid; c < nc_round; c += kFinalThreads) {
        const uint32_t key = c < nc ? sm.cand_key[c] : 0u;
        wave_hist_add_grouped(sm.hist, key & 0xFFu, c < nc && (key >> 8) == pre2);
      }
    } else {
      const int nv_round = (nvalid + kFinalThreads - 1) / kFinalThreads * kFinalThreads;
      for (int i = tid; i < nv_round; i += kFinalThreads) {
        const uint32_t key = i < nvalid ? order_key(sc[i]) : 0u;
        wave_hist_add_grouped(sm.hist, key & 0xFFu, key != 0 && (key >> 8) == pre2);
      }
    }
    __syncthreads();
    find_threshold_bin<kFinalThreads>(sm.hist, 256, need2, sm.wave_sum, sm.found);
    const uint32_t T = (pre2 << 8) | sm.found[0];
    ties = need2 - sm.found[1];
    // Keys of bin b1 above T are selected, keys equal to T are tie candidates.
    if (buffered) {
      for (int c = tid; c < nc; c += kFinalThreads) {
        const uint32_t key = sm.cand_key[c], i = sm.cand_slot[c];
        if (key > T) atomicOr(&sel[i >> 5], 1u << (i & 31));
        else if (key == T) atomicOr(&tie[i >> 5], 1u << (i & 31));
      }
    } else {
      for (int i = tid; i < nvalid; i += kFinalThreads) {
        const uint32_t key = order_key(sc[i]);
        if (!key || (key >> 20) != th.b1) continue;
        if (key > T) atomicOr(&sel[i >> 5], 1u << (i & 31));
        else if (key == T) atomicOr(&tie[i >> 5], 1u << (i & 31));
      }
    }
    __syncthreads();
  }

  if constexpr (kGlobal)
    finish_output_global(sel, tie, words, ties, kk, pool ? sm.pool : nullptr, blk, sm.wave_sum, out + (int64_t)b * k);
  else
    finish_output_lds(sel, tie, words, ties, kk, pool ? sm.pool : nullptr, blk, sm.fin_sum, out + (int64_t)b * k);
}


// Whole selection of one sequence of at most kRowsMax slots in one
// workgroup, the scores held in registers (kPer per thread): three histogram
// passes over the keys in LDS (digits of 12, 12 and 8 bits) find the exact
// k-th key T, then selection and tie bitmaps are written by ballots and
// finish_output_lds emits the ids.  Reads every score once; used when no
// histogram was produced upstream (many sequences of moderate length).
constexpr int kRowsMax = 64 * kFinalThreads;  // 65,536 slots
static_assert(kRowsMax == kTopkRowsMax, "register-resident selection length");

constexpr int kRowsCand = 8192;  // keys kept by the sampled first pass
constexpr int kManyRows = 256;   // rows from which long rows take the multi-workgroup filter
constexpr int kFlaggedGrid = 256;  // workgroups walking the rows that need the full selection

struct RowsSmem {
  int32_t pool[CSA2_TOPK_MAX];
  uint32_t hist[kTopkBins];   // the samples' top digits; the full passes' digits
  uint32_t hist1[kTopkBins];  // top digit of the candidates
  uint32_t hist2[kTopkBins];  // middle digit of the candidates in the threshold bin
  uint32_t hist3[256];        // low digit
  uint32_t sel[kRowsMax / 32];
  uint32_t tie[kRowsMax / 32];
  uint32_t cand_key[kRowsCand];
  uint32_t cand_slot[kRowsCand];
  uint32_t wave_sum[kFinalWaves];
  uint32_t scan_sum[4][kFinalWaves];  // one per scan of the sampled path (never reused)
  uint32_t fin_sum[2 * kFinalWaves];  // the output scan's own
  uint32_t counter[2];                // sampled keys, candidates
  uint32_t found[2];
};

static_assert(sizeof(RowsSmem) <= 160 * 1024, "one workgroup's LDS");

// The exact kk-th largest key T among the nc candidate keys ck[0..nc)
// (1 <= kk <= nc) and how many keys equal to T are taken (ties), given the
// candidates' top-digit histogram hist1 (complete, and hist2 / hist3 zero):
// radix select over digits of 12, 12 and 8 bits, every thread taking keys
// tid, tid + NT, ...  kGrouped: one LDS atomic per distinct bin and
// wavefront (wave_hist_add_grouped) instead of one per key -- for keys that
// crowd into few bins, such as integer-valued scores, whose low bits are
// all equal.  Called by the whole workgroup.
template <int NT, bool kGrouped = false>
__device__ void select_candidates(const uint32_t* ck, int nc, uint32_t kk, const uint32_t* hist1,
                                  uint32_t* hist2, uint32_t* hist3, uint32_t (*scan_sum)[NT / 64],
                                  uint32_t* found, uint32_t& T, uint32_t& ties) {
  const int tid = threadIdx.x;
  find_threshold_bin_once<NT>(hist1, kTopkBins, kk, scan_sum[1], found);
  const uint32_t b1 = found[0];
  const uint32_t need1 = kk - found[1];
  if (kGrouped) {
    for (int base = tid - lane_id(); base < nc; base += NT) {  // uniform over each wavefront
      const int c = base + lane_id();
      const uint32_t key = c < nc ? ck[c] : 0u;
      wave_hist_add_grouped(hist2, (key >> 8) & 0xFFFu, c < nc && (key >> 20) == b1);
    }
  } else {
    for (int c = tid; c < nc; c += NT) {
      const uint32_t key = ck[c];
      if ((key >> 20) == b1) atomicAdd(&hist2[(key >> 8) & 0xFFFu], 1u);
    }
  }
  __syncthreads();
  find_threshold_bin_once<NT>(hist2, kTopkBins, need1, scan_sum[2], found);
  const uint32_t pre2 = (b1 << 12) | found[0];
  const uint32_t need2 = need1 - found[1];
  if (kGrouped) {
    for (int base = tid - lane_id(); base < nc; base += NT) {
      const int c = base + lane_id();
      const uint32_t key = c < nc ? ck[c] : 0u;
      wave_hist_add_grouped(hist3, key & 0xFFu, c < nc && (key >> 8) == pre2);
    }
  } else {
    for (int c = tid; c < nc; c += NT) {
      const uint32_t key = ck[c];
      if ((key >> 8) == pre2) atomicAdd(&hist3[key & 0xFFu], 1u);
    }
  }
  __syncthreads();
  find_threshold_bin_once<NT>(hist3, 256, need2, scan_sum[3], found);
  T = (pre2 << 8) | found[0];
  ties = need2 - found[1];
}

// kCandIn: the row's candidates come from topk_sample_filter_kernel (cand_in
// [n_seq][kTopkCandCap], wcnt_in [n_seq][kTopkFilterWgMax]) instead of the
// sampled first pass here; the scores are loaded only if the full passes
// have to run.
// The selection of row b by the whole workgroup (kFinalThreads threads).
template <int kRowsPer, bool kCandIn>
__device__ void rows_select(RowsSmem& sm, const int b, const float* __restrict__ scores, int64_t n,
                            const int32_t* __restrict__ lens, int32_t len_div, int32_t k,
                            const int32_t* __restrict__ pool, int32_t n_pool, int32_t blk, int32_t* __restrict__ out,
                            const int32_t* __restrict__ gids, const uint2* __restrict__ cand_in,
                            const uint32_t* __restrict__ wcnt_in) {
  // gids: [n_seq][n] ids emitted for the slots (else the slot, or the pool's)
  const int32_t* gid = gids ? gids + (int64_t)b * n : nullptr;
  const int tid = threadIdx.x;
  const int nvalid = (int)valid_slots(n, lens, len_div, b);
  const int words = (nvalid + 31) / 32;
  const float* sc = scores + (int64_t)b * n;
  const uint32_t kk = (uint32_t)k;

  // Slot of register j of this thread: j * kFinalThreads + tid (a
  // wavefront's 64 slots are contiguous and 64-aligned).
  uint32_t key[kRowsPer];
  auto load_keys = [&]() {
    float v[kRowsPer];
#pragma unroll
    for (int j = 0; j < kRowsPer; ++j) v[j] = sc[min(j * kFinalThreads + tid, max(nvalid - 1, 0))];
#pragma unroll
    for (int j = 0; j < kRowsPer; ++j) key[j] = (j * kFinalThreads + tid < nvalid) ? order_key(v[j]) : 0u;
  };
  if constexpr (!kCandIn) load_keys();
  if (pool) {
    const int32_t* pb = pool + (int64_t)b * n_pool;
    for (int i = tid; i < n_pool; i += kFinalThreads) sm.pool[i] = pb[i];
  }
  for (int i = tid; i < kTopkBins; i += kFinalThreads) sm.hist[i] = sm.hist1[i] = sm.hist2[i] = 0;
  if (tid < 256) sm.hist3[tid] = 0;
  for (int i = tid; i < words; i += kFinalThreads) sm.sel[i] = sm.tie[i] = 0;
  if (tid < 2) sm.counter[tid] = 0;
  __syncthreads();

  if constexpr (kCandIn) {
    // Candidates from the filter workgroups' regions: usable if every
    // region holds its whole count and together they are k .. kRowsCand.
    const int n_wg = (int)((n + kFilterSlots - 1) / kFilterSlots);
    static_assert(kRowsMax / kTopkFilterSlots == 8, "at most 8 filter regions per row");
    const uint32_t per_wg = kTopkCandCap / n_wg;
    const uint32_t* wc = wcnt_in + (int64_t)b * kTopkFilterWgMax;
    uint32_t cw[8], off[8], total = 0;
    bool ok = true;
#pragma unroll
    for (int w = 0; w < 8; ++w) {
      cw[w] = w < n_wg ? wc[w] : 0u;
      ok = ok && cw[w] != kNoEstimate && cw[w] <= per_wg;
      off[w] = total;
      total += ok ? cw[w] : 0u;
    }
    if (ok && total >= kk && total <= (uint32_t)kRowsCand) {  // uniform over the workgroup
      // Candidate c = tid + j * NT of the concatenated regions: all of a
      // thread's loads in flight together (clamped addresses).
      const uint2* gc = cand_in + (int64_t)b * kTopkCandCap;
      constexpr int kCandPer = kRowsCand / kFinalThreads;
      uint2 e[kCandPer];
#pragma unroll
      for (int j = 0; j < kCandPer; ++j) {
        const uint32_t c = tid + j * kFinalThreads;
        uint32_t src = 0;
#pragma unroll
        for (int w = 0; w < 8; ++w)
          if (c >= off[w] && c < off[w] + cw[w]) src = w * per_wg + (c - off[w]);
        e[j] = gc[src];
      }
#pragma unroll
      for (int j = 0; j < kCandPer; ++j) {
        const uint32_t c = tid + j * kFinalThreads;
        if (c < total) {
          sm.cand_key[c] = e[j].x;
          sm.cand_slot[c] = e[j].y;
          atomicAdd(&sm.hist1[e[j].x >> 20], 1u);
        }
      }
      __syncthreads();
      uint32_t T, ties;
      select_candidates<kFinalThreads>(sm.cand_key, (int)total, kk, sm.hist1, sm.hist2, sm.hist3, sm.scan_sum,
                                       sm.found, T, ties);
      for (int c = tid; c < (int)total; c += kFinalThreads) {
        const uint32_t key = sm.cand_key[c], i = sm.cand_slot[c];
        if (key > T) atomicOr(&sm.sel[i >> 5], 1u << (i & 31));
        else if (key == T) atomicOr(&sm.tie[i >> 5], 1u << (i & 31));
      }
      __syncthreads();
      finish_output_lds(sm.sel, sm.tie, words, ties, kk, pool ? sm.pool : nullptr, blk, sm.fin_sum,
                        out + (int64_t)b * k, gid);
      return;
    }
    load_keys();
  }

  // Sampled first pass.  One key per thread (slot (tid % kRowsPer) * NT +
  // tid, spread over the row) estimates a lower bound B for the top digit
  // of the k-th key: the bin where the samples counted from the top reach
  // r, about twice the samples that k keys would give.  Every key in bins
  // >= B then goes to an LDS list (positions from a wavefront scan and one
  // LDS atomic per wavefront, so the list is unordered; the top-digit
  // histogram of the list is counted on the way), from which the exact
  // threshold is selected -- if the list holds at least k keys (so it
  // contains the k largest) and fits.  Otherwise the full passes below run.
  // Each scan here has its own wave-sum slot, so none needs a second
  // barrier.
  if constexpr (!kCandIn) {
    const int r = (int)(((int64_t)2 * kk * kFinalThreads + nvalid - 1) / max(nvalid, 1)) + 8;
    if (nvalid >= 4 * (int)kk && r <= kFinalThreads / 4) {  // uniform over the workgroup
      uint32_t smp = 0;
#pragma unroll
      for (int j = 0; j < kRowsPer; ++j)
        if (j == tid % kRowsPer) smp = key[j];
      if (smp) atomicAdd(&sm.hist[smp >> 20], 1u);
      const uint64_t has = __ballot(smp != 0);
      if (lane_id() == 0) atomicAdd(&sm.counter[0], (uint32_t)__popcll(has));
      __syncthreads();  // sample histogram and count complete
      if (sm.counter[0] >= (uint32_t)r) {
        find_threshold_bin_once<kFinalThreads>(sm.hist, kTopkBins, (uint32_t)r, sm.scan_sum[0], sm.found);
        const uint32_t lo = sm.found[0] << 20;  // keys >= lo are kept
        uint32_t cnt = 0;
#pragma unroll
        for (int j = 0; j < kRowsPer; ++j) cnt += (key[j] >= lo && key[j] != 0) ? 1u : 0u;
        const uint32_t incl = wave_inclusive_scan(cnt);
        uint32_t base = 0;
        if (lane_id() == 63) base = atomicAdd(&sm.counter[1], incl);
        uint32_t pos = (uint32_t)__builtin_amdgcn_readlane((int)base, 63) + incl - cnt;
#pragma unroll
        for (int j = 0; j < kRowsPer; ++j) {
          if (key[j] >= lo && key[j] != 0) {
            if (pos < (uint32_t)kRowsCand) {
              sm.cand_key[pos] = key[j];
              sm.cand_slot[pos] = (uint32_t)(j * kFinalThreads + tid);
            }
            atomicAdd(&sm.hist1[key[j] >> 20], 1u);
            ++pos;
          }
        }
        __syncthreads();  // list, its histogram and its length complete
        const uint32_t n_cand = sm.counter[1];
        if (n_cand >= kk && n_cand <= (uint32_t)kRowsCand) {
          uint32_t T, ties;
          select_candidates<kFinalThreads>(sm.cand_key, (int)n_cand, kk, sm.hist1, sm.hist2, sm.hist3,
                                           sm.scan_sum, sm.found, T, ties);
          for (int c = tid; c < (int)n_cand; c += kFinalThreads) {
            const uint32_t key = sm.cand_key[c], i = sm.cand_slot[c];
            if (key > T) atomicOr(&sm.sel[i >> 5], 1u << (i & 31));
            else if (key == T) atomicOr(&sm.tie[i >> 5], 1u << (i & 31));
          }
          __syncthreads();
          finish_output_lds(sm.sel, sm.tie, words, ties, kk, pool ? sm.pool : nullptr, blk, sm.fin_sum,
                            out + (int64_t)b * k, gid);
          return;
        }
      }
      // The estimate did not hold: clear the sample histogram and run the
      // full passes.
      for (int i = tid; i < kTopkBins; i += kFinalThreads) sm.hist[i] = 0;
      __syncthreads();
    }
  }

  // Digit 1: bits 31..20.
  uint32_t mine = 0;
#pragma unroll
  for (int j = 0; j < kRowsPer; ++j) {
    if (key[j]) {
      atomicAdd(&sm.hist[key[j] >> 20], 1u);
      ++mine;
    }
  }
  uint32_t total;
  block_exclusive_scan<kFinalThreads>(mine, sm.wave_sum, &total);  // syncs: histogram complete
  uint32_t T = 1u, ties = 0;  // with every candidate selected: key >= 1
  if (total > kk) {
    find_threshold_bin<kFinalThreads>(sm.hist, kTopkBins, kk, sm.wave_sum, sm.found);
    const uint32_t b1 = sm.found[0];
    const uint32_t need1 = kk - sm.found[1];
    for (int i = tid; i < kTopkBins; i += kFinalThreads) sm.hist[i] = 0;
    __syncthreads();
    // Digit 2: bits 19..8 among the keys of bin b1.
#pragma unroll
    for (int j = 0; j < kRowsPer; ++j)
      if (key[j] && (key[j] >> 20) == b1) atomicAdd(&sm.hist[(key[j] >> 8) & 0xFFFu], 1u);
    __syncthreads();
    find_threshold_bin<kFinalThreads>(sm.hist, kTopkBins, need1, sm.wave_sum, sm.found);
    const uint32_t b2 = sm.found[0];
    const uint32_t need2 = need1 - sm.found[1];
    for (int i = tid; i < 256; i += kFinalThreads) sm.hist[i] = 0;
    __syncthreads();
    const uint32_t pre2 = (b1 << 12) | b2;
    // Digit 3: bits 7..0 (integer-valued scores share their low bits: the
    // atomics are grouped per wavefront).
#pragma unroll
    for (int j = 0; j < kRowsPer; ++j) wave_hist_add_grouped(sm.hist, key[j] & 0xFFu, key[j] && (key[j] >> 8) == pre2);
    __syncthreads();
    find_threshold_bin<kFinalThreads>(sm.hist, 256, need2, sm.wave_sum, sm.found);
    T = (pre2 << 8) | sm.found[0];
    ties = need2 - sm.found[1];
  }
  // Keys above T are selected; keys equal to T are tie candidates (only the
  // lowest `ties` of them are kept).  Lanes 0 and 32 write the two words of
  // their wavefront's 64 slots; every word of the valid range is written.
#pragma unroll
  for (int j = 0; j < kRowsPer; ++j) {
    const int i = j * kFinalThreads + tid;
    const bool take = ties > 0 ? key[j] > T : key[j] >= T;
    const uint64_t ms = __ballot(take);
    const uint64_t mt = __ballot(ties > 0 && key[j] == T);
    const int w = (i - lane_id()) >> 5;
    if (lane_id() == 0 && w < words) {
      sm.sel[w] = (uint32_t)ms;
      sm.tie[w] = (uint32_t)mt;
    }
    if (lane_id() == 32 && w + 1 < words) {
      sm.sel[w + 1] = (uint32_t)(ms >> 32);
      sm.tie[w + 1] = (uint32_t)(mt >> 32);
    }
  }
  __syncthreads();
  finish_output_lds(sm.sel, sm.tie, words, ties, kk, pool ? sm.pool : nullptr, blk, sm.fin_sum,
                    out + (int64_t)b * k, gid);
}


template <int kRowsPer, bool kCandIn = false>
__global__ __launch_bounds__(kFinalThreads) void topk_rows_kernel(const float* __restrict__ scores, int64_t n,
                                                                  const int32_t* __restrict__ lens,
                                                                  int32_t len_div, int32_t k,
                                                                  const int32_t* __restrict__ pool,
                                                                  int32_t n_pool, int32_t blk,
                                                                  int32_t* __restrict__ out,
                                                                  const int32_t* __restrict__ gids,
                                                                  const uint2* __restrict__ cand_in = nullptr,
                                                                  const uint32_t* __restrict__ wcnt_in = nullptr) {
  extern __shared__ __attribute__((aligned(16))) unsigned char smem_raw[];
  rows_select<kRowsPer, kCandIn>(*reinterpret_cast<RowsSmem*>(smem_raw), blockIdx.x, scores, n, lens, len_div, k,
                                 pool, n_pool, blk, out, gids, cand_in, wcnt_in);
}

// Many long rows with k <= kLeanK and no pool: the selection among each
// row's filter candidates in a 512-thread workgroup with LDS for 3,072 of
// them, so that two rows run per CU.  A row it cannot take (no estimate, a
// region overflow, fewer than k or more than kLeanCand candidates) is
// flagged in its wcnt row and left to topk_rows_flagged_kernel.
constexpr int kLeanThreads = 512;
constexpr int kLeanCand = 3072;
constexpr int kLeanK = 512;

struct LeanSmem {
  uint32_t cand_key[kLeanCand];
  uint32_t cand_slot[kLeanCand];
  uint32_t hist1[kTopkBins];
  uint32_t hist2[kTopkBins];
  uint32_t hist3[256];
  uint32_t sel[kRowsMax / 32];
  uint32_t tie[kRowsMax / 32];
  uint32_t scan_sum[4][kLeanThreads / 64];
  uint32_t fin_sum[2 * kLeanThreads / 64];
  uint32_t found[2];
};
static_assert(sizeof(LeanSmem) <= 80 * 1024, "two workgroups per CU");

__global__ __launch_bounds__(kLeanThreads, 2) void topk_cand_select_kernel(int64_t n, const int32_t* __restrict__ lens,
                                                                         int32_t len_div, int32_t k,
                                                                         int32_t* __restrict__ out,
                                                                         const uint2* __restrict__ cand_in,
                                                                         uint32_t* __restrict__ wcnt) {
  extern __shared__ __attribute__((aligned(16))) unsigned char smem_raw[];
  LeanSmem& sm = *reinterpret_cast<LeanSmem*>(smem_raw);
  const int b = blockIdx.x;
  const int tid = threadIdx.x;
  const int nvalid = (int)valid_slots(n, lens, len_div, b);
  const int words = (nvalid + 31) / 32;
  const uint32_t kk = (uint32_t)k;
  uint32_t* wrow = wcnt + (int64_t)b * kTopkFilterWgMax;
  const int n_wg = (int)((n + kFilterSlots - 1) / kFilterSlots);
  const uint32_t per_wg = kTopkCandCap / n_wg;
  uint32_t cw[8], off[8], total = 0;
  bool ok = true;
#pragma unroll
  for (int w = 0; w < 8; ++w) {
    cw[w] = w < n_wg ? wrow[w] : 0u;
    ok = ok && cw[w] != kNoEstimate && cw[w] <= per_wg;
    off[w] = total;
    total += ok ? cw[w] : 0u;
  }
  if (!(ok && total >= kk && total <= (uint32_t)kLeanCand)) {  // uniform over the workgroup
    if (tid == 0) {
      const uint32_t pos = atomicAdd(&wcnt[kCountSlot], 1u);
      wcnt[(int64_t)pos * kTopkFilterWgMax + kFallbackSlot] = (uint32_t)b;
    }
    return;
  }
  for (int i = tid; i < kTopkBins; i += kLeanThreads) sm.hist1[i] = sm.hist2[i] = 0;
  if (tid < 256) sm.hist3[tid] = 0;
  for (int i = tid; i < words; i += kLeanThreads) sm.sel[i] = sm.tie[i] = 0;
  // Candidate c = tid + j * NT of the concatenated regions: all of a
  // thread's loads in flight together (clamped addresses).
  const uint2* gc = cand_in + (int64_t)b * kTopkCandCap;
  constexpr int kCandPer = kLeanCand / kLeanThreads;
  uint2 e[kCandPer];
#pragma unroll
  for (int j = 0; j < kCandPer; ++j) {
    const uint32_t c = tid + j * kLeanThreads;
    uint32_t src = 0;
#pragma unroll
    for (int w = 0; w < 8; ++w)
      if (c >= off[w] && c < off[w] + cw[w]) src = w * per_wg + (c - off[w]);
    e[j] = gc[src];
  }
  __syncthreads();  // the histograms are clear
#pragma unroll
  for (int j = 0; j < kCandPer; ++j) {
    const uint32_t c = tid + j * kLeanThreads;
    if (c < total) {
      sm.cand_key[c] = e[j].x;
      sm.cand_slot[c] = e[j].y;
      atomicAdd(&sm.hist1[e[j].x >> 20], 1u);
    }
  }
  __syncthreads();
  uint32_t T, ties;
  select_candidates<kLeanThreads>(sm.cand_key, (int)total, kk, sm.hist1, sm.hist2, sm.hist3, sm.scan_sum, sm.found,
                                  T, ties);
  for (int c = tid; c < (int)total; c += kLeanThreads) {
    const uint32_t key = sm.cand_key[c], i = sm.cand_slot[c];
    if (key > T) atomicOr(&sm.sel[i >> 5], 1u << (i & 31));
    else if (key == T) atomicOr(&sm.tie[i >> 5], 1u << (i & 31));
  }
  __syncthreads();
  finish_output_lds<kLeanThreads>(sm.sel, sm.tie, words, ties, kk, nullptr, 1, sm.fin_sum, out + (int64_t)b * k);
}

// Many rows filtered while they were scored (PrefillCandOut; k <= kLeanK,
// no pool): the selection among each row's candidates, one workgroup per
// row as in topk_cand_select_kernel, with thread t taking the count of
// block t (at most kLeanThreads blocks).  A row it cannot take (no
// estimate, a block list that overflowed, fewer than k or more than
// kLeanCand candidates) is listed for topk_rows_flagged_kernel<false> and
// flagged in co.flags, so that its whole score row is written again first.
__global__ __launch_bounds__(kLeanThreads, 2) void topk_region_select_kernel(int64_t n,
                                                                           const int32_t* __restrict__ lens,
                                                                           int32_t k, int32_t* __restrict__ out,
                                                                           PrefillCandOut co,
                                                                           uint32_t* __restrict__ wcnt) {
  extern __shared__ __attribute__((aligned(16))) unsigned char smem_raw[];
  LeanSmem& sm = *reinterpret_cast<LeanSmem*>(smem_raw);
  const int b = blockIdx.x;
  const int tid = threadIdx.x;
  const int nvalid = (int)valid_slots(n, lens, 1, b);
  const int words = (nvalid + 31) / 32;
  const uint32_t kk = (uint32_t)k;
  const int nb = co.n_blocks;
  // Four threads per block list: thread (blk, sub) takes entries sub,
  // sub + 4, ... of list blk.  Its first kPer entries are loaded at once,
  // before the count is known (every list has kCandCap places, so the
  // loads stay in bounds; entries past the count are ignored), so that
  // they travel with the count load instead of after the scan.
  constexpr int kTpb = kLeanThreads / (kRowsMax / kCandBlock);
  constexpr int kPer = 8;
  static_assert(kTpb * (kRowsMax / kCandBlock) == kLeanThreads && kTpb * kPer <= kCandCap, "list split");
  const int blk = tid / kTpb, sub = tid % kTpb;
  const uint2* lb = co.cand + ((int64_t)b * nb + min(blk, nb - 1)) * kCandCap;
  uint2 e[kPer];
#pragma unroll
  for (int j = 0; j < kPer; ++j) e[j] = lb[sub + kTpb * j];
  const uint32_t lo = wcnt[(int64_t)b * kTopkFilterWgMax + kThresholdSlot];
  const uint32_t cnt = blk < nb ? co.cnt[(int64_t)b * nb + blk] : 0u;
  uint32_t total;
  const uint32_t off = block_exclusive_scan<kLeanThreads>(sub == 0 ? cnt : 0u, sm.scan_sum[0], &total);
  const uint32_t boff = (uint32_t)__shfl((int)off, lane_id() & ~(kTpb - 1));  // the list's first place
  const bool over = __syncthreads_or(cnt > (uint32_t)kCandCap);
  if (over || lo == kNoEstimate || total < kk || total > (uint32_t)kLeanCand) {  // uniform over the workgroup
    if (tid == 0) {
      const uint32_t pos = atomicAdd(&wcnt[kCountSlot], 1u);
      wcnt[(int64_t)pos * kTopkFilterWgMax + kFallbackSlot] = (uint32_t)b;
      atomicOr(&co.flags[b >> 5], 1u << (b & 31));
    }
    return;
  }
  {
    const u32x4 z = {0u, 0u, 0u, 0u};
    for (int i = tid; i < kTopkBins / 4; i += kLeanThreads)
      reinterpret_cast<u32x4*>(sm.hist1)[i] = reinterpret_cast<u32x4*>(sm.hist2)[i] = z;
    if (tid < 64) reinterpret_cast<u32x4*>(sm.hist3)[tid] = z;
    for (int i = tid; i < (words + 3) / 4; i += kLeanThreads)
      reinterpret_cast<u32x4*>(sm.sel)[i] = reinterpret_cast<u32x4*>(sm.tie)[i] = z;
  }
  __syncthreads();
  auto put = [&](uint32_t c, uint2 v) {
    const uint32_t bits = v.x;
    const uint32_t key = order_key(__builtin_bit_cast(float, bits));
    sm.cand_key[boff + c] = key;
    sm.cand_slot[boff + c] = v.y;
    atomicAdd(&sm.hist1[key >> 20], 1u);
  };
#pragma unroll
  for (int j = 0; j < kPer; ++j)
    if (sub + kTpb * j < (int)cnt) put(sub + kTpb * j, e[j]);
  for (uint32_t c = sub + kTpb * kPer; c < cnt; c += kTpb) put(c, lb[c]);  // lists longer than kTpb * kPer
  __syncthreads();
  uint32_t T, ties;
  select_candidates<kLeanThreads>(sm.cand_key, (int)total, kk, sm.hist1, sm.hist2, sm.hist3, sm.scan_sum, sm.found,
                                  T, ties);
  for (int c = tid; c < (int)total; c += kLeanThreads) {
    const uint32_t key = sm.cand_key[c], i = sm.cand_slot[c];
    if (key > T) atomicOr(&sm.sel[i >> 5], 1u << (i & 31));
    else if (key == T) atomicOr(&sm.tie[i >> 5], 1u << (i & 31));
  }
  __syncthreads();
  finish_output_lds<kLeanThreads>(sm.sel, sm.tie, words, ties, kk, nullptr, 1, sm.fin_sum, out + (int64_t)b * k);
}

// The rows topk_cand_select_kernel or topk_region_select_kernel left: a
// grid of one workgroup per CU claims the listed rows one by one until the
// list is exhausted.  kCandIn: first the selection among up to 8,192 of the
// row's filter candidates, else (and without kCandIn) the full passes over
// the row's scores.
template <bool kCandIn>
__global__ __launch_bounds__(kFinalThreads) void topk_rows_flagged_kernel(const float* __restrict__ scores, int64_t n,
                                                                          const int32_t* __restrict__ lens,
                                                                          int32_t len_div, int32_t k,
                                                                          int32_t* __restrict__ out,
                                                                          const uint2* __restrict__ cand_in,
                                                                          uint32_t* __restrict__ wcnt) {
  extern __shared__ __attribute__((aligned(16))) unsigned char smem_raw[];
  RowsSmem& sm = *reinterpret_cast<RowsSmem*>(smem_raw);
  __shared__ uint32_t claimed;
  const uint32_t count = wcnt[kCountSlot];
  for (;;) {
    if (threadIdx.x == 0) claimed = atomicAdd(&wcnt[kClaimSlot], 1u);
    __syncthreads();
    const uint32_t i = claimed;
    __syncthreads();
    if (i >= count) break;  // uniform
    const int b = (int)wcnt[(int64_t)i * kTopkFilterWgMax + kFallbackSlot];
    rows_select<64, kCandIn>(sm, b, scores, n, lens, len_div, k, nullptr, 0, 1, out, nullptr, cand_in, wcnt);
    __syncthreads();  // LDS is reused by the next row
  }
}
}  // namespace

// Bitmap words per sequence: a multiple of 4, so that every sequence's
// bitmap is 16-byte aligned.
// ------------------------------------------------------ pool selection
// The Top-k of a hierarchical layer's pool slots (at most 16,384 per
// sequence), after the pool scoring kernel has left the j-th largest key
// of every 128-slot tile (tile_bound [n_seq][tiles]; see index_score.hip),
// whose least, B, is a lower bound of the sequence's k-th largest key.
// One 1,024-thread workgroup per sequence; thread t holds slots 16t ..
// 16t + 15.  The keys >= B -- at least k of them when B is a bound, and
// usually few more -- go to an LDS list in slot order (one scan), the exact
// k-th key and its ties are selected among them (radix select over digits
// of 12, 12 and 8 bits), and the list's selected entries are written in
// slot order, which is id order.  When B leaves fewer than k or more than
// kPoolCap keys, the same radix select runs over all the keys.
#ifndef CSA2_POOL_SELECT_THREADS
#define CSA2_POOL_SELECT_THREADS 1024
#endif
constexpr int kPoolSelThreads = CSA2_POOL_SELECT_THREADS;
constexpr int kPoolSelWaves = kPoolSelThreads / 64;
constexpr int kPoolSelMax = 16384;
constexpr int kPoolSelPer = kPoolSelMax / kPoolSelThreads;  // slots per thread
constexpr int kPoolCap = 4096;                               // keys selected from the LDS list

struct PoolSmem {
  int32_t pool[CSA2_TOPK_MAX];
  uint32_t hist1[kTopkBins];
  uint32_t hist2[kTopkBins];
  uint32_t hist3[kTopkBins];
  uint32_t key[kPoolCap];
  uint32_t slot[kPoolCap];
  uint32_t scan_sum[4][kPoolSelWaves];  // the list selection's scans (slots 1..3)
  uint32_t full_sum[3][kPoolSelWaves];  // the scans over all keys
  uint32_t cnt_sum[2 * kPoolSelWaves];
  uint32_t out_sum[2 * kPoolSelWaves];
  uint32_t bmin[kPoolSelWaves];
  uint32_t bmax[kPoolSelWaves];
  uint32_t found[2];
};

__global__ __launch_bounds__(kPoolSelThreads) void pool_select_kernel(const float* __restrict__ scores, int32_t n,
                                                                   int32_t k, const int32_t* __restrict__ pool,
                                                                   int32_t n_pool, int32_t blk,
                                                                   const uint32_t* __restrict__ tile_bound,
                                                                   int32_t* __restrict__ out) {
  constexpr int NT = kPoolSelThreads;
  extern __shared__ __attribute__((aligned(16))) unsigned char smem_raw[];
  PoolSmem& sm = *reinterpret_cast<PoolSmem*>(smem_raw);
  const int b = blockIdx.x, tid = threadIdx.x;
  const uint32_t kk = (uint32_t)k;
  const int n_tiles = (n + 127) / 128;
  const uint32_t tb = tid < n_tiles ? tile_bound[(int64_t)b * n_tiles + tid] : 0xFFFFFFFFu;
  const float* sc = scores + (int64_t)b * n;
  const int s0 = kPoolSelPer * tid;
  uint32_t key[kPoolSelPer];
  if ((n & 3) == 0 && s0 + kPoolSelPer <= n) {
    const f32x4* p4 = reinterpret_cast<const f32x4*>(sc + s0);
    f32x4 v[kPoolSelPer / 4];
#pragma unroll
    for (int i = 0; i < kPoolSelPer / 4; ++i) v[i] = p4[i];
#pragma unroll
    for (int i = 0; i < kPoolSelPer / 4; ++i)
#pragma unroll
      for (int e = 0; e < 4; ++e) key[4 * i + e] = order_key(v[i][e]);
  } else {
#pragma unroll
    for (int j = 0; j < kPoolSelPer; ++j) key[j] = s0 + j < n ? order_key(sc[s0 + j]) : 0u;
  }
  if (pool)
    for (int i = tid; i < n_pool; i += NT) sm.pool[i] = pool[(int64_t)b * n_pool + i];
  for (int i = tid; i < kTopkBins; i += NT) sm.hist1[i] = sm.hist2[i] = sm.hist3[i] = 0u;
  {
    uint32_t lm = 0u;
#pragma unroll
    for (int j = 0; j < kPoolSelPer; ++j) lm = max(lm, key[j]);
    const uint32_t wm = wave_min_u32(tb), wx = wave_max_u32(lm);
    if ((tid & 63) == 0) sm.bmin[tid >> 6] = wm, sm.bmax[tid >> 6] = wx;
  }
  __syncthreads();
  uint32_t B = 0xFFFFFFFFu, kmax = 0u;
#pragma unroll
  for (int i = 0; i < kPoolSelWaves; ++i) B = min(B, sm.bmin[i]), kmax = max(kmax, sm.bmax[i]);
  uint2 cnt = make_uint2(0u, 0u);  // (keys >= B, keys)
#pragma unroll
  for (int j = 0; j < kPoolSelPer; ++j) {
    cnt.x += (key[j] != 0u && key[j] >= B) ? 1u : 0u;
    cnt.y += key[j] != 0u ? 1u : 0u;
  }
  uint2 tot;
  const uint2 before = block_exclusive_scan2_once<NT>(cnt, sm.cnt_sum, &tot);
  // Selection: keys > T, and the lowest `ties` slots with key == T (T = 0:
  // every key is taken).
  uint32_t T = 0u, ties = 0u;
  const bool list = tot.y > kk && tot.x >= kk && tot.x <= (uint32_t)kPoolCap;  // uniform
  if (list) {
    uint32_t pos = before.x;
#pragma unroll
    for (int j = 0; j < kPoolSelPer; ++j) {
      if (key[j] != 0u && key[j] >= B) {
        sm.key[pos] = key[j];
        sm.slot[pos] = (uint32_t)(s0 + j);
        ++pos;
      }
    }
    __syncthreads();
    // The exact kk-th largest among the list by a radix select whose digits
    // are taken over the list's own key range [B, max]: 12 bits at a time
    // from the top of the span, so that keys crowded in a narrow range (the
    // usual case) spread over the bins.
    // Each pass counts the keys in [base, base + width) by bits shift.. of
    // key - base (at most 4,096 bins), and narrows the range to the bin
    // that holds the need-th largest.
    uint32_t base = B, need = kk;
    uint64_t width = (uint64_t)(kmax - B) + 1;
    int shift = max(0, 32 - __clz(kmax - B) - 12);
    uint32_t* hist[3] = {sm.hist1, sm.hist2, sm.hist3};
    for (int pass = 0; pass < 3; ++pass) {
      for (int c = tid; c < (int)tot.x; c += NT) {
        const uint32_t kv = sm.key[c];
        if (kv >= base && (uint64_t)(kv - base) < width) atomicAdd(&hist[pass][(kv - base) >> shift], 1u);
      }
      __syncthreads();
      find_threshold_bin_once<NT>(hist[pass], kTopkBins, need, sm.scan_sum[pass + 1], sm.found);
      base += sm.found[0] << shift;
      need -= sm.found[1];
      if (shift == 0) break;
      width = (uint64_t)1 << shift;
      shift = max(0, shift - 12);
    }
    T = base;
    ties = need;
  } else if (tot.y > kk) {
#pragma unroll
    for (int j = 0; j < kPoolSelPer; ++j) wave_hist_add_grouped(sm.hist1, key[j] >> 20, key[j] != 0u);
    __syncthreads();
    find_threshold_bin_once<NT>(sm.hist1, kTopkBins, kk, sm.full_sum[0], sm.found);
    const uint32_t b1 = sm.found[0], need1 = kk - sm.found[1];
#pragma unroll
    for (int j = 0; j < kPoolSelPer; ++j)
      wave_hist_add_grouped(sm.hist2, (key[j] >> 8) & 0xFFFu, key[j] != 0u && (key[j] >> 20) == b1);
    __syncthreads();
    find_threshold_bin_once<NT>(sm.hist2, kTopkBins, need1, sm.full_sum[1], sm.found);
    const uint32_t pre2 = (b1 << 12) | sm.found[0], need2 = need1 - sm.found[1];
#pragma unroll
    for (int j = 0; j < kPoolSelPer; ++j)
      wave_hist_add_grouped(sm.hist3, key[j] & 0xFFu, key[j] && (key[j] >> 8) == pre2);
    __syncthreads();
    find_threshold_bin_once<NT>(sm.hist3, 256, need2, sm.full_sum[2], sm.found);
    T = (pre2 << 8) | sm.found[0];
    ties = need2 - sm.found[1];
  }
  // Output in slot order: the list entries [e0, e1) of this thread, or its
  // own 16 slots.  A taken key's position = keys above T before it + ties
  // taken before it.
  const int32_t* pl = pool ? sm.pool : nullptr;
  int32_t* ob = out + (int64_t)b * k;
  const int per = list ? ((int)tot.x + NT - 1) / NT : kPoolSelPer;
  const int e0 = list ? min((int)tot.x, tid * per) : 0, e1 = list ? min((int)tot.x, e0 + per) : kPoolSelPer;
  auto item = [&](int e, uint32_t& kv, uint32_t& slot) {
    if (list) {
      kv = sm.key[e];
      slot = sm.slot[e];
    } else {
      kv = 0u;
#pragma unroll
      for (int j = 0; j < kPoolSelPer; ++j)
        if (j == e) kv = key[j];
      slot = (uint32_t)(s0 + e);
    }
  };
  uint2 c2 = make_uint2(0u, 0u);  // (keys > T, keys == T)
  for (int e = e0; e < e1; ++e) {
    uint32_t kv, slot;
    item(e, kv, slot);
    c2.x += kv > T ? 1u : 0u;
    c2.y += (T != 0u && kv == T) ? 1u : 0u;
  }
  uint2 t2;
  const uint2 b2 = block_exclusive_scan2_once<NT>(c2, sm.out_sum, &t2);
  uint32_t pgt = b2.x, peq = b2.y;
  for (int e = e0; e < e1; ++e) {
    uint32_t kv, slot;
    item(e, kv, slot);
    int32_t pos = -1;
    if (kv > T) {
      pos = (int32_t)(pgt + min(peq, ties));
      ++pgt;
    } else if (T != 0u && kv == T) {
      if (peq < ties) pos = (int32_t)(pgt + peq);
      ++peq;
    }
    if (pos >= 0 && pos < k) ob[pos] = pl ? pl[slot / blk] * blk + (int32_t)(slot % blk) : (int32_t)slot;
  }
  const uint32_t n_sel = t2.x + min(t2.y, ties);
  for (uint32_t i = n_sel + tid; i < kk; i += NT) ob[i] = -1;
}

static int64_t bitmap_words(int64_t n) { return ((n + 31) / 32 + 3) / 4 * 4; }

size_t topk_workspace_bytes(int64_t n, int32_t n_seq) {
  const int64_t words = bitmap_words(n);
  const int64_t tie_words = (n + 31) / 32 > kTopkLdsWords ? words : 0;
  return (size_t)n_seq * (kCandBytes + kTopkBins * sizeof(uint32_t) + (words + tie_words) * sizeof(uint32_t) +
                          kTopkFilterWgMax * sizeof(uint32_t) + kPoolTiles * sizeof(uint32_t)) + 64;
}

// Layout: cand, hist, bits, tie (long inputs), wcnt; ws is 16-byte aligned.
TopkWs topk_ws_carve(void* ws, int64_t n, int32_t n_seq) {
  TopkWs w;
  char* p = reinterpret_cast<char*>(ws);
  w.cand = reinterpret_cast<uint2*>(p);
  p += (size_t)n_seq * kCandBytes;
  w.hist = reinterpret_cast<uint32_t*>(p);
  p += (size_t)n_seq * kTopkBins * sizeof(uint32_t);
  w.words_cap = bitmap_words(n);
  w.bits = reinterpret_cast<uint32_t*>(p);
  p += (size_t)n_seq * w.words_cap * sizeof(uint32_t);
  w.tie = reinterpret_cast<uint32_t*>(p);  // used (and sized) only past kTopkLdsWords words
  if ((n + 31) / 32 > kTopkLdsWords) p += (size_t)n_seq * w.words_cap * sizeof(uint32_t);
  w.wcnt = reinterpret_cast<uint32_t*>(p);
  p += (size_t)n_seq * kTopkFilterWgMax * sizeof(uint32_t);
  w.bound = reinterpret_cast<uint32_t*>(p);
  return w;
}

csa2_status topk_launch(const float* scores, int64_t n, const int32_t* lens, int32_t len_div, int32_t k,
                        const int32_t* pool, int32_t n_pool, int32_t blk, int32_t* out, const TopkWs& ws,
                        bool hist_ready, int32_t n_seq, hipStream_t stream, const int32_t* gids) {
  if (n_seq == 0) return CSA2_OK;
  CSA2_REQUIRE(!gids || (!hist_ready && !pool && n <= kRowsMax), CSA2_EINVAL,
               "csa2_topk: emitted ids need the single-workgroup selection");
  static bool attr_set = false;
  if (!attr_set) {
    if (hipFuncSetAttribute(reinterpret_cast<const void*>(topk_final_kernel<false>),
                            hipFuncAttributeMaxDynamicSharedMemorySize,
                            (int)sizeof(FinalSmem)) != hipSuccess ||
        hipFuncSetAttribute(reinterpret_cast<const void*>(topk_final_kernel<true>),
                            hipFuncAttributeMaxDynamicSharedMemorySize,
                            (int)sizeof(FinalSmem)) != hipSuccess ||
        hipFuncSetAttribute(reinterpret_cast<const void*>(topk_rows_kernel<16>),
                            hipFuncAttributeMaxDynamicSharedMemorySize, (int)sizeof(RowsSmem)) != hipSuccess ||
        hipFuncSetAttribute(reinterpret_cast<const void*>(topk_rows_kernel<32>),
                            hipFuncAttributeMaxDynamicSharedMemorySize, (int)sizeof(RowsSmem)) != hipSuccess ||
        hipFuncSetAttribute(reinterpret_cast<const void*>(topk_rows_kernel<64>),
                            hipFuncAttributeMaxDynamicSharedMemorySize, (int)sizeof(RowsSmem)) != hipSuccess ||
        hipFuncSetAttribute(reinterpret_cast<const void*>(topk_rows_kernel<64, true>),
                            hipFuncAttributeMaxDynamicSharedMemorySize, (int)sizeof(RowsSmem)) != hipSuccess ||
        hipFuncSetAttribute(reinterpret_cast<const void*>(topk_rows_flagged_kernel<true>),
                            hipFuncAttributeMaxDynamicSharedMemorySize, (int)sizeof(RowsSmem)) != hipSuccess ||
        hipFuncSetAttribute(reinterpret_cast<const void*>(topk_cand_select_kernel),
                            hipFuncAttributeMaxDynamicSharedMemorySize, (int)sizeof(LeanSmem)) != hipSuccess ||
        hipFuncSetAttribute(reinterpret_cast<const void*>(pool_select_kernel),
                            hipFuncAttributeMaxDynamicSharedMemorySize, (int)sizeof(PoolSmem)) != hipSuccess)
      return launch_status("csa2_topk (shared memory attribute)");
    attr_set = true;
  }
  if (!hist_ready && n > 32 * kFinalThreads && n <= kRowsMax && n_seq >= kManyRows) {
    // Many long rows: the threshold estimate and the candidates on many
    // workgroups per row, then the selection per row.
    hipLaunchKernelGGL(topk_sample_kernel, dim3(n_seq), dim3(kPassThreads), 0, stream, scores, n, lens, len_div,
                       k, ws);
    const dim3 grid((uint32_t)((n + kFilterSlots - 1) / kFilterSlots), n_seq);
    if (n % 4 == 0 && (reinterpret_cast<uintptr_t>(scores) & 15) == 0)
      hipLaunchKernelGGL(topk_sample_filter_kernel<true>, grid, dim3(kPassThreads), 0, stream, scores, n, lens,
                         len_div, ws);
    else
      hipLaunchKernelGGL(topk_sample_filter_kernel<false>, grid, dim3(kPassThreads), 0, stream, scores, n, lens,
                         len_div, ws);
    if (k <= kLeanK && !pool && !gids) {
      hipLaunchKernelGGL(topk_cand_select_kernel, dim3(n_seq), dim3(kLeanThreads), sizeof(LeanSmem), stream, n, lens,
                         len_div, k, out, ws.cand, ws.wcnt);
      hipLaunchKernelGGL(topk_rows_flagged_kernel<true>, dim3(std::min(n_seq, kFlaggedGrid)), dim3(kFinalThreads),
                         sizeof(RowsSmem), stream, scores, n, lens, len_div, k, out, ws.cand, ws.wcnt);
    } else {
      hipLaunchKernelGGL((topk_rows_kernel<64, true>), dim3(n_seq), dim3(kFinalThreads), sizeof(RowsSmem), stream,
                         scores, n, lens, len_div, k, pool, n_pool, blk, out, gids, ws.cand, ws.wcnt);
    }
    return launch_status("csa2_topk");
  }
  if (!hist_ready && n <= kRowsMax) {
    if (n <= 16 * kFinalThreads)
      hipLaunchKernelGGL(topk_rows_kernel<16>, dim3(n_seq), dim3(kFinalThreads), sizeof(RowsSmem), stream, scores,
                         n, lens, len_div, k, pool, n_pool, blk, out, gids);
    else if (n <= 32 * kFinalThreads)
      hipLaunchKernelGGL(topk_rows_kernel<32>, dim3(n_seq), dim3(kFinalThreads), sizeof(RowsSmem), stream, scores,
                         n, lens, len_div, k, pool, n_pool, blk, out, gids);
    else
      hipLaunchKernelGGL(topk_rows_kernel<64>, dim3(n_seq), dim3(kFinalThreads), sizeof(RowsSmem), stream, scores,
                         n, lens, len_div, k, pool, n_pool, blk, out, gids);
    return launch_status("csa2_topk");
  }
  if (!hist_ready && n > 0)
    hipLaunchKernelGGL(topk_hist_kernel, dim3((uint32_t)((n + kHistSlots - 1) / kHistSlots), n_seq),
                       dim3(kPassThreads), 0, stream, scores, n, lens, len_div, ws.hist);
  if (n > kDirectMax)
    hipLaunchKernelGGL(topk_filter_kernel, dim3((uint32_t)((n + kFilterSlots - 1) / kFilterSlots), n_seq),
                       dim3(kPassThreads), 0, stream, scores, n, lens, len_div, k, ws);
  if ((n + 31) / 32 > kTopkLdsWords)
    hipLaunchKernelGGL(topk_final_kernel<true>, dim3(n_seq), dim3(kFinalThreads), sizeof(FinalSmem), stream,
                       scores, n, lens, len_div, k, pool, n_pool, blk, ws, out);
  else
    hipLaunchKernelGGL(topk_final_kernel<false>, dim3(n_seq), dim3(kFinalThreads), sizeof(FinalSmem), stream,
                       scores, n, lens, len_div, k, pool, n_pool, blk, ws, out);
  return launch_status("csa2_topk");
}

// The pool Top-k after bounded pool scoring (pool_select_kernel): n <=
// kPoolSelMax slots per sequence, k <= CSA2_TOPK_MAX; ws.bound holds the
// scoring kernel's tile bounds.
csa2_status pool_select_launch(const float* scores, int64_t n, int32_t k, const int32_t* pool, int32_t n_pool,
                               int32_t blk, const TopkWs& ws, int32_t* out, int32_t n_seq, hipStream_t stream) {
  if (n_seq == 0) return CSA2_OK;
  CSA2_REQUIRE(n >= 1 && n <= kPoolSelMax && k >= 1 && k <= CSA2_TOPK_MAX && n_pool <= CSA2_TOPK_MAX &&
                   (reinterpret_cast<uintptr_t>(scores) & 15) == 0,
               CSA2_ESHAPE, "pool selection: bad shape");
  static bool attr_set = false;
  if (!attr_set) {
    if (hipFuncSetAttribute(reinterpret_cast<const void*>(pool_select_kernel),
                            hipFuncAttributeMaxDynamicSharedMemorySize, (int)sizeof(PoolSmem)) != hipSuccess)
      return launch_status("pool selection (shared memory attribute)");
    attr_set = true;
  }
  hipLaunchKernelGGL(pool_select_kernel, dim3(n_seq), dim3(kPoolSelThreads), sizeof(PoolSmem), stream, scores,
                     (int32_t)n, k, pool, n_pool, blk, static_cast<const uint32_t*>(ws.bound), out);
  return launch_status("pool selection");
}

// Whether a prefill chunk's rows (n slots each, n_rows of them, Top-k) are
// selected from candidates filtered while they are scored: the shapes that
// the many-row selection takes, with k <= kLeanK.
bool prefill_filter_applies(int64_t n, int32_t n_rows, int32_t k) {
  return n > 32 * kFinalThreads && n <= kRowsMax && n_rows >= kManyRows && k <= kLeanK;
}

// The selection of many rows filtered while they are scored
// (prefill_filter_applies; lens = the rows' visible counts): stage 0 takes
// each row's threshold estimate from its sampled scores, stage 1 selects
// among each row's candidates (co) and lists and flags the rows it cannot
// take, stage 2 runs the full selection of the listed rows over their
// rescored rows.
csa2_status prefill_select_launch(int stage, const float* scores, int64_t n, const int32_t* lens, int32_t k,
                                  int32_t* out, const TopkWs& ws, const PrefillCandOut& co, int32_t n_rows,
                                  hipStream_t stream) {
  if (n_rows == 0) return CSA2_OK;
  CSA2_REQUIRE(prefill_filter_applies(n, n_rows, k) && co.n_blocks == (n + kCandBlock - 1) / kCandBlock &&
                   co.n_blocks <= kLeanThreads,
               CSA2_ESHAPE, "prefill selection: bad shape");
  static bool attr_set = false;
  if (!attr_set) {
    if (hipFuncSetAttribute(reinterpret_cast<const void*>(topk_region_select_kernel),
                            hipFuncAttributeMaxDynamicSharedMemorySize, (int)sizeof(LeanSmem)) != hipSuccess ||
        hipFuncSetAttribute(reinterpret_cast<const void*>(topk_rows_flagged_kernel<false>),
                            hipFuncAttributeMaxDynamicSharedMemorySize, (int)sizeof(RowsSmem)) != hipSuccess)
      return launch_status("prefill selection (shared memory attribute)");
    attr_set = true;
  }
  if (stage == 0)
    hipLaunchKernelGGL(topk_sample_kernel, dim3(n_rows), dim3(kPassThreads), 0, stream, scores, n, lens, 1, k, ws);
  else if (stage == 1)
    hipLaunchKernelGGL(topk_region_select_kernel, dim3(n_rows), dim3(kLeanThreads), sizeof(LeanSmem), stream, n,
                       lens, k, out, co, ws.wcnt);
  else
    hipLaunchKernelGGL(topk_rows_flagged_kernel<false>, dim3(std::min(n_rows, kFlaggedGrid)), dim3(kFinalThreads),
                       sizeof(RowsSmem), stream, scores, n, lens, 1, k, out, nullptr, ws.wcnt);
  return launch_status("prefill selection");
}

}  // namespace csa2
