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
#include "select_dev.hpp"

namespace csa2 {
namespace {

constexpr int kTilesPerWave = 8;                       // 16 keys per tile
constexpr int kKeysPerWG = 4 * kTilesPerWave * 16;     // 512 keys, 4 wavefronts

// Weighted ReLU sum of four heads, ((w0 r0 + w1 r1) + w2 r2) + w3 r3, every
// product and sum rounded on its own (no fused multiply-add).  ReLU is the
// median of (x, 0, +inf): one v_med3_f32, equal to fmaxf(x, 0) for every
// value an MFMA produces (a quiet NaN gives 0), where fmaxf costs a
// canonicalising max in front of its own.  The +inf bound is hidden from
// constant folding, which would turn the median back into fmaxf.
__device__ __forceinline__ float relu_wsum4(const f32x4& acc, const float* wh) {
#pragma clang fp contract(off)
  float inf = __builtin_inff();
  asm("" : "+s"(inf));
  float part = wh[0] * __builtin_amdgcn_fmed3f(acc[0], 0.f, inf);
#pragma unroll
  for (int r = 1; r < 4; ++r) part = part + wh[r] * __builtin_amdgcn_fmed3f(acc[r], 0.f, inf);
  return part;
}

// The j-th largest (with multiplicity) of the 64 x 8 order keys k[] of a
// wavefront (0 if fewer than j are nonzero): j - 1 times the largest is
// removed (one copy, from the lowest lane holding it), then the largest
// left is taken.
__device__ __forceinline__ uint32_t wave_jth_largest(uint32_t (&k)[8], int j) {
  const int lane = threadIdx.x & 63;
  for (int p = 1; p < j; ++p) {
    uint32_t lm = k[0];
#pragma unroll
    for (int t = 1; t < 8; ++t) lm = max(lm, k[t]);
    const uint32_t wm = wave_max_u32(lm);
    if (wm == 0) return 0;
    const uint64_t who = __ballot(lm == wm);
    if (lane == __ffsll((unsigned long long)who) - 1) {
      bool done = false;
#pragma unroll
      for (int t = 0; t < 8; ++t)
        if (!done && k[t] == wm) {
          k[t] = 0;
          done = true;
        }
    }
  }
  uint32_t lm = k[0];
#pragma unroll
  for (int t = 1; t < 8; ++t) lm = max(lm, k[t]);
  return wave_max_u32(lm);
}

// kHist: also add the scores' top key digits into a per-sequence histogram
// (ghist [n_seq][4096]) for the Top-k that follows.
// tile_bound (pool mode, may be null): for the selection that follows, the
// j-th largest order key of every tile of 128 slots, j = ceil(k / tiles),
// in tile_bound[b][tile] (0 when the tile has fewer than j keys or j >
// kBoundJMax).  The least of a sequence's tile values, B, is a lower bound
// of its k-th largest key: every tile has j keys >= B, so at least k keys
// are >= B.
constexpr int kBoundJMax = 16;

template <bool kPool, bool kWeights, bool kHist>
__global__ __launch_bounds__(256) void index_score_kernel(
    const uint16_t* __restrict__ q, const float* __restrict__ w, const uint16_t* __restrict__ keys,
    int64_t key_cap, const int32_t* __restrict__ lens, int32_t len_div,
    const int32_t* __restrict__ pool, int32_t n_pool, int32_t blk, float* __restrict__ scores,
    int64_t n_out, uint32_t* __restrict__ ghist, uint32_t* __restrict__ tile_bound, int32_t bound_j) {
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
  const bool bound = kPool && tile_bound != nullptr;
  const int64_t n_tiles = (n_out + 127) / 128;
  // Grid-stride over chunks of kKeysPerWG keys (one histogram flush per workgroup).
  for (int64_t chunk = blockIdx.x; chunk * kKeysPerWG < n_out; chunk += gridDim.x) {
    const int64_t base = chunk * kKeysPerWG + (int64_t)wave * (kTilesPerWave * 16);
    u32x4 kv[kTilesPerWave][2];
    bool valid[kTilesPerWave];
    // Pool mode: every tile's block id first (clamped slots, all loads in
    // flight together; slot < n_out = n_pool * blk <= 2^20 fits 32 bits),
    // then the key rows they name.
    int32_t blk_id[kTilesPerWave];
    if (kPool) {
#pragma unroll
      for (int t = 0; t < kTilesPerWave; ++t) {
        const uint32_t s32 = (uint32_t)min(base + t * 16 + n, n_out - 1);
        blk_id[t] = pool[(int64_t)b * n_pool + s32 / (uint32_t)blk];
      }
    }
#pragma unroll
    for (int t = 0; t < kTilesPerWave; ++t) {
      const int64_t slot = base + t * 16 + n;
      int64_t row = slot;
      bool ok = slot < n_valid;
      if (kPool) {
        row = (int64_t)blk_id[t] * blk + (int64_t)((uint32_t)slot % (uint32_t)blk);
        ok = ok && blk_id[t] >= 0 && row < L && row < key_cap;
      }
      valid[t] = ok;
      // Unconditional load of a clamped row (an invalid slot reads row 0 and
      // is masked below), so the wavefront's loads are all in flight together.
      const u32x4* kp = reinterpret_cast<const u32x4*>(kb + (ok ? row : 0) * 64 + 16 * g);
      kv[t][0] = __builtin_nontemporal_load(kp);
      kv[t][1] = __builtin_nontemporal_load(kp + 1);
    }
    uint32_t okeys[kTilesPerWave];
#pragma unroll
    for (int t = 0; t < kTilesPerWave; ++t) {
      if (!valid[t]) kv[t][0] = kv[t][1] = u32x4{0, 0, 0, 0};
      f32x4 acc = {0.f, 0.f, 0.f, 0.f};
      acc = mfma16x16x32(qa[0], as_bf16x8(kv[t][0]), acc);
      acc = mfma16x16x32(qa[1], as_bf16x8(kv[t][1]), acc);
      // acc[r] = q_{4g+r} . key n.
      const float part = relu_wsum4(acc, wh);
      const float score = fold16_add(part);  // heads 0..3 + heads 4..7
      const int64_t slot = base + t * 16 + n;
      okeys[t] = 0u;
      if (g == 0 && slot < n_out) {
        sb[slot] = valid[t] ? score : kNegInf;
        const uint32_t key = order_key(score);
        if (kHist && valid[t] && key) atomicAdd(&hist[key >> 20], 1u);
        okeys[t] = valid[t] ? key : 0u;
      }
    }
    if (bound) {
      const uint32_t tb = bound_j <= kBoundJMax ? wave_jth_largest(okeys, bound_j) : 0u;
      const int64_t tile = base / 128;  // this wavefront's 128 slots
      if ((threadIdx.x & 63) == 0 && tile < n_tiles) tile_bound[(int64_t)b * n_tiles + tile] = tb;
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
                int32_t n_pool, int32_t blk, float* scores, int64_t n_out, uint32_t* ghist, uint32_t* bound_inv,
                int32_t bound_j) {
  if (ghist)
    hipLaunchKernelGGL((index_score_kernel<kPool, kWeights, true>), grid, dim3(256), 0, stream, q, w, keys,
                       key_cap, lens, len_div, pool, n_pool, blk, scores, n_out, ghist, bound_inv, bound_j);
  else
    hipLaunchKernelGGL((index_score_kernel<kPool, kWeights, false>), grid, dim3(256), 0, stream, q, w, keys,
                       key_cap, lens, len_div, pool, n_pool, blk, scores, n_out, ghist, bound_inv, bound_j);
}

// ------------------------------------------------------------------ prefill
// Indexer scores of a causal prefill chunk: n_q queries (query i at token
// t0 + i) against the keys of compressed entries, entry e visible to query i
// iff e < vis_i = min(n_entries, (t0 + i + 1) / ratio).  This is a dense
// contraction of (query, head) rows with entry keys, so both MFMA operands
// carry real data: a 256-thread workgroup takes 32 queries against 512
// entries (128 per wavefront = 8 column tiles of 16).  Each wavefront holds
// its entries' key fragments in registers and walks 8 groups of 4 queries,
// whose query fragments come from LDS.  A group takes two row tiles per
// column tile, rows 4i + h = (query i of the group, head h) and (query i,
// head 4 + h), so that output lane (n, g) of the two products holds all 8
// heads of query g and entry n: the ReLU sum over heads is local to the
// lane, and the 64 lanes hold 64 different scores.  What happens to a score
// depends on the mode:
//   kPfAll      every score goes out (-inf past the query's visible entries);
//   kPfSampled  the block is the 1,024 entries a row's threshold estimate
//               reads (64 runs of 16, one at the start of each 64th of the
//               entries; grid.x = 2; a column tile is one run) and only
//               their scores go out;
//   kPfCand     only the scores at or above the query's threshold (and
//               inside its visible entries) go out, as (score bits, entry)
//               pairs into the query's list for the workgroup's 512
//               entries, each at a position taken from the query's LDS
//               counter, and the count -- so the score matrix never reaches
//               memory;
//   kPfRescore  kPfAll for query blocks holding a row that the selection
//               over the candidates could not take, up to the last visible
//               entry of the block.
constexpr int kPfQ = 32;          // queries per workgroup
constexpr int kPfE = 512;         // entries per workgroup
constexpr int kPfCols = kPfE / (4 * 16);  // column tiles per wavefront (8)
constexpr int kPfAll = 0, kPfSampled = 1, kPfCand = 2, kPfRescore = 3;
static_assert(kPfE == kCandBlock, "one candidate list per query and workgroup");

// Weighted ReLU sum of the 8 heads, head 0 first, each product and sum
// rounded on its own; ReLU as in relu_wsum4.
__device__ __forceinline__ float relu_wsum8(const f32x4& lo, const f32x4& hi, const float* wh) {
#pragma clang fp contract(off)
  float inf = __builtin_inff();
  asm("" : "+s"(inf));
  float sum = wh[0] * __builtin_amdgcn_fmed3f(lo[0], 0.f, inf);
#pragma unroll
  for (int r = 1; r < 4; ++r) sum = sum + wh[r] * __builtin_amdgcn_fmed3f(lo[r], 0.f, inf);
#pragma unroll
  for (int r = 0; r < 4; ++r) sum = sum + wh[4 + r] * __builtin_amdgcn_fmed3f(hi[r], 0.f, inf);
  return sum;
}

// Four workgroups per CU (32 KB of LDS each): at most 128 registers.
template <bool kWeights, int kMode>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(4, 4))) void prefill_score_kernel(
    const uint16_t* __restrict__ q, const float* __restrict__ w, const uint16_t* __restrict__ keys,
    int64_t n_entries, int64_t t0, int32_t ratio, int32_t n_q, float* __restrict__ scores,
    int32_t* __restrict__ n_vis, int32_t* __restrict__ win_len, int32_t win, PrefillCandOut co) {
  __shared__ __attribute__((aligned(16))) uint16_t qs[kPfQ * 8 * 64];   // [query*8 + head][dim]
  __shared__ int32_t vis_s[kPfQ];                                       // visible entries per query
  __shared__ float thr_s[kPfQ];                                         // candidate threshold per query
  __shared__ uint32_t cnt_s[kPfQ];                                      // candidates per query
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int n = lane & 15, g = lane >> 4;
  const int64_t q0 = (int64_t)blockIdx.y * kPfQ;
  if constexpr (kMode == kPfRescore) {
    // Visible counts grow with the query, so the block's last query sees
    // the most entries.
    const int64_t vis_last = min(n_entries, (t0 + min(q0 + kPfQ, (int64_t)n_q)) / ratio);
    if (co.flags[blockIdx.y] == 0u || (int64_t)blockIdx.x * kPfE >= vis_last) return;  // uniform
  }
  const int64_t e_w = (int64_t)blockIdx.x * kPfE + wave * 128;  // this wavefront's first position
  // Entry of position v of the block's entry range: v itself, or for the
  // sampled block the v-th sampled entry (n_entries >= 1,024: the runs
  // are disjoint and inside the range).
  const int64_t run = n_entries >> 6;
  auto entry_of = [&](int64_t v) -> int64_t {
    return kMode == kPfSampled ? (v >> 4) * run + (v & 15) : v;
  };

  // Key fragments of the wavefront's 8 column tiles (clamped rows; entries
  // past n_entries are never stored).
  u32x4 kf[kPfCols][2];
#pragma unroll
  for (int c = 0; c < kPfCols; ++c) {
    const int64_t e = min(entry_of(e_w + 16 * c + n), n_entries - 1);
    const u32x4* kp = reinterpret_cast<const u32x4*>(keys + e * 64 + 16 * g);
    kf[c][0] = kp[0];
    kf[c][1] = kp[1];
  }
  // The 32 queries' indexer Q into LDS (clamped rows past n_q).
#pragma unroll
  for (int i = 0; i < (kPfQ * 8 * 64) / (8 * 256); ++i) {
    const int v = tid + 256 * i;              // 16-byte vector index
    const int64_t qr = min(q0 + (v >> 6), (int64_t)n_q - 1);
    *reinterpret_cast<u32x4*>(&qs[v * 8]) =
        reinterpret_cast<const u32x4*>(q + qr * 8 * 64)[v & 63];
  }
  if (tid < kPfQ) {
    const int64_t t = t0 + q0 + tid;
    const int32_t vis = (int32_t)min(n_entries, (t + 1) / ratio);
    vis_s[tid] = vis;
    if (blockIdx.x == 0 && q0 + tid < n_q) {
      if (n_vis) n_vis[q0 + tid] = vis;
      if (win_len) win_len[q0 + tid] = (int32_t)min((int64_t)win, t + 1);  // tokens max(0, t-win+1) .. t
    }
    if constexpr (kMode == kPfCand) {
      thr_s[tid] = q0 + tid < n_q ? key_threshold(co.thr[(q0 + tid) * co.thr_stride]) : __builtin_nanf("");
      cnt_s[tid] = 0u;
    }
  }
  if constexpr (kMode == kPfCand)
    if (blockIdx.x == 0 && tid == 0) co.flags[blockIdx.y] = 0u;
  __syncthreads();

  // Entry of column tile c for this lane: e0 + 16 * c (a sampled tile is
  // one run: run apart).  Entries fit in 32 bits (n_entries <= 2^30).
  const int e0 = (int)entry_of(e_w + n);
  const int e_step = kMode == kPfSampled ? (int)run : 16;
  const int ne = (int)n_entries;
  const int64_t list_pitch = (int64_t)co.n_blocks * kCandCap;
#pragma unroll 1
  for (int qg = 0; qg < kPfQ / 4; ++qg) {
    // Row m = n of the two row tiles: query 4qg + n/4, heads n%4 and 4 + n%4,
    // dims 16g..16g+15.
    const uint16_t* ar = &qs[((4 * qg + (n >> 2)) * 8 + (n & 3)) * 64 + 16 * g];
    const bf16x8 a0 = as_bf16x8(reinterpret_cast<const u32x4*>(ar)[0]);
    const bf16x8 a1 = as_bf16x8(reinterpret_cast<const u32x4*>(ar)[1]);
    const bf16x8 b0 = as_bf16x8(reinterpret_cast<const u32x4*>(ar + 4 * 64)[0]);
    const bf16x8 b1 = as_bf16x8(reinterpret_cast<const u32x4*>(ar + 4 * 64)[1]);
    const int qi = 4 * qg + g;                 // this lane's query within the block
    const int64_t qrow = q0 + qi;
    float wh[8] = {1.f, 1.f, 1.f, 1.f, 1.f, 1.f, 1.f, 1.f};
    if (kWeights) {
      const int64_t qc = min(qrow, (int64_t)n_q - 1);
#pragma unroll
      for (int r = 0; r < 8; ++r) wh[r] = w[qc * 8 + r];
    }
    const int vis = vis_s[qi];
    float t = 0.f;
    uint2* ldst = nullptr;
    if constexpr (kMode == kPfCand) {
      t = thr_s[qi];  // NaN: no estimate, or a row past n_q -- admits nothing
      ldst = co.cand + qrow * list_pitch + (int64_t)blockIdx.x * kCandCap;
    }
    const bool row_ok = qrow < n_q;
    float* dst = scores + qrow * n_entries;
#pragma unroll
    for (int c = 0; c < kPfCols; ++c) {
      f32x4 lo = {0.f, 0.f, 0.f, 0.f}, hi = {0.f, 0.f, 0.f, 0.f};
      lo = mfma16x16x32(a0, as_bf16x8(kf[c][0]), lo);
      hi = mfma16x16x32(b0, as_bf16x8(kf[c][0]), hi);
      lo = mfma16x16x32(a1, as_bf16x8(kf[c][1]), lo);
      hi = mfma16x16x32(b1, as_bf16x8(kf[c][1]), hi);
      const float score = relu_wsum8(lo, hi, wh);
      const int e = e0 + e_step * c;
      if constexpr (kMode == kPfCand) {
        if (score >= t && e < vis) {
          const uint32_t pos = atomicAdd(&cnt_s[qi], 1u);
          if (pos < (uint32_t)kCandCap) ldst[pos] = make_uint2(__builtin_bit_cast(uint32_t, score), (uint32_t)e);
        }
      } else {
        // 16 lanes store 16 consecutive entries of one query.
        if (row_ok && e < ne) __builtin_nontemporal_store(e < vis ? score : kNegInf, dst + e);
      }
    }
  }
  if constexpr (kMode == kPfCand) {
    __syncthreads();
    if (tid < kPfQ && q0 + tid < n_q) co.cnt[(q0 + tid) * co.n_blocks + blockIdx.x] = cnt_s[tid];
  }
}


// ------------------------------------------------------- flat, local Top-k
// Flat scoring with a selection per workgroup: workgroup w of a sequence
// scores the contiguous slots [w * kLocalSlots, (w + 1) * kLocalSlots) into
// LDS (no score leaves the workgroup) and keeps its own Top-k by (score
// descending, slot ascending).  The sequence's Top-k lies in the union of
// these, so it is the Top-k of the G * k candidates, ties to the lower
// candidate index, which is the lower slot: candidates are written in slot
// order, workgroup after workgroup, as (score, slot) at
// cand[b][w * k .. w * k + k), padded with -inf.
constexpr int kLocalChunks = 16;
constexpr int kLocalSlots = kLocalChunks * kKeysPerWG;  // 8,192 slots per workgroup

template <bool kWeights>
__global__ __launch_bounds__(256) void index_score_local_kernel(
    const uint16_t* __restrict__ q, const float* __restrict__ w, const uint16_t* __restrict__ keys,
    int64_t key_cap, const int32_t* __restrict__ lens, int32_t k, float* __restrict__ cand_score,
    int32_t* __restrict__ cand_slot) {
  __shared__ uint32_t lk[kLocalSlots];  // order keys of the range (0: not a candidate)
  __shared__ uint32_t hist[kTopkBins];
  __shared__ uint32_t selw[kLocalSlots / 32], tiew[kLocalSlots / 32];
  __shared__ uint32_t wave_sum[4];
  __shared__ uint32_t found[2];
  const int b = blockIdx.y, tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int n = lane & 15, g = lane >> 4;
  const int64_t n_valid = min(key_cap, (int64_t)lens[b]);
  const int64_t s_begin = (int64_t)blockIdx.x * kLocalSlots;

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
#pragma unroll 1
  for (int c = 0; c < kLocalChunks; ++c) {
    const int local0 = c * kKeysPerWG + wave * (kTilesPerWave * 16);
    u32x4 kv[kTilesPerWave][2];
    bool valid[kTilesPerWave];
#pragma unroll
    for (int t = 0; t < kTilesPerWave; ++t) {
      const int64_t slot = s_begin + local0 + t * 16 + n;
      valid[t] = slot < n_valid;
      const u32x4* kp = reinterpret_cast<const u32x4*>(kb + (valid[t] ? slot : 0) * 64 + 16 * g);
      kv[t][0] = __builtin_nontemporal_load(kp);
      kv[t][1] = __builtin_nontemporal_load(kp + 1);
    }
#pragma unroll
    for (int t = 0; t < kTilesPerWave; ++t) {
      if (!valid[t]) kv[t][0] = kv[t][1] = u32x4{0, 0, 0, 0};
      f32x4 acc = {0.f, 0.f, 0.f, 0.f};
      acc = mfma16x16x32(qa[0], as_bf16x8(kv[t][0]), acc);
      acc = mfma16x16x32(qa[1], as_bf16x8(kv[t][1]), acc);
      const float part = relu_wsum4(acc, wh);
      const float score = fold16_add(part);  // heads 0..3 + heads 4..7
      if (g == 0) lk[local0 + t * 16 + n] = valid[t] ? order_key(score) : 0u;
    }
  }
  __syncthreads();

  // The range's k-th key T (radix select over digits of 12, 12 and 8 bits)
  // and how many keys equal to T are taken; every candidate if at most k.
  const uint32_t kk = (uint32_t)k;
  constexpr int kPer = kLocalSlots / 256;
  uint32_t cnt = 0;
#pragma unroll
  for (int j = 0; j < kPer; ++j) cnt += lk[tid + 256 * j] != 0u ? 1u : 0u;
  uint32_t total;
  block_exclusive_scan<256>(cnt, wave_sum, &total);
  uint32_t T = 1u, ties = 0u;
  if (total > kk) {
    for (int i = tid; i < kTopkBins; i += 256) hist[i] = 0;
    __syncthreads();
#pragma unroll
    for (int j = 0; j < kPer; ++j) {
      const uint32_t key = lk[tid + 256 * j];
      if (key) atomicAdd(&hist[key >> 20], 1u);
    }
    __syncthreads();
    find_threshold_bin<256>(hist, kTopkBins, kk, wave_sum, found);
    const uint32_t b1 = found[0], need1 = kk - found[1];
    for (int i = tid; i < kTopkBins; i += 256) hist[i] = 0;
    __syncthreads();
#pragma unroll
    for (int j = 0; j < kPer; ++j) {
      const uint32_t key = lk[tid + 256 * j];
      if (key && (key >> 20) == b1) atomicAdd(&hist[(key >> 8) & 0xFFFu], 1u);
    }
    __syncthreads();
    find_threshold_bin<256>(hist, kTopkBins, need1, wave_sum, found);
    const uint32_t pre2 = (b1 << 12) | found[0], need2 = need1 - found[1];
    for (int i = tid; i < 256; i += 256) hist[i] = 0;
    __syncthreads();
#pragma unroll
    for (int j = 0; j < kPer; ++j) {
      const uint32_t key = lk[tid + 256 * j];
      if (key && (key >> 8) == pre2) atomicAdd(&hist[key & 0xFFu], 1u);
    }
    __syncthreads();
    find_threshold_bin<256>(hist, 256, need2, wave_sum, found);
    T = (pre2 << 8) | found[0];
    ties = need2 - found[1];
  }
  // Selection and tie bitmaps of the range by ballots over 64-slot groups.
#pragma unroll 4
  for (int r = 0; r < kLocalSlots / 256; ++r) {
    const int s0 = (wave + 4 * r) * 64;
    const uint32_t key = lk[s0 + lane];
    const uint64_t ms = __ballot(ties > 0 ? key > T : key >= T);  // T >= 1: key 0 never taken
    const uint64_t mt = __ballot(ties > 0 && key == T);
    if (lane == 0) {
      selw[s0 >> 5] = (uint32_t)ms;
      tiew[s0 >> 5] = (uint32_t)mt;
    } else if (lane == 32) {
      selw[(s0 >> 5) + 1] = (uint32_t)(ms >> 32);
      tiew[(s0 >> 5) + 1] = (uint32_t)(mt >> 32);
    }
  }
  __syncthreads();
  // Thread tid owns word tid (slots 32 tid .. +31): the lowest `ties` tie
  // slots join, then the candidates go out in slot order.
  uint32_t sw = selw[tid];
  if (ties > 0) {
    uint32_t x = tiew[tid];
    uint32_t dummy;
    const uint32_t rank = block_exclusive_scan<256>(__popc(x), wave_sum, &dummy);
    if (rank < ties) {
      if (rank + __popc(x) > ties)
        for (uint32_t m = rank; m < ties; ++m) {
          sw |= x & (0u - x);
          x &= x - 1;
        }
      else
        sw |= x;
    }
  }
  uint32_t n_sel;
  uint32_t pos = block_exclusive_scan<256>(__popc(sw), wave_sum, &n_sel);
  const int64_t c0 = ((int64_t)b * gridDim.x + blockIdx.x) * kk;
  float* cs = cand_score + c0;
  int32_t* ci = cand_slot + c0;
  while (sw) {
    const int bit = __ffs(sw) - 1;
    sw &= sw - 1;
    const int local = 32 * tid + bit;
    if (pos < kk) {
      cs[pos] = order_key_value(lk[local]);
      ci[pos] = (int32_t)(s_begin + local);
    }
    ++pos;
  }
  for (uint32_t i = n_sel + tid; i < kk; i += 256) {
    cs[i] = kNegInf;
    ci[i] = 0;
  }
}

}  // namespace

// tile_bound / bound_k (pool mode): also the tile bounds of the bound_k-th
// largest key described at index_score_kernel.
csa2_status index_score_launch(const uint16_t* q, const float* w, const uint16_t* keys, int64_t key_cap,
                               const int32_t* lens, int32_t len_div, const int32_t* pool,
                               int32_t n_pool, int32_t blk, float* scores, int64_t n_out, int32_t n_seq,
                               uint32_t* ghist, hipStream_t stream, uint32_t* tile_bound, int32_t bound_k) {
  if (n_seq == 0 || n_out == 0) return CSA2_OK;
  // About four workgroups per CU in total; each loops over chunks of 512
  // keys, so a fused histogram is flushed by few workgroups (its hot bins
  // see one global atomic per workgroup).
  const int64_t chunks = (n_out + kKeysPerWG - 1) / kKeysPerWG;
  const int64_t per_seq = std::max<int64_t>(1, std::min<int64_t>(chunks, (1024 + n_seq - 1) / n_seq));
  CSA2_REQUIRE(n_seq <= 65535, CSA2_ESHAPE, "csa2_index_score: grid too large");
  const dim3 grid((uint32_t)per_seq, (uint32_t)n_seq);
  const int64_t tiles = (n_out + 127) / 128;  // 128-slot tiles, one per wavefront pass
  const int32_t bound_j = tile_bound ? (int32_t)std::min<int64_t>((bound_k + tiles - 1) / tiles, kBoundJMax + 1) : 0;
  if (pool) {
    if (w)
      launch_one<true, true>(grid, stream, q, w, keys, key_cap, lens, 1, pool, n_pool, blk, scores, n_out, ghist,
                             tile_bound, bound_j);
    else
      launch_one<true, false>(grid, stream, q, w, keys, key_cap, lens, 1, pool, n_pool, blk, scores, n_out, ghist,
                              tile_bound, bound_j);
  } else {
    if (w)
      launch_one<false, true>(grid, stream, q, w, keys, key_cap, lens, len_div, pool, 0, 1, scores, n_out, ghist,
                              nullptr, 0);
    else
      launch_one<false, false>(grid, stream, q, w, keys, key_cap, lens, len_div, pool, 0, 1, scores, n_out, ghist,
                               nullptr, 0);
  }
  return launch_status("csa2_index_score");
}

}  // namespace csa2

namespace csa2 {

// Workgroups per sequence of the flat scoring with local selection.
int64_t index_score_local_groups(int64_t key_cap) { return (key_cap + kLocalSlots - 1) / kLocalSlots; }

// Whether a flat selection of k over key_cap positions for n_seq sequences
// keeps per-workgroup candidates instead of writing every score (the
// groups, else 0): the candidates must fit the single-workgroup selection,
// and up to kTopkRowsMax positions the scoring workgroups must fill the
// chip (each streams its 8,192 positions at a latency-bound rate: 4 groups
// x 32 sequences took 75 us against 44 us for scores written and selected,
// 8 x 32 took 80 against 95 us).
int64_t flat_local_groups(int64_t key_cap, int32_t k, int32_t n_seq) {
  const int64_t groups = index_score_local_groups(key_cap);
  if (groups * k > kTopkRowsMax) return 0;
  if (key_cap > kTopkRowsMax) return groups;
  return groups >= 4 && groups * n_seq >= 256 ? groups : 0;
}

csa2_status index_score_local_launch(const uint16_t* q, const float* w, const uint16_t* keys, int64_t key_cap,
                                     const int32_t* lens, int32_t k, float* cand_score, int32_t* cand_slot,
                                     int32_t n_seq, hipStream_t stream) {
  if (n_seq == 0 || key_cap == 0) return CSA2_OK;
  const int64_t groups = index_score_local_groups(key_cap);
  CSA2_REQUIRE(groups <= 0x7FFFFFFF && n_seq <= 65535 && k >= 1 && k <= CSA2_TOPK_MAX, CSA2_ESHAPE,
               "flat local selection: bad shape");
  const dim3 grid((uint32_t)groups, (uint32_t)n_seq);
  if (w)
    hipLaunchKernelGGL(index_score_local_kernel<true>, grid, dim3(256), 0, stream, q, w, keys, key_cap, lens, k,
                       cand_score, cand_slot);
  else
    hipLaunchKernelGGL(index_score_local_kernel<false>, grid, dim3(256), 0, stream, q, w, keys, key_cap, lens, k,
                       cand_score, cand_slot);
  return launch_status("csa2_index_score (local selection)");
}

namespace {

template <int kMode>
void prefill_launch_mode(dim3 grid, hipStream_t stream, const uint16_t* q, const float* w, const uint16_t* keys,
                         int64_t n_entries, int64_t t0, int32_t ratio, int32_t n_q, float* scores, int32_t* n_vis,
                         int32_t* win_len, int32_t win, const PrefillCandOut& co) {
  if (w)
    hipLaunchKernelGGL((prefill_score_kernel<true, kMode>), grid, dim3(256), 0, stream, q, w, keys, n_entries, t0,
                       ratio, n_q, scores, n_vis, win_len, win, co);
  else
    hipLaunchKernelGGL((prefill_score_kernel<false, kMode>), grid, dim3(256), 0, stream, q, w, keys, n_entries,
                       t0, ratio, n_q, scores, n_vis, win_len, win, co);
}

}  // namespace

csa2_status prefill_score_launch(const uint16_t* q, const float* w, const uint16_t* keys, int64_t n_entries,
                                 int64_t t0, int32_t ratio, int32_t n_q, float* scores, int32_t* n_vis,
                                 int32_t* win_len, int32_t win, hipStream_t stream) {
  if (n_q == 0 || n_entries == 0) return CSA2_OK;
  const int64_t gx = (n_entries + kPfE - 1) / kPfE, gy = (n_q + kPfQ - 1) / kPfQ;
  CSA2_REQUIRE(gy <= 65535, CSA2_ESHAPE, "csa2_prefill_index_score: too many queries");
  prefill_launch_mode<kPfAll>(dim3((uint32_t)gx, (uint32_t)gy), stream, q, w, keys, n_entries, t0, ratio, n_q,
                              scores, n_vis, win_len, win, PrefillCandOut{});
  return launch_status("csa2_prefill_index_score");
}

// The scoring passes of a prefill selection filtered while scoring:
// stage 0 scores the sampled entries (and writes n_vis and win_len),
// stage 1 writes the candidates at or above co.thr, stage 2 rescores the
// query blocks flagged in co.flags.  1,024 <= n_entries <= kTopkRowsMax.
csa2_status prefill_filter_launch(int stage, const uint16_t* q, const float* w, const uint16_t* keys,
                                  int64_t n_entries, int64_t t0, int32_t ratio, int32_t n_q, float* scores,
                                  int32_t* n_vis, int32_t* win_len, int32_t win, const PrefillCandOut& co,
                                  hipStream_t stream) {
  if (n_q == 0) return CSA2_OK;
  CSA2_REQUIRE(n_entries >= 1024 && n_entries <= kTopkRowsMax && (n_q + kPfQ - 1) / kPfQ <= 65535, CSA2_ESHAPE,
               "prefill selection: need 1,024 <= n_entries <= 65,536 and fewer than 2^21 queries");
  CSA2_REQUIRE(stage == 0 || (co.cnt && co.cand && co.flags && co.n_blocks == (n_entries + kPfE - 1) / kPfE &&
                              (stage == 2 || co.thr)),
               CSA2_EINVAL, "prefill selection: candidate buffers missing");
  const uint32_t gy = (uint32_t)((n_q + kPfQ - 1) / kPfQ);
  const uint32_t gx = (uint32_t)((n_entries + kPfE - 1) / kPfE);
  if (stage == 0)
    prefill_launch_mode<kPfSampled>(dim3(1024 / kPfE, gy), stream, q, w, keys, n_entries, t0, ratio, n_q, scores,
                                    n_vis, win_len, win, co);
  else if (stage == 1)
    prefill_launch_mode<kPfCand>(dim3(gx, gy), stream, q, w, keys, n_entries, t0, ratio, n_q, scores, nullptr,
                                 nullptr, win, co);
  else
    prefill_launch_mode<kPfRescore>(dim3(gx, gy), stream, q, w, keys, n_entries, t0, ratio, n_q, scores, nullptr,
                                    nullptr, win, co);
  return launch_status("csa2_prefill_chunk (indexer scores)");
}

}  // namespace csa2
