// Steps (d) + (e) for many queries over one cache sequence (a prefill
// chunk): two wavefronts attend for one query over all of its rows.
//
// [P1 "Compressed Sparse Attention 2 (CSA2)"]: each query attends with its
// own main Q over its selected positions; [P1 "Causal Encoder-Decoder: Half
// the Prefill"]: plus a 128-token window; [P3]: keys and values share one
// 512-d latent (K = V); [P1 "FP4 KV, ..."]: rows are E2M1 values with one
// E4M3 scale per 16 channels.  The arithmetic is that of the workgroup
// kernels in sparse_attn.hip (f16 operands, exact dequantisation, fp32
// accumulation, P split into f16 hi + lo); what differs is the schedule:
//   - a chunk of FP4 rows whose E4M3 scales are all <= 1.25 (|x| <= 7.5)
//     takes P rounded once to f16 (to nearest) instead of hi + lo: the
//     output then moves by at most 2^-11 * 7.5 < 3.7e-3 per element (each
//     weight is off by at most 2^-11 of itself, and the weights of the
//     normaliser are exact), inside the 5e-3 absolute bound, with one P X
//     product instead of two (per wavefront, from its own channels' scales;
//     window chunks and chunks with larger scales keep hi + lo);
//   - a query's two wavefronts split the channels: wavefront w loads,
//     converts and stores channels 256w..256w+255 of every row, keeps O for
//     those channels (16 heads x 256, fp32) in registers for the whole
//     query and its half of main Q, and computes S over its half; the two
//     partial S tiles are added through LDS once per chunk, so that both
//     wavefronts hold the same S (IEEE addition is commutative) and take
//     the same softmax steps without any other exchange.  About 240
//     registers each: two wavefronts per SIMD, which hide each other's
//     latencies;
//   - the rows go in chunks of 32 (two tiles of 16); the raw loads of the
//     next chunk of selected rows (32 code bytes + 4 scale bytes per lane
//     and tile) are issued a chunk ahead, their row ids taken from the
//     query's ids, which are staged in LDS once;
//   - S^T = X Q^T on v_mfma_f32_16x16x32_f16 from the converted registers
//     (lane (n, g): row n, channels 256w + 64g .. +63), while the converted
//     rows also go to the wavefront's own half tile in LDS, from which the
//     P X product reads its B operands transposed (ds_read_b64_tr_b16: rows
//     4g..4g+3 of each tile along K);
//   - the next chunk's rows are converted, stored and multiplied by Q inside
//     the current chunk's P X loop, as the LDS tile frees up (LDS
//     operations of one wavefront complete in order), with each MFMA
//     followed by a few VALU instructions in issue order;
//   - the softmax reference maximum is set once per head, by the first
//     chunk with a row; later chunks are exponentiated against it, which
//     gives the same softmax (the weights are exact up to rounding whatever
//     the reference) as long as no weight exceeds 2^kLazyLog2 (inside f16's
//     range).  A query where one would is attended again against its exact
//     maximum, found by a pass of S alone: never on ordinary scores, and at
//     most twice the work.
// The window chunks come last, read straight from the window rows (shared
// with the neighbouring queries through the L2: queries are dealt to the
// XCDs in contiguous runs).
//
// Citation keys: [P1] "DeepSeek AI Released DeepSeek-V4.1-Flash with 1M
// Context, FP4 KV Cache, and Cross-Layer Attention Reuse"; [P3]
// "DeepSeek-V4.1 Flash: Pushing the Limits of KV Cache Compression".
#include <type_traits>

#include "attn_dev.hpp"
#include "common.hpp"

namespace csa2 {

namespace {

constexpr float kLazyLog2 = 15.f;
constexpr int kValuPerMfma = 3;  // VALU instructions issued after each MFMA (see pair_pv_next)
// Window rows are read straight from memory (the L2, mostly): each channel
// group's loads are issued kWinLead groups ahead of its use.
constexpr int kWinLead = 3;
constexpr int kWaveMaxIdx = kAttnManyMaxIdx;  // selected rows per query (at most)

// One window row of zeros: the address of every window row past a query's
// window (its values convert to 0 and need no masking).
__device__ __attribute__((aligned(16))) const uint32_t kWaveZeroRow[2 * CSA2_LATENT / 4] = {};

// Loads through the global address space (global_load: counted by vmcnt
// alone, unlike flat loads, which also count against the LDS counter).
typedef const __attribute__((address_space(1))) u32x4* gu32x4p;
typedef const __attribute__((address_space(1))) uint32_t* gu32p;

struct WaveArgs {
  const uint8_t* codes;
  const uint8_t* scales;
  int64_t cap;
  int64_t kv_row0;
};

// Scores of a chunk as exponents of 2 (lane (n, g): z[4t + j] = row 4g+j of
// tile t, head n; -inf for rows not attended over) and their maximum per
// head.
__device__ __forceinline__ float wave_scores(const f32x4 (&s)[2], const uint64_t (&ok)[2], float scale_log2, int g,
                                             float (&z)[8]) {
  float m = kNegInf;
#pragma unroll
  for (int t = 0; t < 2; ++t) {
    const uint32_t ok4 = (uint32_t)(ok[t] >> (4 * g));
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      z[4 * t + j] = ((ok4 >> j) & 1) ? s[t][j] * scale_log2 : kNegInf;
      m = fmaxf(m, z[4 * t + j]);
    }
  }
  return fold32_max(fold16_max(m));
}

// Softmax weights of a chunk against the reference maximum, as the A
// operands of the P X product (hi[0..3] / lo[0..3]: P hi / lo of rows
// 4g..4g+3 of tile 0, then of tile 1).  The first chunk with a row sets the
// reference; returns false when a later chunk exceeds it by more than
// kLazyLog2 (unless the reference is fixed): the pass is then abandoned at
// the end of the step (after its loads have been issued, so that every
// path to the next step passes them).
template <class St>
__device__ __forceinline__ bool wave_softmax(St& st, const f32x4 (&s)[2], const uint64_t (&ok)[2],
                                             float scale_log2, int g, bool fixed, u32x4& hi, u32x4& lo,
                                             bool single = false) {
  float z[8];
  const float m = wave_scores(s, ok, scale_log2, g, z);
  // (Uniform selects, no branch: the step stays one block.)  The first
  // chunk with a row sets the reference (O and l are still 0).
  const bool above = !fixed && __ballot(m > st.m_run + kLazyLog2) != 0;
  const bool unset = __ballot(st.m_run != kNegInf) == 0;
  st.m_run = (above && unset) ? m : st.m_run;
  // Rows not attended over have z = -inf and weight exp2(-inf) = 0; the
  // reference is -inf only while no row has been seen (then every z is).
  const float mr = st.m_run == kNegInf ? 0.f : st.m_run;
  float p[8];
  float lsum = 0.f;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    p[i] = __builtin_amdgcn_exp2f(z[i] - mr);
    lsum += p[i];
  }
  st.l_run += fold32_add(fold16_add(lsum));
  if (!single) {
    // P = hi + lo in f16 (toward zero; p - hi is exact in binary32).
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const f16x2 h = __builtin_bit_cast(f16x2, __builtin_amdgcn_cvt_pkrtz(p[2 * i], p[2 * i + 1]));
      const f16x2 l =
          __builtin_bit_cast(f16x2, __builtin_amdgcn_cvt_pkrtz(p[2 * i] - (float)h[0], p[2 * i + 1] - (float)h[1]));
      hi[i] = __builtin_bit_cast(uint32_t, h);
      lo[i] = __builtin_bit_cast(uint32_t, l);
    }
  } else {
    // P rounded once to f16, to nearest.
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const f16x2 h = {(_Float16)p[2 * i], (_Float16)p[2 * i + 1]};
      hi[i] = __builtin_bit_cast(uint32_t, h);
      lo[i] = 0u;
    }
  }
  return !(above && !unset);
}

typedef short wave_v4s __attribute__((ext_vector_type(4)));

// ------------------------------------------------ the kernel
constexpr int kPPitch = CSA2_LATENT / 2 + 8;  // LDS row pitch of a half tile, f16 elements

struct PairState {
  f32x4 o[16];  // block b: lane (n, g), element j = head 4g+j, channel 256w + 16b + n
  float m_run;
  float l_run;
};

// The raw loads of one chunk, this wavefront's half of each row.
struct PairSlot {
  u32x4 c[2][2];   // tile t: 32 code bytes (channels 256w + 64g .. +63)
  uint32_t s4[2];  // tile t: their 4 scale bytes
  uint64_t ok[2];
};

__device__ __forceinline__ void pair_issue(PairSlot& sl, const WaveArgs& a, int32_t id0, int32_t id1, int w, int g) {
#pragma unroll
  for (int t = 0; t < 2; ++t) {
    const int32_t id = t ? id1 : id0;
    const bool ok = id >= 0 && id < a.cap;
    const int64_t row = a.kv_row0 + (ok ? id : 0);
    const gu32x4p cp = (gu32x4p)(a.codes + row * CSA2_CODE_BYTES + 128 * w + 32 * g);
    sl.c[t][0] = cp[0];
    sl.c[t][1] = cp[1];
    sl.s4[t] = *(gu32p)(a.scales + row * CSA2_SCALE_BYTES + 16 * w + 4 * g);
    sl.ok[t] = __ballot(ok);
  }
}

// Whether every scale byte of the chunk in sl (this wavefront's channels
// of both tiles; rows that are not attended count as 0) is an E4M3 value
// <= 1.25 (code 0x3A), so that every dequantised |x| <= 6 * 1.25: per byte,
// the low 7 bits + 0x45 reach bit 7 iff they exceed 0x3A (no carry crosses
// a byte), and a set sign bit counts as large.  Uniform over the wavefront.
__device__ __forceinline__ bool fp4_chunk_small(const PairSlot& sl, int n) {
  uint32_t big = 0u;
#pragma unroll
  for (int t = 0; t < 2; ++t) {
    const uint32_t s4 = ((sl.ok[t] >> n) & 1) ? sl.s4[t] : 0u;
    big |= ((s4 & 0x7F7F7F7Fu) + 0x45454545u) | s4;
  }
  return __ballot((big & 0x80808080u) != 0u) == 0;
}

struct PairFp4Src {
  static constexpr bool kHas = true;
  const PairSlot& sl;
  uint32_t sc[2][4];
  __device__ __forceinline__ PairFp4Src(const PairSlot& s, int n) : sl(s) {
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      const uint32_t s4 = ((s.ok[t] >> n) & 1) ? s.s4[t] : 0u;
      sc[t][0] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(s4, 1.0f, false));
      sc[t][1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(s4, 1.0f, true));
      sc[t][2] = sc[t][3] = 0u;
    }
  }
  __device__ __forceinline__ void issue(int) {}
  // Channel group k (0..7): channels 256w + 64g + 8k .. +7, scale byte k / 2.
  __device__ __forceinline__ u32x4 x(int t, int k) const {
    return dequant8_f16(sl.c[t][k >> 2][k & 3], scale_pair(sc[t], k));
  }
};

template <int kWin>
struct PairWinSrc {
  static constexpr bool kHas = true;
  gu32x4p p[2];  // the lane's 64 channels of its row in each tile (or of the zero row)
  u32x4 v[2][8];
  __device__ __forceinline__ void issue(int k) {
    if (k < 8) {
      v[0][k] = p[0][k];
      v[1][k] = p[1][k];
    }
  }
  __device__ __forceinline__ u32x4 x(int t, int k) const { return bf16x8_to_f16x8(v[t][k]); }
};

struct PairNoSrc {
  static constexpr bool kHas = false;
  __device__ __forceinline__ void issue(int) {}
  __device__ __forceinline__ u32x4 x(int, int) const { return u32x4{0u, 0u, 0u, 0u}; }
};

struct PairBGroup {
  wave_v4s t[4][2];
};

// The B operands of the P X blocks kk + 4i (i = 0..3) of this wavefront's
// half tile.
__device__ __forceinline__ PairBGroup pair_read_group(const uint16_t* xs, int kk, int n, int g) {
  PairBGroup r;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const uint16_t* a0 = &xs[(4 * g + (n >> 2)) * kPPitch + 16 * (kk + 4 * i) + 4 * (n & 3)];
#pragma unroll
    for (int t = 0; t < 2; ++t)
      r.t[i][t] = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
          (__attribute__((address_space(3))) wave_v4s*)(a0 + 16 * t * kPPitch));
  }
  return r;
}

// O += lo X over this wavefront's half tile (the lo part of P of a chunk
// whose hi part goes through pair_pv_next<false>).
__device__ __forceinline__ void pair_pv_lo(PairState& st, const uint16_t* xs, u32x4 lo, int n, int g) {
#pragma unroll
  for (int kk = 0; kk < 4; ++kk) {
    const PairBGroup cur = pair_read_group(xs, kk, n, g);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const uint2 u0 = __builtin_bit_cast(uint2, cur.t[i][0]), u1 = __builtin_bit_cast(uint2, cur.t[i][1]);
      st.o[kk + 4 * i] = mfma16x16x32_f16(as_f16x8(lo), as_f16x8(u32x4{u0.x, u0.y, u1.x, u1.y}), st.o[kk + 4 * i]);
    }
  }
}

// O += P X over this wavefront's 256 channels, and the next chunk's half
// rows: group k (local channels 64g + 8k..) is stored once the blocks
// k/2 + 4i that read those columns have been read.
template <bool kLo = true, class Src>
__device__ __forceinline__ void pair_pv_next(PairState& st, uint16_t* xs, u32x4 hi, u32x4 lo, const u32x4 (&qv)[8],
                                             Src&& src, f32x4 (&s_next)[2], int n, int g) {
  f32x4 s_odd[2] = {{0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}};
#pragma unroll
  for (int k = 0; k < 2 * kWinLead; ++k) src.issue(k);
  PairBGroup cur = pair_read_group(xs, 0, n, g);
#pragma unroll
  for (int kk = 0; kk < 4; ++kk) {
    PairBGroup nxt;
    if (kk < 3) nxt = pair_read_group(xs, kk + 1, n, g);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int b = kk + 4 * i;
      const uint2 u0 = __builtin_bit_cast(uint2, cur.t[i][0]), u1 = __builtin_bit_cast(uint2, cur.t[i][1]);
      const f16x8 bx = as_f16x8(u32x4{u0.x, u0.y, u1.x, u1.y});
      st.o[b] = mfma16x16x32_f16(as_f16x8(hi), bx, st.o[b]);
      if constexpr (kLo) st.o[b] = mfma16x16x32_f16(as_f16x8(lo), bx, st.o[b]);
    }
    if constexpr (std::remove_reference_t<Src>::kHas) {
#pragma unroll
      for (int k = 2 * kk; k < 2 * kk + 2; ++k)
#pragma unroll
        for (int t = 0; t < 2; ++t) {
          const u32x4 x = src.x(t, k);
          *reinterpret_cast<u32x4*>(&xs[(16 * t + n) * kPPitch + 64 * g + 8 * k]) = x;
          if (k & 1)
            s_odd[t] = mfma16x16x32_f16(as_f16x8(x), as_f16x8(qv[k]), s_odd[t]);
          else
            s_next[t] = mfma16x16x32_f16(as_f16x8(x), as_f16x8(qv[k]), s_next[t]);
        }
      src.issue(2 * kk + 2 * kWinLead);
      src.issue(2 * kk + 2 * kWinLead + 1);
    }
    __builtin_amdgcn_sched_group_barrier(0x100, 8, 0);
#pragma unroll
    for (int i = 0; i < (kLo ? 12 : 8); ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x002, kValuPerMfma, 0);
    }
    __builtin_amdgcn_sched_group_barrier(0x200, 4, 0);
    __builtin_amdgcn_sched_barrier(0);
    if (kk < 3) cur = nxt;
  }
  if constexpr (std::remove_reference_t<Src>::kHas) {
    s_next[0] += s_odd[0];
    s_next[1] += s_odd[1];
  }
}

// S = the two wavefronts' partial S tiles added (the same sum, bit for
// bit, in both: IEEE addition is commutative).  Two barriers: the second
// keeps the next exchange's stores behind this one's loads.
__device__ __forceinline__ void pair_exchange(f32x4 (&s)[2], f32x4* ex, int w, int lane) {
  ex[(2 * w + 0) * 64 + lane] = s[0];
  ex[(2 * w + 1) * 64 + lane] = s[1];
  lds_barrier();
  const f32x4 o0 = ex[(2 * (1 - w) + 0) * 64 + lane], o1 = ex[(2 * (1 - w) + 1) * 64 + lane];
  s[0] = s[0] + o0;
  s[1] = s[1] + o1;
  lds_barrier();
}

template <int kWin>
__global__ __launch_bounds__(128) __attribute__((amdgpu_waves_per_eu(2, 2))) void attn_pair_kernel(
    const uint16_t* __restrict__ q, const uint8_t* __restrict__ codes, const uint8_t* __restrict__ scales,
    int64_t cap, int32_t q_per_seq, const int32_t* __restrict__ idx, int32_t k_idx,
    const uint8_t* __restrict__ swa, int64_t swa_q_stride_rows, const int32_t* __restrict__ swa_len,
    int32_t swa_max, float scale_log2, float* __restrict__ out) {
  __shared__ __attribute__((aligned(16))) uint16_t xs_all[2][32 * kPPitch];
  __shared__ f32x4 ex[4 * 64];
  __shared__ int32_t ids_s[kWaveMaxIdx];
  const int tid = threadIdx.x, lane = tid & 63, n = lane & 15, g = lane >> 4;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  uint16_t* xs = xs_all[w];
  const int nq = gridDim.x, per = nq / 8, rem = nq % 8;
  const int xcd = blockIdx.x % 8;
  const int qb = xcd * per + min(xcd, rem) + blockIdx.x / 8;

  WaveArgs a;
  a.codes = codes;
  a.scales = scales;
  a.cap = cap;
  a.kv_row0 = (int64_t)(qb / q_per_seq) * cap;
  const int32_t* qidx = idx + (int64_t)qb * k_idx;
  const int n_fc = (k_idx + 31) / 32;
  {
    int32_t v[kWaveMaxIdx / 128];
#pragma unroll
    for (int i = 0; i < kWaveMaxIdx / 128; ++i) v[i] = k_idx > 0 ? qidx[min(128 * i + tid, k_idx - 1)] : -1;
#pragma unroll
    for (int i = 0; i < kWaveMaxIdx / 128; ++i) ids_s[128 * i + tid] = 128 * i + tid < k_idx ? v[i] : -1;
  }
  lds_barrier();
  auto id_of = [&](int c, int t) -> int32_t { return c < n_fc ? ids_s[32 * c + 16 * t + n] : -1; };

  const int n_swa = min(swa_len[qb], swa_max);
  const int n_wc = (n_swa + 31) / 32;
  constexpr int kWinRowBytes = 2 * CSA2_LATENT;
  auto win_src = [&](int wc) -> PairWinSrc<kWin> {
    PairWinSrc<kWin> src;
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      const int j = 32 * wc + 16 * t + n;
      const uint8_t* row = j < n_swa ? swa + ((int64_t)qb * swa_q_stride_rows + j) * kWinRowBytes
                                     : reinterpret_cast<const uint8_t*>(kWaveZeroRow);
      src.p[t] = (gu32x4p)(row + 2 * (256 * w + 64 * g));
    }
    return src;
  };
  auto win_ok = [&](int wc, uint64_t (&ok)[2]) {
    ok[0] = __ballot(32 * wc + n < n_swa);
    ok[1] = __ballot(32 * wc + 16 + n < n_swa);
  };

  // This wavefront's half of main Q as f16: head n, channels 256w + 64g ..
  u32x4 qv[8];
  {
    const u32x4* qp = reinterpret_cast<const u32x4*>(q + ((int64_t)qb * 16 + n) * CSA2_LATENT + 256 * w + 64 * g);
#pragma unroll
    for (int i = 0; i < 8; ++i) qv[i] = qp[i];
#pragma unroll
    for (int i = 0; i < 8; ++i) qv[i] = bf16x8_to_f16x8(qv[i]);
  }

  bool fixed = false;
  float m_fix = kNegInf;
  PairState st;
attend:
#pragma unroll
  for (int b = 0; b < 16; ++b) st.o[b] = f32x4{0.f, 0.f, 0.f, 0.f};
  st.m_run = m_fix;
  st.l_run = 0.f;
  {
    PairSlot ring;
    pair_issue(ring, a, id_of(0, 0), id_of(0, 1), w, g);
    f32x4 s_cur[2] = {{0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}};
    uint64_t ok_cur[2] = {0, 0};
    auto first = [&](auto&& src) {
#pragma unroll
      for (int k = 0; k < 8; ++k) src.issue(k);
#pragma unroll
      for (int k = 0; k < 8; ++k)
#pragma unroll
        for (int t = 0; t < 2; ++t) {
          const u32x4 x = src.x(t, k);
          *reinterpret_cast<u32x4*>(&xs[(16 * t + n) * kPPitch + 64 * g + 8 * k]) = x;
          s_cur[t] = mfma16x16x32_f16(as_f16x8(x), as_f16x8(qv[k]), s_cur[t]);
        }
    };
    bool small_cur = false;  // the FP4 chunk in xs takes a single f16 P
    if (n_fc > 0) {
      small_cur = fp4_chunk_small(ring, n);
      first(PairFp4Src(ring, n));
      ok_cur[0] = ring.ok[0];
      ok_cur[1] = ring.ok[1];
      pair_issue(ring, a, id_of(1, 0), id_of(1, 1), w, g);
    } else if (n_wc > 0) {
      first(win_src(0));
      win_ok(0, ok_cur);
    }
    bool bad = false;
#pragma unroll 1
    for (int c = 0; c + 1 < n_fc; ++c) {
      pair_exchange(s_cur, ex, w, lane);
      u32x4 hi, lo;
      f32x4 s_next[2] = {{0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}};
      const bool small_next = fp4_chunk_small(ring, n);
      bad |= !wave_softmax(st, s_cur, ok_cur, scale_log2, g, fixed, hi, lo, small_cur);
      if (!small_cur) pair_pv_lo(st, xs, lo, n, g);
      pair_pv_next<false>(st, xs, hi, lo, qv, PairFp4Src(ring, n), s_next, n, g);
      small_cur = small_next;
      ok_cur[0] = ring.ok[0];
      ok_cur[1] = ring.ok[1];
      pair_issue(ring, a, id_of(c + 2, 0), id_of(c + 2, 1), w, g);
      s_cur[0] = s_next[0];
      s_cur[1] = s_next[1];
      if (bad) goto exceeded;
    }
    if (n_fc > 0 && n_wc > 0) {
      pair_exchange(s_cur, ex, w, lane);
      u32x4 hi, lo;
      f32x4 s_next[2] = {{0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}};
      const bool fits = wave_softmax(st, s_cur, ok_cur, scale_log2, g, fixed, hi, lo, small_cur);
      if (!small_cur) pair_pv_lo(st, xs, lo, n, g);
      pair_pv_next<false>(st, xs, hi, lo, qv, win_src(0), s_next, n, g);
      win_ok(0, ok_cur);
      s_cur[0] = s_next[0];
      s_cur[1] = s_next[1];
      if (!fits) goto exceeded;
    }
#pragma unroll 1
    for (int wc = 0; wc + 1 < n_wc; ++wc) {
      pair_exchange(s_cur, ex, w, lane);
      u32x4 hi, lo;
      const bool fits = wave_softmax(st, s_cur, ok_cur, scale_log2, g, fixed, hi, lo);
      f32x4 s_next[2] = {{0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}};
      pair_pv_next(st, xs, hi, lo, qv, win_src(wc + 1), s_next, n, g);
      win_ok(wc + 1, ok_cur);
      s_cur[0] = s_next[0];
      s_cur[1] = s_next[1];
      if (!fits) goto exceeded;
    }
    if (n_fc > 0 || n_wc > 0) {
      pair_exchange(s_cur, ex, w, lane);
      u32x4 hi, lo;
      const bool fits = wave_softmax(st, s_cur, ok_cur, scale_log2, g, fixed, hi, lo);
      f32x4 s_next[2];
      pair_pv_next(st, xs, hi, lo, qv, PairNoSrc{}, s_next, n, g);
      if (!fits) goto exceeded;
    }
  }
  {
    float inv[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const float l = __int_as_float(__builtin_amdgcn_ds_bpermute(4 * (4 * g + j), __float_as_int(st.l_run)));
      inv[j] = l > 0.f ? 1.f / l : 0.f;
    }
    float* po = out + ((int64_t)qb * 16 + 4 * g) * CSA2_LATENT + 256 * w + n;
#pragma unroll
    for (int b = 0; b < 16; ++b)
#pragma unroll
      for (int j = 0; j < 4; ++j) po[j * CSA2_LATENT + 16 * b] = st.o[b][j] * inv[j];
    return;
  }

exceeded:
  // Both wavefronts take the same decision (the same S, the same steps):
  // the exact maximum over all the query's rows, then the query again.
  {
    float m = kNegInf;
#pragma unroll 1
    for (int c = 0; c < n_fc; ++c) {
      PairSlot sl;
      pair_issue(sl, a, id_of(c, 0), id_of(c, 1), w, g);
      const PairFp4Src src(sl, n);
      f32x4 s[2] = {{0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}};
#pragma unroll
      for (int k = 0; k < 8; ++k)
#pragma unroll
        for (int t = 0; t < 2; ++t) s[t] = mfma16x16x32_f16(as_f16x8(src.x(t, k)), as_f16x8(qv[k]), s[t]);
      pair_exchange(s, ex, w, lane);
      float z[8];
      m = fmaxf(m, wave_scores(s, sl.ok, scale_log2, g, z));
    }
#pragma unroll 1
    for (int wc = 0; wc < n_wc; ++wc) {
      PairWinSrc<kWin> src = win_src(wc);
#pragma unroll
      for (int k = 0; k < 8; ++k) src.issue(k);
      uint64_t ok[2];
      win_ok(wc, ok);
      f32x4 s[2] = {{0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}};
#pragma unroll
      for (int k = 0; k < 8; ++k)
#pragma unroll
        for (int t = 0; t < 2; ++t) s[t] = mfma16x16x32_f16(as_f16x8(src.x(t, k)), as_f16x8(qv[k]), s[t]);
      pair_exchange(s, ex, w, lane);
      float z[8];
      m = fmaxf(m, wave_scores(s, ok, scale_log2, g, z));
    }
    m_fix = m;
    fixed = true;
  }
  goto attend;
}

}  // namespace

// Launch: one 128-thread workgroup (two wavefronts) per query over bf16
// window rows (win = kWinBf16).
csa2_status attn_many_launch(const uint16_t* q, int32_t n_q, const csa2_fp4_kv& kv, int32_t q_per_seq,
                             const int32_t* idx, int32_t k_idx, const uint8_t* swa, int win,
                             int64_t swa_q_stride_rows, const int32_t* swa_len, int32_t swa_max, float scale_log2,
                             float* out, hipStream_t stream) {
  CSA2_REQUIRE(k_idx <= kWaveMaxIdx && win == kWinBf16, CSA2_EINVAL,
               "attention (many queries): k_idx above 512 or an unsupported window type");
  hipLaunchKernelGGL(attn_pair_kernel<kWinBf16>, dim3(n_q), dim3(128), 0, stream, q, kv.codes, kv.scales, kv.cap,
                     q_per_seq, idx, k_idx, swa, swa_q_stride_rows, swa_len, swa_max, scale_log2, out);
  return launch_status("csa2_sparse_attn");
}

}  // namespace csa2
