// Steps (d) + (e) for many queries over one cache sequence (a prefill
// chunk): one wavefront attends for one query over all of its rows.
//
// [P1 "Compressed Sparse Attention 2 (CSA2)"]: each query attends with its
// own main Q over its selected positions; [P1 "Causal Encoder-Decoder: Half
// the Prefill"]: plus a 128-token window; [P3]: keys and values share one
// 512-d latent (K = V); [P1 "FP4 KV, ..."]: rows are E2M1 values with one
// E4M3 scale per 16 channels.  The arithmetic is that of the workgroup
// kernels in sparse_attn.hip (f16 operands, exact dequantisation, fp32
// accumulation, P split into f16 hi + lo); what differs is the schedule:
//   - no cross-wavefront step at all: O (16 heads x 512 channels, fp32)
//     stays in the wavefront's accumulation registers for the whole query,
//     and the softmax statistics are folded across lanes only;
//   - the rows go in chunks of 32 (two tiles of 16); the raw loads of the
//     next chunk of selected rows (64 code bytes + 8 scale bytes per lane
//     and tile) are issued a chunk ahead, their row ids taken from the
//     query's ids, which are staged in LDS once;
//   - S^T = X Q^T on v_mfma_f32_16x16x32_f16 from the converted registers
//     (lane (n, g): row n, channels 128g..128g+127; main Q, f16, stays in
//     registers as the B operand), while the converted rows also go to the
//     wavefront's own LDS tile, from which the P X product reads its B
//     operands transposed (ds_read_b64_tr_b16: rows 4g..4g+3 of each tile
//     along K);
//   - the next chunk's rows are converted, stored and multiplied by Q inside
//     the current chunk's P X loop, eight channels at a time as the LDS
//     tile frees up (LDS operations of one wavefront complete in order),
//     with each MFMA followed by a few VALU instructions in issue order: a
//     lone wavefront on its SIMD issues in order, so that an MFMA waiting
//     for the matrix unit would otherwise hold back the conversions;
//   - the softmax reference maximum is set once per head, by the first
//     chunk with a row; later chunks are exponentiated against it, which
//     gives the same softmax (the weights are exact up to rounding whatever
//     the reference) as long as no weight exceeds 2^kLazyLog2 (inside f16's
//     range).  A query where one would is attended again against its exact
//     maximum, found by a pass of S alone: never on ordinary scores, and at
//     most twice the work.
// The window chunks come last, read straight from the window rows (shared
// with the neighbouring queries through the L2: queries are dealt to the
// XCDs in contiguous runs), each channel group's loads issued kWinLead
// groups ahead.
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
constexpr int kValuPerMfma = 3;  // VALU instructions issued after each MFMA (see wave_pv_next)
constexpr int kWPitch = CSA2_LATENT + 8;  // LDS row pitch, f16 elements
constexpr int kWaveMaxIdx = kAttnWaveMaxIdx;  // selected rows per query (at most)

// One window row of zeros: the address of every window row past a query's
// window (its values convert to 0 and need no masking).
__device__ __attribute__((aligned(16))) const uint32_t kWaveZeroRow[2 * CSA2_LATENT / 4] = {};

// Loads through the global address space (global_load: counted by vmcnt
// alone, unlike flat loads, which also count against the LDS counter).
typedef const __attribute__((address_space(1))) u32x4* gu32x4p;
typedef const __attribute__((address_space(1))) uint64_t* gu64p;

struct WaveState {
  f32x4 o[32];  // block b: lane (n, g), element j = head 4g+j, channel 16b + n
  float m_run;  // reference maximum of head n (every lane group holds it)
  float l_run;  // running denominator of head n (likewise)
};

// One ring slot: the raw loads of one chunk (two tiles of 16 selected rows).
struct WaveSlot {
  u32x4 c[2][4];
  uint2 s8[2];
  uint64_t ok[2];  // bit n (and n + 16, n + 32, n + 48): row n of the tile is attended over
};

struct WaveArgs {
  const uint8_t* codes;
  const uint8_t* scales;
  int64_t cap;
  int64_t kv_row0;
};

__device__ __forceinline__ void wave_issue(WaveSlot& sl, const WaveArgs& a, int32_t id0, int32_t id1, int g) {
#pragma unroll
  for (int t = 0; t < 2; ++t) {
    const int32_t id = t ? id1 : id0;
    const bool ok = id >= 0 && id < a.cap;
    // A row that is not attended over reads row 0 of the sequence; its
    // scales are replaced by 0 where they are used.
    const int64_t row = a.kv_row0 + (ok ? id : 0);
    const gu32x4p cp = (gu32x4p)(a.codes + row * CSA2_CODE_BYTES + 64 * g);
#pragma unroll
    for (int i = 0; i < 4; ++i) sl.c[t][i] = cp[i];
    const uint64_t s8 = *(gu64p)(a.scales + row * CSA2_SCALE_BYTES + 8 * g);
    sl.s8[t] = make_uint2((uint32_t)s8, (uint32_t)(s8 >> 32));
    sl.ok[t] = __ballot(ok);
  }
}

// Sources of the next chunk's converted rows: tile t, channel group k (8
// channels of the lane's 128).
// No next chunk (the query's last).
struct WaveNoSrc {
  static constexpr bool kHas = false;
  __device__ __forceinline__ void issue(int) {}
  __device__ __forceinline__ u32x4 x(int, int) const { return u32x4{0u, 0u, 0u, 0u}; }
};

struct WaveFp4Src {
  static constexpr bool kHas = true;
  __device__ __forceinline__ void issue(int) {}
  const WaveSlot& sl;
  uint32_t sc[2][4];
  __device__ __forceinline__ WaveFp4Src(const WaveSlot& s, int n) : sl(s) {
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      const bool ok = (s.ok[t] >> n) & 1;
      scales_f16(ok ? s.s8[t].x : 0u, ok ? s.s8[t].y : 0u, sc[t]);
    }
  }
  __device__ __forceinline__ u32x4 x(int t, int k) const {
    return dequant8_f16(sl.c[t][k >> 2][k & 3], scale_pair(sc[t], k));
  }
};

// Window rows are read straight from memory (the L2, mostly): each channel
// group's loads are issued kWinLead groups ahead of its use.
constexpr int kWinLead = 3;

template <int kWin>
struct WaveWinSrc {
  static constexpr bool kHas = true;
  gu32x4p p[2];  // the lane's 128 channels of its row in each tile (or of the zero row)
  u32x4 v[2][16];
  __device__ __forceinline__ void issue(int k) {
    if (k < 16) {
      v[0][k] = p[0][k];
      v[1][k] = p[1][k];
    }
  }
  __device__ __forceinline__ u32x4 x(int t, int k) const { return kWin == kWinF16 ? v[t][k] : bf16x8_to_f16x8(v[t][k]); }
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
__device__ __forceinline__ bool wave_softmax(WaveState& st, const f32x4 (&s)[2], const uint64_t (&ok)[2],
                                             float scale_log2, int g, bool fixed, u32x4& hi, u32x4& lo) {
  float z[8];
  const float m = wave_scores(s, ok, scale_log2, g, z);
  // (Uniform selects, no branch: the step stays one block.)  The first
  // chunk with a row sets the reference (O and l are still 0).
  const bool above = !fixed && __ballot(m > st.m_run + kLazyLog2) != 0;
  const bool unset = __ballot(st.m_run != kNegInf) == 0;
  st.m_run = (above && unset) ? m : st.m_run;
  float p[8];
  float lsum = 0.f;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    p[i] = (z[i] == kNegInf) ? 0.f : __builtin_amdgcn_exp2f(z[i] - st.m_run);
    lsum += p[i];
  }
  st.l_run += fold32_add(fold16_add(lsum));
  // P = hi + lo in f16 (toward zero; p - hi is exact in binary32).
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const f16x2 h = __builtin_bit_cast(f16x2, __builtin_amdgcn_cvt_pkrtz(p[2 * i], p[2 * i + 1]));
    const f16x2 l = __builtin_bit_cast(f16x2, __builtin_amdgcn_cvt_pkrtz(p[2 * i] - (float)h[0], p[2 * i + 1] - (float)h[1]));
    hi[i] = __builtin_bit_cast(uint32_t, h);
    lo[i] = __builtin_bit_cast(uint32_t, l);
  }
  return !(above && !unset);
}

typedef short wave_v4s __attribute__((ext_vector_type(4)));

// The B operands of the P X blocks kk + 8i (i = 0..3): X[rows 4g..4g+3 of
// each tile][channel 16b + n].  Lane n of group g addresses row 4g + n/4,
// channels 16b + 4(n%4)..+3, and receives channel 16b + n of rows
// 4g..4g+3 (ds_read_b64_tr_b16).
struct WaveBGroup {
  wave_v4s t[4][2];
};

__device__ __forceinline__ WaveBGroup wave_read_group(const uint16_t* xs, int kk, int n, int g) {
  WaveBGroup r;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const uint16_t* a0 = &xs[(4 * g + (n >> 2)) * kWPitch + 16 * (kk + 8 * i) + 4 * (n & 3)];
#pragma unroll
    for (int t = 0; t < 2; ++t)
      r.t[i][t] = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
          (__attribute__((address_space(3))) wave_v4s*)(a0 + 16 * t * kWPitch));
  }
  return r;
}

// O += P X for the current chunk (rows 0..31 of the LDS tile xs), and the
// next chunk from src.  Channel group k of the next chunk (channels
// 128g + 8k.. of each lane, both tiles) is stored once the P X blocks that
// read those LDS columns (blocks k/2 + 8i: channels 16b..16b+15) have been
// read, and multiplied by Q into s_next; the reads of each group of blocks
// are issued one group ahead of their products.
template <class Src>
__device__ __forceinline__ void wave_pv_next(WaveState& st, uint16_t* xs, u32x4 hi, u32x4 lo, const u32x4 (&qv)[16],
                                             Src&& src, f32x4 (&s_next)[2], int n, int g) {
  // S^T of the next chunk in two partial sums per tile (even and odd
  // channel groups), so that consecutive products do not wait on each
  // other; added at the end.
  f32x4 s_odd[2] = {{0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}};
#pragma unroll
  for (int k = 0; k < 2 * kWinLead; ++k) src.issue(k);
  WaveBGroup cur = wave_read_group(xs, 0, n, g);
#pragma unroll
  for (int kk = 0; kk < 8; ++kk) {
    WaveBGroup nxt;
    if (kk < 7) nxt = wave_read_group(xs, kk + 1, n, g);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int b = kk + 8 * i;
      const uint2 u0 = __builtin_bit_cast(uint2, cur.t[i][0]), u1 = __builtin_bit_cast(uint2, cur.t[i][1]);
      const f16x8 bx = as_f16x8(u32x4{u0.x, u0.y, u1.x, u1.y});
      st.o[b] = mfma16x16x32_f16(as_f16x8(hi), bx, st.o[b]);
      st.o[b] = mfma16x16x32_f16(as_f16x8(lo), bx, st.o[b]);
    }
    if constexpr (std::remove_reference_t<Src>::kHas) {
#pragma unroll
      for (int k = 2 * kk; k < 2 * kk + 2; ++k)
#pragma unroll
        for (int t = 0; t < 2; ++t) {
          const u32x4 x = src.x(t, k);
          *reinterpret_cast<u32x4*>(&xs[(16 * t + n) * kWPitch + 128 * g + 8 * k]) = x;
          if (k & 1)
            s_odd[t] = mfma16x16x32_f16(as_f16x8(x), as_f16x8(qv[k]), s_odd[t]);
          else
            s_next[t] = mfma16x16x32_f16(as_f16x8(x), as_f16x8(qv[k]), s_next[t]);
        }
      src.issue(2 * kk + 2 * kWinLead);
      src.issue(2 * kk + 2 * kWinLead + 1);
    }
    // Issue order within the group: the next group's LDS reads, then each
    // MFMA followed by a few VALU conversions (one wavefront per SIMD
    // issues in order: an MFMA waiting for the matrix unit holds back the
    // VALU work behind it), then the LDS stores.
    __builtin_amdgcn_sched_group_barrier(0x100, 8, 0);
#pragma unroll
    for (int i = 0; i < 12; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x002, kValuPerMfma, 0);
    }
    __builtin_amdgcn_sched_group_barrier(0x200, 4, 0);
    __builtin_amdgcn_sched_barrier(0);
    if (kk < 7) cur = nxt;
  }
  if constexpr (std::remove_reference_t<Src>::kHas) {
    s_next[0] += s_odd[0];
    s_next[1] += s_odd[1];
  }
}

template <int kWin>
__global__ __launch_bounds__(64) void attn_wave_kernel(
    const uint16_t* __restrict__ q, const uint8_t* __restrict__ codes, const uint8_t* __restrict__ scales,
    int64_t cap, int32_t q_per_seq, const int32_t* __restrict__ idx, int32_t k_idx,
    const uint8_t* __restrict__ swa, int64_t swa_q_stride_rows, const int32_t* __restrict__ swa_len,
    int32_t swa_max, float scale_log2, float* __restrict__ out) {
  __shared__ __attribute__((aligned(16))) uint16_t xs[32 * kWPitch];
  __shared__ int32_t ids_s[kWaveMaxIdx];
  const int lane = threadIdx.x, n = lane & 15, g = lane >> 4;
  // XCD x (linear workgroup id mod 8) takes a contiguous run of queries,
  // whose windows overlap in its L2.
  const int nq = gridDim.x, per = nq / 8, rem = nq % 8;
  const int xcd = blockIdx.x % 8;
  const int qb = xcd * per + min(xcd, rem) + blockIdx.x / 8;

  WaveArgs a;
  a.codes = codes;
  a.scales = scales;
  a.cap = cap;
  a.kv_row0 = (int64_t)(qb / q_per_seq) * cap;
  const int32_t* qidx = idx + (int64_t)qb * k_idx;
  // The query's row ids, staged in LDS once (-1 past k_idx up to a whole
  // chunk), so that the ring's refills take them from there: no vector
  // memory load in the loop but the rows themselves.
  const int n_fc = (k_idx + 31) / 32;  // chunks of selected rows
  {
    // All loads first (clamped addresses), then the stores.
    int32_t v[kWaveMaxIdx / 64];
#pragma unroll
    for (int i = 0; i < kWaveMaxIdx / 64; ++i) v[i] = k_idx > 0 ? qidx[min(64 * i + lane, k_idx - 1)] : -1;
#pragma unroll
    for (int i = 0; i < kWaveMaxIdx / 64; ++i) ids_s[64 * i + lane] = 64 * i + lane < k_idx ? v[i] : -1;
  }
  __builtin_amdgcn_s_waitcnt(0xc07f);  // (lgkmcnt 0: the LDS stores above are done)
  __builtin_amdgcn_wave_barrier();
  // Row n of tile t of chunk c.
  auto id_of = [&](int c, int t) -> int32_t { return c < n_fc ? ids_s[32 * c + 16 * t + n] : -1; };

  const int n_swa = min(swa_len[qb], swa_max);
  const int n_wc = (n_swa + 31) / 32;  // chunks of window rows
  constexpr int kWinRowBytes = 2 * CSA2_LATENT;
  auto win_src = [&](int w) -> WaveWinSrc<kWin> {
    WaveWinSrc<kWin> src;
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      const int j = 32 * w + 16 * t + n;
      const uint8_t* row = j < n_swa ? swa + ((int64_t)qb * swa_q_stride_rows + j) * kWinRowBytes
                                     : reinterpret_cast<const uint8_t*>(kWaveZeroRow);
      src.p[t] = (gu32x4p)(row + (kWinRowBytes / 4) * g);
    }
    return src;
  };
  auto win_ok = [&](int w, uint64_t (&ok)[2]) {
    ok[0] = __ballot(32 * w + n < n_swa);
    ok[1] = __ballot(32 * w + 16 + n < n_swa);
  };

  // Main Q as f16 (the B operand of S): head n, channels 128g..128g+127.
  u32x4 qv[16];
  {
    const u32x4* qp = reinterpret_cast<const u32x4*>(q + ((int64_t)qb * 16 + n) * CSA2_LATENT + 128 * g);
#pragma unroll
    for (int i = 0; i < 16; ++i) qv[i] = qp[i];
#pragma unroll
    for (int i = 0; i < 16; ++i) qv[i] = bf16x8_to_f16x8(qv[i]);
  }

  // A pass with the lazily set reference maximum; if some chunk exceeds it
  // by more than kLazyLog2 the query is attended again against its exact
  // maximum (a pass of S alone finds it).
  bool fixed = false;
  float m_fix = kNegInf;
  WaveState st;
attend:
#pragma unroll
  for (int b = 0; b < 32; ++b) st.o[b] = f32x4{0.f, 0.f, 0.f, 0.f};
  st.m_run = m_fix;
  st.l_run = 0.f;
  {
    WaveSlot ring;
    wave_issue(ring, a, id_of(0, 0), id_of(0, 1), g);

    // The first chunk: converted, stored and multiplied by Q.
    f32x4 s_cur[2] = {{0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}};
    uint64_t ok_cur[2] = {0, 0};
    auto first = [&](auto&& src) {
#pragma unroll
      for (int k = 0; k < 16; ++k) src.issue(k);
#pragma unroll
      for (int k = 0; k < 16; ++k)
#pragma unroll
        for (int t = 0; t < 2; ++t) {
          const u32x4 x = src.x(t, k);
          *reinterpret_cast<u32x4*>(&xs[(16 * t + n) * kWPitch + 128 * g + 8 * k]) = x;
          s_cur[t] = mfma16x16x32_f16(as_f16x8(x), as_f16x8(qv[k]), s_cur[t]);
        }
    };
    if (n_fc > 0) {
      first(WaveFp4Src(ring, n));
      ok_cur[0] = ring.ok[0];
      ok_cur[1] = ring.ok[1];
      wave_issue(ring, a, id_of(1, 0), id_of(1, 1), g);
    } else if (n_wc > 0) {
      first(win_src(0));
      win_ok(0, ok_cur);
    }

    // Selected rows: iteration c attends chunk c; the next chunk is in the
    // ring slot, which is then refilled with the chunk after it.  The only
    // exit besides the count (a reference maximum exceeded) follows the
    // refill, so that every path to the slot's use passes the loads issued
    // after it.
    bool bad = false;
#pragma unroll 1
    for (int c = 0; c + 1 < n_fc; ++c) {
      u32x4 hi, lo;
      bad |= !wave_softmax(st, s_cur, ok_cur, scale_log2, g, fixed, hi, lo);
      f32x4 s_next[2] = {{0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}};
      wave_pv_next(st, xs, hi, lo, qv, WaveFp4Src(ring, n), s_next, n, g);
      ok_cur[0] = ring.ok[0];
      ok_cur[1] = ring.ok[1];
      wave_issue(ring, a, id_of(c + 2, 0), id_of(c + 2, 1), g);
      s_cur[0] = s_next[0];
      s_cur[1] = s_next[1];
      if (bad) goto exceeded;
    }
    // The last chunk of selected rows, followed by the first window chunk
    // (if any).
    if (n_fc > 0 && n_wc > 0) {
      u32x4 hi, lo;
      const bool fits = wave_softmax(st, s_cur, ok_cur, scale_log2, g, fixed, hi, lo);
      f32x4 s_next[2] = {{0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}};
      wave_pv_next(st, xs, hi, lo, qv, win_src(0), s_next, n, g);
      win_ok(0, ok_cur);
      s_cur[0] = s_next[0];
      s_cur[1] = s_next[1];
      if (!fits) goto exceeded;
    }
    // Window chunks but the last: the current chunk is w.
#pragma unroll 1
    for (int w = 0; w + 1 < n_wc; ++w) {
      u32x4 hi, lo;
      const bool fits = wave_softmax(st, s_cur, ok_cur, scale_log2, g, fixed, hi, lo);
      f32x4 s_next[2] = {{0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}};
      wave_pv_next(st, xs, hi, lo, qv, win_src(w + 1), s_next, n, g);
      win_ok(w + 1, ok_cur);
      s_cur[0] = s_next[0];
      s_cur[1] = s_next[1];
      if (!fits) goto exceeded;
    }
    // The query's last chunk (selected or window), after the loops: straight
    // code, so that the loops keep one path each.
    if (n_fc > 0 || n_wc > 0) {
      u32x4 hi, lo;
      const bool fits = wave_softmax(st, s_cur, ok_cur, scale_log2, g, fixed, hi, lo);
      f32x4 s_next[2];
      wave_pv_next(st, xs, hi, lo, qv, WaveNoSrc{}, s_next, n, g);
      if (!fits) goto exceeded;
    }
  }

  {
    // out = O / l per head (0 for a head with nothing attended over).
    float inv[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const float l = __int_as_float(__builtin_amdgcn_ds_bpermute(4 * (4 * g + j), __float_as_int(st.l_run)));
      inv[j] = l > 0.f ? 1.f / l : 0.f;
    }
    float* po = out + ((int64_t)qb * 16 + 4 * g) * CSA2_LATENT + n;
#pragma unroll
    for (int b = 0; b < 32; ++b)
#pragma unroll
      for (int j = 0; j < 4; ++j) po[j * CSA2_LATENT + 16 * b] = st.o[b][j] * inv[j];
    return;
  }

exceeded:
  // The exact maximum of every head over all the query's rows (the same S
  // products as above, summed in channel order: an order that differs from
  // the main pass's moves a score by rounding only, which a reference
  // maximum tolerates), then the query again against it.
  {
    float m = kNegInf;
#pragma unroll 1
    for (int c = 0; c < n_fc; ++c) {
      WaveSlot sl;
      wave_issue(sl, a, id_of(c, 0), id_of(c, 1), g);
      const WaveFp4Src src(sl, n);
      f32x4 s[2] = {{0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}};
#pragma unroll
      for (int k = 0; k < 16; ++k)
#pragma unroll
        for (int t = 0; t < 2; ++t) s[t] = mfma16x16x32_f16(as_f16x8(src.x(t, k)), as_f16x8(qv[k]), s[t]);
      float z[8];
      m = fmaxf(m, wave_scores(s, sl.ok, scale_log2, g, z));
    }
#pragma unroll 1
    for (int w = 0; w < n_wc; ++w) {
      WaveWinSrc<kWin> src = win_src(w);
#pragma unroll
      for (int k = 0; k < 16; ++k) src.issue(k);
      uint64_t ok[2];
      win_ok(w, ok);
      f32x4 s[2] = {{0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}};
#pragma unroll
      for (int k = 0; k < 16; ++k)
#pragma unroll
        for (int t = 0; t < 2; ++t) s[t] = mfma16x16x32_f16(as_f16x8(src.x(t, k)), as_f16x8(qv[k]), s[t]);
      float z[8];
      m = fmaxf(m, wave_scores(s, ok, scale_log2, g, z));
    }
    m_fix = m;
    fixed = true;
  }
  goto attend;
}

}  // namespace

// Launch: one 64-thread workgroup per query.  win: kWinBf16 or kWinF16.
csa2_status attn_wave_launch(const uint16_t* q, int32_t n_q, const csa2_fp4_kv& kv, int32_t q_per_seq,
                             const int32_t* idx, int32_t k_idx, const uint8_t* swa, int win,
                             int64_t swa_q_stride_rows, const int32_t* swa_len, int32_t swa_max, float scale_log2,
                             float* out, hipStream_t stream) {
  CSA2_REQUIRE(k_idx <= kWaveMaxIdx && (win == kWinF16 || win == kWinBf16), CSA2_EINVAL,
               "attention (one wavefront per query): k_idx above 512 or an unsupported window type");
  if (win == kWinF16)
    hipLaunchKernelGGL(attn_wave_kernel<kWinF16>, dim3(n_q), dim3(64), 0, stream, q, kv.codes, kv.scales, kv.cap,
                       q_per_seq, idx, k_idx, swa, swa_q_stride_rows, swa_len, swa_max, scale_log2, out);
  else
    hipLaunchKernelGGL(attn_wave_kernel<kWinBf16>, dim3(n_q), dim3(64), 0, stream, q, kv.codes, kv.scales, kv.cap,
                       q_per_seq, idx, k_idx, swa, swa_q_stride_rows, swa_len, swa_max, scale_log2, out);
  return launch_status("csa2_sparse_attn");
}

}  // namespace csa2
