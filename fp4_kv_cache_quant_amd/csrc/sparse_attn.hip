// Steps (d) + (e): gather and dequantise the selected FP4 main-KV rows and
// attend over them together with the layer's bf16 sliding window.
//
// [P1 "Compressed Sparse Attention 2 (CSA2)"]: each layer attends with its
// own main Q over the selected positions; [P1 "Causal Encoder-Decoder: Half
// the Prefill"]: a 128-token window runs in every layer; [P3]: keys and
// values share one 512-d latent (K = V).  [P1 "FP4 KV, ..."]: rows are E2M1
// values with one E4M3 scale per 16 channels.
//
// Online softmax over chunks.  A query's attended rows (k_idx selected FP4
// rows and swa_max window rows, in tiles of 16) are cut into chunks of W
// tiles (W = wavefronts per workgroup: 8 when there are few queries, 2 when
// there are many, so that four workgroups share a CU), the window tiles
// spread evenly over the chunks.  A workgroup walks a run of chunks of one
// query; per chunk:
//   1. each wavefront owns one tile; lane (n = l%16, g = l/16) loads row n's
//      channels 128g..128g+127 (FP4: 64 code bytes + 8 scale bytes; SWA: 256
//      bytes of bf16) and converts them to f16 in registers: an FP4 pair is
//      one v_cvt_scalef32_pk_f16_fp4 (at scale 1: the exact E2M1 values)
//      and one packed f16 multiply by the E4M3 scale, which is exact (a
//      product of 2- and 4-bit significands inside the f16 normal range);
//      a bf16 window pair is widened and packed to f16 (round toward zero:
//      exact for |x| in [2^-14, 65504], larger magnitudes saturate), an
//      E4M3 window pair is one exact v_cvt_scalef32_pk_f16_fp8, and f16
//      window rows (converted once per layer for many queries) are used as
//      loaded;
//   2. S^T = X Q^T on v_mfma_f32_16x16x32_f16 (16 steps over 512 channels),
//      the converted registers being the A operand and the main Q (rounded
//      to f16 the same way) the B operand; the rows also go to LDS for the
//      second product;
//   3. softmax statistics per head against the running maximum (max, then
//      exp2 and sum); P is split into f16 hi + lo parts (P ~ hi + lo to
//      about 2^-21) so the PV product keeps fp32-level accuracy;
//   4. O = O * 2^(m_old - m_new) + P X: each wavefront owns 512/W channels
//      as column tiles of 16 channels whose B operands (8 rows x 16
//      channels) are two transposing LDS reads (ds_read_b64_tr_b16); the
//      next chunk's rows are loaded meanwhile.
// With one workgroup per query the normalised output is written directly;
// otherwise each workgroup writes its unnormalised O and (max, sum) per
// head and a second kernel merges them (log-sum-exp weights).  A rank's
// share of a context-parallel split (csa2_sparse_attn_partial) is the same
// computation left unnormalised: O and (max, sum) per head, the max in
// base-2 units; csa2_attn_merge combines the ranks' shares with the same
// log-sum-exp merge.
//
// Citation keys: [P1] "DeepSeek AI Released DeepSeek-V4.1-Flash with 1M
// Context, FP4 KV Cache, and Cross-Layer Attention Reuse"; [P3]
// "DeepSeek-V4.1 Flash: Pushing the Limits of KV Cache Compression".
#include <algorithm>
#include <mutex>
#include <string>

#include "attn_dev.hpp"
#include "common.hpp"

namespace csa2 {

constexpr int kXPitch = CSA2_LATENT + 8;       // LDS row pitch, f16 elements

// One window row of zeros (bf16 / f16 / E4M3 all read 0 from it): the
// address of every window row past a query's window.
__device__ __attribute__((aligned(16))) const uint32_t kZeroRow[2 * CSA2_LATENT / 4] = {};

inline int attn_tiles(int32_t k_idx, int32_t swa_max) { return (k_idx + 15) / 16 + (swa_max + 15) / 16; }
inline int attn_chunks(int32_t k_idx, int32_t swa_max, int waves) {
  return (attn_tiles(k_idx, swa_max) + waves - 1) / waves;
}

namespace {

// With 8 wavefronts (one workgroup per CU) main Q is staged once in LDS;
// with 2 wavefronts (four workgroups per CU) Q stays in registers.  Either
// way the next chunk's rows are loaded while the current one is computed.
template <int W>
struct AttnCfg {
  static constexpr bool kQLds = (W == 8);
  static constexpr int kRows = 16 * W;           // rows per chunk
  static constexpr int kPPitch = kRows + 8;      // P pitch, f16 elements
  static constexpr int kCT = 4 * (8 / W);        // column tiles per wavefront
  static constexpr int kSlices = 8 / W;          // 64-channel slices per wavefront
};

template <int W>
struct AttnSmem {
  uint16_t qs[AttnCfg<W>::kQLds ? 16 * kXPitch : 8];  // main Q, f16 [head][channel]
  uint16_t xs[AttnCfg<W>::kRows * kXPitch];            // the chunk's rows, f16 [row][channel]
  uint16_t ps[2][16 * AttnCfg<W>::kPPitch];            // P = hi + lo, f16 [head][row]
  float red_m[W][16];
  float red_l[W][16];
  float alpha[16];                                     // rescale of the running O per head
  float l_fin[16];                                     // final softmax denominator per head
};

// Running state of one workgroup over its chunks: O for 16 heads x this
// wavefront's 512/W channels (column tile c: channels 64*(S*wave + c/4) +
// 16*(c%4) + n, head 4g + j in element j), the running max of head n, and
// (threads 0..15) the running denominator of head tid.
template <int W>
struct AttnState {
  f32x4 o[AttnCfg<W>::kCT];
  float m_run;
  float l_run;
};

// One wavefront's tile of a chunk: which rows, and this lane's raw loads
// (FP4: 4 x 16 code bytes in raw[0..3] + 8 scale bytes; window: 16 x 16
// bytes of bf16).
struct AttnTile {
  u32x4 raw[16];
  uint2 s8;
  uint8_t* dst;  // window slot that receives the step's new row (read from elsewhere), or null
  int32_t id;
  int row0;
  bool swa, in_range, ok;
};

struct AttnArgs {
  int qb;  // the query this workgroup attends for
  const uint8_t* codes;
  const uint8_t* scales;
  int64_t cap;
  int64_t kv_row0;  // first row of the query's cache sequence (qb / q_per_seq) * cap
  int32_t q_per_seq;
  const int32_t* idx;
  int32_t k_idx;
  const uint8_t* swa;  // window rows: bf16 (1,024 B) or E4M3 (512 B) per row
  int64_t swa_q_stride_rows;
  int32_t n_swa;
  const uint8_t* new_win;  // the step's new window row of this query's sequence, or null
  int32_t slot;            // its window slot, (lens - 1) % swa_max (-1: none)
  int n_tiles, swa_tiles;
};

// Which tile wavefront `wave` owns in chunk ch: FP4 tiles of 16 selected rows
// and window tiles of 16 rows, the window tiles spread evenly over the
// chunks so that every chunk moves about the same bytes.  For an FP4 tile
// the lane's row id is loaded (the first, dependent load).
template <int W>
__device__ __forceinline__ void tile_begin(AttnTile& t, const AttnArgs& a, int ch, int wave, int n) {
  const int tile = ch * W + wave;
  const int swa_before = (tile * a.swa_tiles) / a.n_tiles;  // < 2^20: 32-bit
  t.in_range = tile < a.n_tiles;
  t.swa = t.in_range && ((tile + 1) * a.swa_tiles) / a.n_tiles > swa_before;
  t.row0 = t.swa ? swa_before * 16 : (tile - swa_before) * 16;
  t.id = -1;
  if (!t.swa) {
    const int r = t.row0 + n;
    t.id = (t.in_range && r < a.k_idx) ? a.idx[(int64_t)a.qb * a.k_idx + r] : -1;
  }
}

// The row loads of a tile (unconditional, clamped addresses: all in flight
// together).  Window rows are bf16 (16 loads of 16 bytes per lane) or, with
// kWin == kWinE4m3, E4M3 bytes (8 loads).
template <int kWin>
__device__ __forceinline__ void tile_load(AttnTile& t, const AttnArgs& a, int n, int g) {
  const int qb = a.qb;
  if (!t.swa) {
    t.ok = t.id >= 0 && t.id < a.cap;
    const int64_t row = a.kv_row0 + (t.ok ? t.id : 0);
    const u32x4* cp = reinterpret_cast<const u32x4*>(a.codes + row * CSA2_CODE_BYTES + 64 * g);
#pragma unroll
    for (int i = 0; i < 4; ++i) t.raw[i] = cp[i];
    // (A row that is not attended over reads a clamped address; its scales
    // are taken as 0 where they are used, not here, so that this load does
    // not have to complete before the next ones are issued.)
    t.s8 = *reinterpret_cast<const uint2*>(a.scales + row * CSA2_SCALE_BYTES + 8 * g);
  } else {
    const int j = t.row0 + n;
    t.ok = t.in_range && j < a.n_swa;
    constexpr int kRowBytes = kWin == kWinE4m3 ? CSA2_LATENT : 2 * CSA2_LATENT;
    // A row past the window reads the zero row instead (its values then
    // convert to 0 and need no masking).  The slot of the step's token reads
    // the new row, which the chunk then stores into that slot.
    const uint8_t* ring = a.swa + ((int64_t)qb * a.swa_q_stride_rows + j) * kRowBytes;
    const bool fresh = t.ok && j == a.slot;
    t.dst = fresh ? const_cast<uint8_t*>(ring) + (kRowBytes / 4) * g : nullptr;
    const uint8_t* row = fresh ? a.new_win : t.ok ? ring : reinterpret_cast<const uint8_t*>(kZeroRow);
    const u32x4* sp = reinterpret_cast<const u32x4*>(row + (kRowBytes / 4) * g);
#pragma unroll
    for (int i = 0; i < (kWin == kWinE4m3 ? 8 : 16); ++i) t.raw[i] = sp[i];
  }
}

// Compute one chunk from the loaded tile (`between` runs after the softmax
// statistics, before the PV product: the next chunk's loads go there).
template <int W, int kWin, typename QB, typename Between>
__device__ __forceinline__ void attn_chunk(AttnSmem<W>& sm, AttnState<W>& st, const AttnTile& t,
                                           const QB& qb_operand, float scale_log2, Between between) {
  constexpr int kRows = AttnCfg<W>::kRows, kPPitch = AttnCfg<W>::kPPitch, kSlices = AttnCfg<W>::kSlices;
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int n = lane & 15, g = lane >> 4;
  const int row_local = wave * 16 + n;

  // ---- dequantise, stage in LDS, and S^T[row][head] on MFMA
  f32x4 s = {0.f, 0.f, 0.f, 0.f};
  if (!t.swa) {
    // The lane's 8 scale bytes as f16 (exact E4M3 conversions, two per
    // instruction): sc[i] holds scale bytes 2i (low half) and 2i + 1.
    // A row that is not attended over dequantises to zeros: scales 0.
    const uint32_t s8x = t.ok ? t.s8.x : 0u, s8y = t.ok ? t.s8.y : 0u;
    uint32_t sc[4];
    sc[0] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(s8x, 1.0f, false));
    sc[1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(s8x, 1.0f, true));
    sc[2] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(s8y, 1.0f, false));
    sc[3] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(s8y, 1.0f, true));
#pragma unroll
    for (int k = 0; k < 16; ++k) {
      // Channels 8k .. 8k+7 of the lane's 128 use scale byte k / 2, splat
      // into both halves.
      const uint32_t w = sc[k >> 2];
      const f16x2 s2 = __builtin_bit_cast(f16x2, ((k >> 1) & 1) ? byte_perm(w, w, 0x03020302u)
                                                                 : byte_perm(w, w, 0x01000100u));
      const u32x4 x = dequant8_f16(t.raw[k >> 2][k & 3], s2);
      *reinterpret_cast<u32x4*>(&sm.xs[row_local * kXPitch + 128 * g + 8 * k]) = x;
      s = mfma16x16x32_f16(as_f16x8(x), as_f16x8(qb_operand(k)), s);
    }
  } else {
    // (Rows past the window were loaded from the zero row.)  The step's new
    // window row joins the ring here: the lanes that hold it store it.
    if (t.dst) {
      u32x4* d = reinterpret_cast<u32x4*>(t.dst);
#pragma unroll
      for (int i = 0; i < (kWin == kWinE4m3 ? 8 : 16); ++i) d[i] = t.raw[i];
    }
#pragma unroll
    for (int k = 0; k < 16; ++k) {
      const u32x4 x = kWin == kWinE4m3 ? fp8x8_to_f16x8(t.raw[k >> 1][2 * (k & 1)], t.raw[k >> 1][2 * (k & 1) + 1])
                                       : bf16x8_to_f16x8(t.raw[k]);
      *reinterpret_cast<u32x4*>(&sm.xs[row_local * kXPitch + 128 * g + 8 * k]) = x;
      s = mfma16x16x32_f16(as_f16x8(x), as_f16x8(qb_operand(k)), s);
    }
  }
  const uint64_t rows_ok = __ballot(t.ok);  // bit n (lanes 0..15) = row n of this wavefront
  float z[4];
  const uint32_t ok4 = (uint32_t)(rows_ok >> (4 * g));
#pragma unroll
  for (int j = 0; j < 4; ++j) z[j] = ((ok4 >> j) & 1) ? s[j] * scale_log2 : kNegInf;

  // ---- softmax statistics of the chunk, per head n, against the running
  // max (online softmax across the workgroup's chunks)
  float m = fmaxf(fmaxf(z[0], z[1]), fmaxf(z[2], z[3]));
  m = fold32_max(fold16_max(m));
  if (g == 0) sm.red_m[wave][n] = m;
  lds_barrier();
  float M = st.m_run;
#pragma unroll
  for (int w = 0; w < W; ++w) M = fmaxf(M, sm.red_m[w][n]);
  float p[4];
  float lsum = 0.f;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    p[j] = (z[j] == kNegInf) ? 0.f : __builtin_amdgcn_exp2f(z[j] - M);
    lsum += p[j];
  }
  {
    // P = hi + lo in f16 (toward zero; p - hi is exact in binary32).
    const f16x2 h01 = __builtin_bit_cast(f16x2, __builtin_amdgcn_cvt_pkrtz(p[0], p[1]));
    const f16x2 h23 = __builtin_bit_cast(f16x2, __builtin_amdgcn_cvt_pkrtz(p[2], p[3]));
    const f16x2 l01 = __builtin_bit_cast(f16x2, __builtin_amdgcn_cvt_pkrtz(p[0] - (float)h01[0], p[1] - (float)h01[1]));
    const f16x2 l23 = __builtin_bit_cast(f16x2, __builtin_amdgcn_cvt_pkrtz(p[2] - (float)h23[0], p[3] - (float)h23[1]));
    const int o = n * kPPitch + wave * 16 + 4 * g;
    *reinterpret_cast<uint2*>(&sm.ps[0][o]) = uint2{__builtin_bit_cast(uint32_t, h01), __builtin_bit_cast(uint32_t, h23)};
    *reinterpret_cast<uint2*>(&sm.ps[1][o]) = uint2{__builtin_bit_cast(uint32_t, l01), __builtin_bit_cast(uint32_t, l23)};
  }
  lsum = fold32_add(fold16_add(lsum));
  if (g == 0) sm.red_l[wave][n] = lsum;
  const float alpha_n = (st.m_run == kNegInf) ? 0.f : __builtin_amdgcn_exp2f(st.m_run - M);
  if (tid < 16) sm.alpha[tid] = alpha_n;
  st.m_run = M;
  lds_barrier();
  between();

  // ---- O = O * alpha + P X for this wavefront's channel slices (on the
  // first chunk O = 0 and alpha = 0: no special case, so that the chunk
  // loop is not peeled)
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const float a = sm.alpha[4 * g + j];
#pragma unroll
    for (int c = 0; c < AttnCfg<W>::kCT; ++c) st.o[c][j] *= a;
  }
  if (tid < 16) {
    float l = 0.f;
#pragma unroll
    for (int w = 0; w < W; ++w) l += sm.red_l[w][tid];
    st.l_run = st.l_run * alpha_n + l;
  }
#pragma unroll
  for (int ks = 0; ks < kRows / 32; ++ks) {
    const f16x8 ph = as_f16x8(*reinterpret_cast<const u32x4*>(&sm.ps[0][n * kPPitch + 32 * ks + 8 * g]));
    const f16x8 pl = as_f16x8(*reinterpret_cast<const u32x4*>(&sm.ps[1][n * kPPitch + 32 * ks + 8 * g]));
#pragma unroll
    for (int sl = 0; sl < kSlices; ++sl) {
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        // B = X[rows 32ks + 8g .. +7][channels ch .. ch+15] by two transposing
        // LDS reads (ds_read_b64_tr_b16): within each 16-lane group, lane i
        // receives element i%4 of the 4-channel pieces addressed by lanes
        // 4e + i/4 (e = 0..3), so lane n addresses row 4h + n/4 of the
        // half, channels ch + 4(n%4) .. +3, and receives channel ch + n of
        // rows 4h .. 4h+3.
        const int ch = 64 * (kSlices * wave + sl) + 16 * c;
        const int r0 = 32 * ks + 8 * g + (n >> 2);
        const uint16_t* a0 = &sm.xs[r0 * kXPitch + ch + 4 * (n & 3)];
        typedef short v4s __attribute__((ext_vector_type(4)));
        const v4s lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (__attribute__((address_space(3))) v4s*)(a0));
        const v4s hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (__attribute__((address_space(3))) v4s*)(a0 + 4 * kXPitch));
        const uint2 l2 = __builtin_bit_cast(uint2, lo), h2 = __builtin_bit_cast(uint2, hi);
        const f16x8 bc = as_f16x8(u32x4{l2.x, l2.y, h2.x, h2.y});
        st.o[4 * sl + c] = mfma16x16x32_f16(ph, bc, st.o[4 * sl + c]);
        st.o[4 * sl + c] = mfma16x16x32_f16(pl, bc, st.o[4 * sl + c]);
      }
    }
  }
}

// One workgroup = chunks [split * per_split, ...) of query blockIdx.y.  With
// one split and an output the workgroup covers the whole query and writes
// the normalised output; otherwise (several splits, or out == null for a
// rank's share) it writes its unnormalised O and (max, sum) per head to
// part_o / part_ml.
template <int W, int kWin>
__global__ __launch_bounds__(64 * W, 8 / W) void attn_kernel(
    const uint16_t* __restrict__ q, const uint8_t* __restrict__ codes,
    const uint8_t* __restrict__ scales, int64_t cap, int32_t q_per_seq,
    const int32_t* __restrict__ idx, int32_t k_idx, const uint8_t* swa, int64_t swa_q_stride_rows,
    const int32_t* __restrict__ swa_len, int32_t swa_max, const uint8_t* __restrict__ new_win,
    const int32_t* __restrict__ win_lens, float scale_log2, int32_t per_split, float* __restrict__ part_o,
    float2* __restrict__ part_ml, int32_t n_split, float* __restrict__ out) {
  using Cfg = AttnCfg<W>;
  __shared__ __attribute__((aligned(16))) AttnSmem<W> sm;
  constexpr int kSlices = Cfg::kSlices;
  const int split = blockIdx.x;
  const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int n = lane & 15, g = lane >> 4;
  // Workgroups are dealt to the 8 XCDs round-robin (linear id mod 8).  With
  // one workgroup per query, XCD x takes a contiguous run of queries, so
  // that neighbouring queries -- whose windows overlap in all but one row
  // when they are consecutive tokens -- share that XCD's L2.
  int qb = blockIdx.y;
  if (gridDim.x == 1) {
    const int nq = gridDim.y, per = nq / 8, rem = nq % 8;
    const int x = blockIdx.y % 8, i = blockIdx.y / 8;
    qb = x * per + min(x, rem) + i;
  }

  // Main Q: loaded first so that its loads overlap the index and row loads.
  // Registers: lane (n, g) holds head n, channels 128g..128g+127 (the B
  // operand of S).  LDS: 16-byte pieces spread over the workgroup.
  constexpr int kQPer = Cfg::kQLds ? 1024 / (64 * W) : 16;
  u32x4 qv[kQPer];
  if (Cfg::kQLds) {
    const u32x4* qp = reinterpret_cast<const u32x4*>(q + (int64_t)qb * 16 * CSA2_LATENT);
#pragma unroll
    for (int i = 0; i < kQPer; ++i) qv[i] = qp[tid + 64 * W * i];
  } else {
    const u32x4* qp = reinterpret_cast<const u32x4*>(q + ((int64_t)qb * 16 + n) * CSA2_LATENT + 128 * g);
#pragma unroll
    for (int i = 0; i < kQPer; ++i) qv[i] = qp[i];
#pragma unroll
    for (int i = 0; i < kQPer; ++i) qv[i] = bf16x8_to_f16x8(qv[i]);
  }

  AttnArgs a;
  a.qb = qb;
  a.codes = codes;
  a.scales = scales;
  a.cap = cap;
  a.kv_row0 = (int64_t)(qb / q_per_seq) * cap;
  a.q_per_seq = q_per_seq;
  a.idx = idx;
  a.k_idx = k_idx;
  a.swa = swa;
  a.swa_q_stride_rows = swa_q_stride_rows;
  a.n_swa = min(swa_len[qb], swa_max);
  constexpr int kWinRowBytes = kWin == kWinE4m3 ? CSA2_LATENT : 2 * CSA2_LATENT;
  a.new_win = new_win ? new_win + (int64_t)(qb / q_per_seq) * kWinRowBytes : nullptr;
  a.slot = new_win ? (win_lens[qb / q_per_seq] - 1) % max(swa_max, 1) : -1;
  a.swa_tiles = (swa_max + 15) / 16;
  a.n_tiles = (k_idx + 15) / 16 + a.swa_tiles;
  const int n_chunks = (a.n_tiles + W - 1) / W;
  const int c_begin = split * per_split, c_end = min(n_chunks, c_begin + per_split);

  AttnTile cur;
  tile_begin<W>(cur, a, c_begin, wave, n);
  tile_load<kWin>(cur, a, n, g);
  if (Cfg::kQLds) {
#pragma unroll
    for (int i = 0; i < kQPer; ++i) {
      const int c = tid + 64 * W * i;
      *reinterpret_cast<u32x4*>(&sm.qs[(c >> 6) * kXPitch + 8 * (c & 63)]) = bf16x8_to_f16x8(qv[i]);
    }
    lds_barrier();
  }
  auto qb_operand = [&](int k) -> u32x4 {
    if (Cfg::kQLds) return *reinterpret_cast<const u32x4*>(&sm.qs[n * kXPitch + 128 * g + 8 * k]);
    return qv[k & (kQPer - 1)];
  };

  AttnState<W> st;
#pragma unroll
  for (int c = 0; c < Cfg::kCT; ++c) st.o[c] = f32x4{0.f, 0.f, 0.f, 0.f};
  st.m_run = kNegInf;
  st.l_run = 0.f;
#pragma unroll 1
  for (int ch = c_begin; ch < c_end; ++ch) {
    const bool has_next = ch + 1 < c_end;
    if (ch != c_begin) lds_barrier();  // the previous chunk's LDS reads are done
    AttnTile nxt;
    if (has_next) tile_begin<W>(nxt, a, ch + 1, wave, n);  // index loads of the next chunk
    attn_chunk<W, kWin>(sm, st, cur, qb_operand, scale_log2, [&]() {
      if (has_next) tile_load<kWin>(nxt, a, n, g);  // its row loads overlap this chunk's PV
    });
    if (has_next) cur = nxt;
  }

  if (n_split == 1 && out) {
    if (tid < 16) sm.l_fin[tid] = st.l_run;
    lds_barrier();
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int head = 4 * g + j;
      const float l = sm.l_fin[head];
      const float inv = l > 0.f ? 1.f / l : 0.f;
#pragma unroll
      for (int sl = 0; sl < kSlices; ++sl)
#pragma unroll
        for (int c = 0; c < 4; ++c)
          out[((int64_t)qb * 16 + head) * CSA2_LATENT + 64 * (kSlices * wave + sl) + 16 * c + n] =
              st.o[4 * sl + c][j] * inv;
    }
    return;
  }
  float* po = part_o + ((int64_t)qb * n_split + split) * (16 * CSA2_LATENT);
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int head = 4 * g + j;
#pragma unroll
    for (int sl = 0; sl < kSlices; ++sl)
#pragma unroll
      for (int c = 0; c < 4; ++c) po[head * CSA2_LATENT + 64 * (kSlices * wave + sl) + 16 * c + n] = st.o[4 * sl + c][j];
  }
  if (tid < 16) part_ml[((int64_t)qb * n_split + split) * 16 + tid] = make_float2(st.m_run, st.l_run);
}

// Merge n_parts partials of one (head, query) with log-sum-exp weights:
//   o_h = sum_c 2^(m_c - M) O_c / sum_c 2^(m_c - M) l_c,  M = max_c m_c.
// One 128-thread workgroup per (head, query), one float4 of the head's 512
// channels per thread; partial c of query q is at part_o + q * o_q +
// c * o_c (floats) and part_ml + q * ml_q + c * ml_c (float2 per head).  The
// partials are taken in batches of 16 whose loads (partial O and (m, l),
// clamped addresses) are all issued together; a running maximum rescales
// across batches.  kNorm: the normalised output; otherwise the merged
// unnormalised O and (M, sum of 2^(m_c - M) l_c) per head in out_ml.
template <bool kNorm>
__global__ __launch_bounds__(128) void attn_combine_kernel(const float* __restrict__ part_o,
                                                           const float2* __restrict__ part_ml, int32_t n_split,
                                                           int64_t o_q, int64_t o_c, int64_t ml_q, int64_t ml_c,
                                                           float* __restrict__ out, float2* __restrict__ out_ml) {
  const int h = blockIdx.x, qb = blockIdx.y, tid = threadIdx.x;
  const float2* ml = part_ml + (int64_t)qb * ml_q + h;
  const f32x4* pall = reinterpret_cast<const f32x4*>(part_o + (int64_t)qb * o_q + h * CSA2_LATENT) + tid;
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  float den = 0.f, Mq = kNegInf;
  constexpr int kB = 16;
  for (int c0 = 0; c0 < n_split; c0 += kB) {
    f32x4 v[kB];
    float2 m[kB];
#pragma unroll
    for (int cb = 0; cb < kB; ++cb) {
      const int c = min(c0 + cb, n_split - 1);
      v[cb] = pall[(int64_t)c * (o_c / 4)];
      m[cb] = ml[(int64_t)c * ml_c];
    }
    float Mb = Mq;
#pragma unroll
    for (int cb = 0; cb < kB; ++cb) Mb = fmaxf(Mb, m[cb].x);
    const float r = (Mq == kNegInf) ? 0.f : exp2f(Mq - Mb);
    den *= r;
    acc *= r;
#pragma unroll
    for (int cb = 0; cb < kB; ++cb) {
      const float e = (c0 + cb >= n_split || m[cb].x == kNegInf) ? 0.f : exp2f(m[cb].x - Mb);
      den += e * m[cb].y;
      acc += e * v[cb];
    }
    Mq = Mb;
  }
  f32x4* o4 = reinterpret_cast<f32x4*>(out + ((int64_t)qb * 16 + h) * CSA2_LATENT);
  if constexpr (kNorm) {
    const float inv = den > 0.f ? 1.f / den : 0.f;
    o4[tid] = acc * inv;
  } else {
    o4[tid] = acc;
    if (tid == 0) out_ml[(int64_t)qb * 16 + h] = make_float2(Mq, den);
  }
}

}  // namespace

// Launch shape: 8-wavefront workgroups (128-row chunks) split over the
// chunks of each query when there are few queries, so that the chip fills
// (a combine kernel merges the splits); 4-wavefront workgroups (64-row
// chunks, two per CU) covering a whole query each when there are many (no
// partials).
struct AttnPlan {
  int waves, splits, per_split;
};

static AttnPlan attn_plan(int32_t n_q, int32_t k_idx, int32_t swa_max) {
  AttnPlan p;
  if (n_q >= 1024) {
    p.waves = 2;
    p.per_split = attn_chunks(k_idx, swa_max, 2);
    p.splits = 1;
    return p;
  }
  p.waves = 8;
  const int n_chunks = attn_chunks(k_idx, swa_max, 8);
  const int want = std::max(1, std::min(n_chunks, (int)((1024 + (int64_t)n_q - 1) / std::max(1, n_q))));
  p.per_split = (n_chunks + want - 1) / want;
  p.splits = (n_chunks + p.per_split - 1) / p.per_split;
  return p;
}

size_t attn_workspace_bytes(int32_t n_q, int32_t k_idx, int32_t swa_max) {
  const AttnPlan p = attn_plan(n_q, k_idx, swa_max);
  if (p.splits == 1) return 0;
  const size_t o_bytes = (size_t)n_q * p.splits * 16 * CSA2_LATENT * sizeof(float);
  const size_t ml_bytes = (size_t)n_q * p.splits * 16 * sizeof(float2);
  return o_bytes + ml_bytes;
}

csa2_status attn_many_launch(const uint16_t* q, int32_t n_q, const csa2_fp4_kv& kv, int32_t q_per_seq,
                             const int32_t* idx, int32_t k_idx, const uint8_t* swa, int win,
                             int64_t swa_q_stride_rows, const int32_t* swa_len, int32_t swa_max, float scale_log2,
                             float* out, hipStream_t stream);

template <int kWin>
static void attn_dispatch(const AttnPlan& p, int32_t n_q, const uint16_t* q, const csa2_fp4_kv& kv,
                          int32_t q_per_seq, const int32_t* idx, int32_t k_idx, const uint8_t* swa,
                          int64_t swa_q_stride_rows, const int32_t* swa_len, int32_t swa_max,
                          const uint8_t* new_win, const int32_t* win_lens, float scale_log2, float* part_o,
                          float2* part_ml, float* out, hipStream_t stream) {
  if (p.waves == 8)
    hipLaunchKernelGGL((attn_kernel<8, kWin>), dim3(p.splits, n_q), dim3(64 * 8), 0, stream, q, kv.codes,
                       kv.scales, kv.cap, q_per_seq, idx, k_idx, swa, swa_q_stride_rows, swa_len, swa_max,
                       new_win, win_lens, scale_log2, p.per_split, part_o, part_ml, p.splits, out);
  else
    hipLaunchKernelGGL((attn_kernel<2, kWin>), dim3(p.splits, n_q), dim3(64 * 2), 0, stream, q, kv.codes,
                       kv.scales, kv.cap, q_per_seq, idx, k_idx, swa, swa_q_stride_rows, swa_len, swa_max,
                       new_win, win_lens, scale_log2, p.per_split, part_o, part_ml, p.splits, out);
}

// win: the window rows' element type -- kWinBf16 (bf16 [*][512], converted
// to f16 toward zero in the kernel) or kWinE4m3 (E4M3 bytes [*][512]).
// new_win / win_lens: the step's new window row per sequence ([*][512] in
// the window's element type), or null, and the sequences' positions after
// the step's append: the new row goes to window slot (lens - 1) % swa_max.
// out_ml == null: the normalised output in out.  Otherwise a rank's share:
// the unnormalised O in out and (max in base-2 units, sum) per head in
// out_ml [n_q][16].
static csa2_status attn_launch_impl(const uint16_t* q, int32_t n_q, const csa2_fp4_kv& kv, int32_t q_per_seq,
                                    const int32_t* idx, int32_t k_idx, const void* swa, int win,
                                    int64_t swa_q_stride_rows, const int32_t* swa_len, int32_t swa_max,
                                    const void* new_win, const int32_t* win_lens, float sm_scale, float* out,
                                    float2* out_ml, void* ws, hipStream_t stream) {
  if (n_q == 0) return CSA2_OK;
  const AttnPlan p = attn_plan(n_q, k_idx, swa_max);
  float* part_o = nullptr;
  float2* part_ml = nullptr;
  if (p.splits > 1) {
    char* base = reinterpret_cast<char*>(ws);
    part_o = reinterpret_cast<float*>(base);
    base += (size_t)n_q * p.splits * 16 * CSA2_LATENT * sizeof(float);
    part_ml = reinterpret_cast<float2*>(base);
  }
  const float scale_log2 = sm_scale * 1.4426950408889634f;
  const uint8_t* sw = reinterpret_cast<const uint8_t*>(swa);
  const uint8_t* nw = reinterpret_cast<const uint8_t*>(new_win);
  // Many queries over bf16 window rows with no step window row (the
  // prefill chunk): the two-wavefronts-per-query kernel of attn_many.hip.
  float* kout = out;
  if (out_ml && p.splits == 1) {  // a share from one workgroup per query: written in place
    part_o = out;
    part_ml = out_ml;
    kout = nullptr;
  }
  if (p.waves == 2 && !new_win && !out_ml && k_idx <= kAttnManyMaxIdx && win == kWinBf16)
    return attn_many_launch(q, n_q, kv, q_per_seq, idx, k_idx, sw, win, swa_q_stride_rows, swa_len, swa_max,
                            scale_log2, out, stream);
  if (win == kWinE4m3)
    attn_dispatch<kWinE4m3>(p, n_q, q, kv, q_per_seq, idx, k_idx, sw, swa_q_stride_rows, swa_len, swa_max,
                            nw, win_lens, scale_log2, part_o, part_ml, kout, stream);
  else
    attn_dispatch<kWinBf16>(p, n_q, q, kv, q_per_seq, idx, k_idx, sw, swa_q_stride_rows, swa_len, swa_max,
                            nw, win_lens, scale_log2, part_o, part_ml, kout, stream);
  if (p.splits > 1) {
    const int64_t o_c = 16 * CSA2_LATENT, o_q = p.splits * o_c, ml_q = p.splits * 16;
    if (out_ml)
      hipLaunchKernelGGL(attn_combine_kernel<false>, dim3(16, n_q), dim3(128), 0, stream, part_o, part_ml,
                         p.splits, o_q, o_c, ml_q, (int64_t)16, out, out_ml);
    else
      hipLaunchKernelGGL(attn_combine_kernel<true>, dim3(16, n_q), dim3(128), 0, stream, part_o, part_ml,
                         p.splits, o_q, o_c, ml_q, (int64_t)16, out, nullptr);
  }
  return launch_status(out_ml ? "csa2_sparse_attn_partial" : "csa2_sparse_attn");
}

csa2_status attn_launch(const uint16_t* q, int32_t n_q, const csa2_fp4_kv& kv, int32_t q_per_seq,
                        const int32_t* idx, int32_t k_idx, const void* swa, int win,
                        int64_t swa_q_stride_rows, const int32_t* swa_len, int32_t swa_max, const void* new_win,
                        const int32_t* win_lens, float sm_scale, float* out, void* ws, hipStream_t stream) {
  return attn_launch_impl(q, n_q, kv, q_per_seq, idx, k_idx, swa, win, swa_q_stride_rows, swa_len, swa_max,
                          new_win, win_lens, sm_scale, out, nullptr, ws, stream);
}

// A rank's share (bf16 or E4M3 window rows, no step window row).
csa2_status attn_partial_launch(const uint16_t* q, int32_t n_q, const csa2_fp4_kv& kv, int32_t q_per_seq,
                                const int32_t* idx, int32_t k_idx, const void* swa, int win,
                                int64_t swa_q_stride_rows, const int32_t* swa_len, int32_t swa_max, float sm_scale,
                                float* out_o, float* out_ml, void* ws, hipStream_t stream) {
  return attn_launch_impl(q, n_q, kv, q_per_seq, idx, k_idx, swa, win, swa_q_stride_rows, swa_len, swa_max,
                          nullptr, nullptr, sm_scale, out_o, reinterpret_cast<float2*>(out_ml), ws, stream);
}

// The softmax over the union of n_parts shares: parts_o [n_parts][n_q][16][512],
// parts_ml [n_parts][n_q][16][2] -> out [n_q][16][512].
csa2_status attn_merge_launch(const float* parts_o, const float* parts_ml, int32_t n_parts, int32_t n_q, float* out,
                              hipStream_t stream) {
  if (n_q == 0) return CSA2_OK;
  const int64_t o_q = 16 * CSA2_LATENT, o_c = (int64_t)n_q * o_q;
  hipLaunchKernelGGL(attn_combine_kernel<true>, dim3(16, n_q), dim3(128), 0, stream, parts_o,
                     reinterpret_cast<const float2*>(parts_ml), n_parts, o_q, o_c, (int64_t)16, (int64_t)n_q * 16,
                     out, nullptr);
  return launch_status("csa2_attn_merge");
}

// ------------------------------------------------- static scratch
// For callers that cannot allocate: the split partials of
// csa2_sparse_attn_noalloc live in this file-scope array (one copy per GPU
// the library runs on, held until the process ends).  Host code never
// passes the array's name to a kernel -- on the host it is only a stand-in
// for the symbol -- but the device address that hipGetSymbolAddress returns
// for the current device, looked up once per device and kept.
constexpr size_t kAttnScratchBytes = size_t(16) << 20;
static __device__ __align__(256) uint8_t scratch[kAttnScratchBytes];

namespace {
std::mutex g_scratch_mu;
void* g_scratch_ptr[64] = {};
}  // namespace

csa2_status attn_scratch(void** ptr, size_t* bytes) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) {
    set_error("csa2_sparse_attn_noalloc: no current device (or device index >= 64)");
    return CSA2_EHIP;
  }
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p) {
      set_error(std::string("csa2_sparse_attn_noalloc: hipGetSymbolAddress: ") + hipGetErrorString(e));
      return CSA2_EHIP;
    }
    g_scratch_ptr[dev] = p;
  }
  *ptr = g_scratch_ptr[dev];
  *bytes = kAttnScratchBytes;
  return CSA2_OK;
}

}  // namespace csa2
