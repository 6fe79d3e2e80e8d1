// Steps (d) + (e): gather and dequantise the selected FP4 main-KV rows and
// attend over them together with the layer's bf16 sliding window.
//
// [P1 "Compressed Sparse Attention 2 (CSA2)"]: each layer attends with its
// own main Q over the selected positions; [P1 "Causal Encoder-Decoder: Half
// the Prefill"]: a 128-token window runs in every layer; [P3]: keys and
// values share one 512-d latent (K = V).  [P1 "FP4 KV, ..."]: rows are E2M1
// values with one E4M3 scale per 16 channels.
//
// Split-K with online softmax.  A query's attended rows (k_idx selected FP4
// rows and swa_max window rows, in tiles of 16) are cut into chunks of 8
// tiles, the window tiles spread evenly over the chunks; one 512-thread
// workgroup handles one chunk of one query:
//   1. each wavefront owns one tile; lane (n = l%16, g = l/16) loads row n's
//      channels 128g..128g+127 (FP4: 64 code bytes + 8 scale bytes; SWA: 256
//      bytes of bf16) and dequantises in registers (byte-table lookups for
//      the E2M1 magnitudes, one exact binary32 multiply by the E4M3 scale);
//   2. S^T = X Q^T on v_mfma_f32_16x16x32_bf16 (16 steps over 512 channels),
//      the dequantised registers being the A operand directly and the main Q
//      (staged once per workgroup in LDS) the B operand; the rows also go to
//      LDS for the second product;
//   3. softmax statistics per head over the chunk (max, then exp2 and sum);
//      P is split into bf16 hi + lo parts (P ~ hi + lo to 2^-16) so the PV
//      product keeps fp32-level accuracy on bf16 MFMA;
//   4. O = P X: wavefront w computes channels 64w..64w+63 as 4 column
//      tiles whose B operands come from 8-byte LDS reads of 8 rows, split
//      into per-column vectors;
//   5. the chunk writes its unnormalised O and (max, sum) per head.
// A second kernel merges the chunks of each query (log-sum-exp weights).
//
// Citation keys: [P1] "DeepSeek AI Released DeepSeek-V4.1-Flash with 1M
// Context, FP4 KV Cache, and Cross-Layer Attention Reuse"; [P3]
// "DeepSeek-V4.1 Flash: Pushing the Limits of KV Cache Compression".
#include <algorithm>

#include "common.hpp"

namespace csa2 {

constexpr int kAttnWaves = 8;                  // wavefronts per workgroup
constexpr int kAttnRows = 16 * kAttnWaves;     // rows per workgroup chunk (16 per wavefront)
constexpr int kXPitch = CSA2_LATENT + 8;       // LDS row pitch, bf16 elements
constexpr int kPPitch = kAttnRows + 8;         // LDS P pitch, bf16 elements
constexpr int kMaxSplits = 128;

inline int attn_tiles(int32_t k_idx, int32_t swa_max) { return (k_idx + 15) / 16 + (swa_max + 15) / 16; }
inline int attn_splits(int32_t k_idx, int32_t swa_max) {
  return (attn_tiles(k_idx, swa_max) + kAttnWaves - 1) / kAttnWaves;
}

namespace {

// Dequantise 8 channels -- code dword dw, channel i in nibble i -- with the
// binary32 scale s into 4 bf16 pairs.  The E2M1 magnitude indexes two 8-entry
// byte tables (high and low byte of its bf16 value) through v_perm_b32, the
// code's sign bit is ORed into the high byte, the bf16 is widened to binary32,
// multiplied by s (exact: at most 2 x 4 significant bits) and narrowed back by
// taking the upper half (exact for the same reason).
__device__ __forceinline__ u32x4 dequant8(uint32_t dw, float s) {
  constexpr uint32_t kHi03 = 0x3F3F3F00u, kHi47 = 0x40404040u;  // bf16 high bytes of m = 0..3 / 4..7
  constexpr uint32_t kLo03 = 0xC0800000u, kLo47 = 0xC0804000u;  // bf16 low bytes
  const uint32_t sel_e = dw & 0x07070707u;          // channels 0, 2, 4, 6
  const uint32_t sel_o = (dw >> 4) & 0x07070707u;   // channels 1, 3, 5, 7
  const uint32_t hi_e = byte_perm(kHi47, kHi03, sel_e) | ((dw & 0x08080808u) << 4);
  const uint32_t lo_e = byte_perm(kLo47, kLo03, sel_e);
  const uint32_t hi_o = byte_perm(kHi47, kHi03, sel_o) | (dw & 0x80808080u);
  const uint32_t lo_o = byte_perm(kLo47, kLo03, sel_o);
  u32x4 r;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const uint32_t widen = 0x0C0Cu | ((uint32_t)j << 16) | ((uint32_t)(4 + j) << 24);  // [0, 0, lo_j, hi_j]
    const float fe = __builtin_bit_cast(float, byte_perm(hi_e, lo_e, widen)) * s;
    const float fo = __builtin_bit_cast(float, byte_perm(hi_o, lo_o, widen)) * s;
    r[j] = byte_perm(__builtin_bit_cast(uint32_t, fo), __builtin_bit_cast(uint32_t, fe), 0x07060302u);
  }
  return r;
}

// E4M3FN scale byte as binary32 (sign, NaN for S.1111.111).
__device__ __forceinline__ float e4m3_value(uint32_t c) {
  const uint32_t mag = c & 0x7Fu;
  const float v = (mag == 0x7Fu) ? __builtin_nanf("") : e4m3_pos_value(mag);
  return (c & 0x80u) ? -v : v;
}

struct AttnSmem {
  uint16_t qs[16 * kXPitch];                // main Q, bf16 [head][channel]
  uint16_t xs[kAttnRows * kXPitch];         // the chunk's rows, bf16 [row][channel]
  uint16_t ps[2][16 * kPPitch];             // P = hi + lo, bf16 [head][row]
  float red_m[kAttnWaves][16];
  float red_l[kAttnWaves][16];
  float alpha[16];                          // rescale of the running O per head
  float l_fin[16];                          // final softmax denominator per head
};

// Running state of one workgroup over its chunks: O for 16 heads x this
// wavefront's 64 channels (column tile c = channels 64*wave + 4n + c, head
// 4g + j in element j), the running max of head n, and (threads 0..15) the
// running denominator of head tid.
struct AttnState {
  f32x4 o[4];
  float m_run;
  float l_run;
};

// One chunk of 8 tiles, the wavefront's tile specialised on its kind (FP4
// rows or window rows) so that its loads are unconditional and issued
// together; every wavefront runs the same barrier sequence.
template <bool kSwa>
__device__ __forceinline__ void attn_chunk(
    AttnSmem& sm, AttnState& st, bool first, const u32x4 (&qreg)[1024 / (64 * kAttnWaves)],
    const uint8_t* __restrict__ codes, const uint8_t* __restrict__ scales, int64_t cap, int32_t q_per_seq,
    const int32_t* __restrict__ idx, int32_t k_idx, const uint16_t* __restrict__ swa,
    int64_t swa_q_stride_rows, int32_t n_swa, int row0, bool tile_in_range, float scale_log2) {
  const int qb = blockIdx.y;
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int n = lane & 15, g = lane >> 4;
  const int row_local = wave * 16 + n;

  // ---- 1. loads of this lane's quarter (channels 128g..128g+127) of row n
  u32x4 raw[kSwa ? 16 : 4];
  uint2 s8 = {0u, 0u};
  bool ok;
  if (!kSwa) {
    const int r = row0 + n;  // selected-row slot
    const int32_t id = (tile_in_range && r < k_idx) ? idx[(int64_t)qb * k_idx + r] : -1;
    ok = id >= 0 && id < cap;
    const int64_t row = (int64_t)(qb / q_per_seq) * cap + (ok ? id : 0);
    const u32x4* cp = reinterpret_cast<const u32x4*>(codes + row * CSA2_CODE_BYTES + 64 * g);
#pragma unroll
    for (int i = 0; i < 4; ++i) raw[i] = cp[i];
    s8 = *reinterpret_cast<const uint2*>(scales + row * CSA2_SCALE_BYTES + 8 * g);
  } else {
    const int j = row0 + n;  // window row
    ok = tile_in_range && j < n_swa;
    const u32x4* sp = reinterpret_cast<const u32x4*>(
        swa + ((int64_t)qb * swa_q_stride_rows + (ok ? j : 0)) * CSA2_LATENT + 128 * g);
#pragma unroll
    for (int t = 0; t < 16; ++t) raw[t] = sp[t];
  }
  if (first) {
    // Main Q (loaded by the caller before the row loads) into LDS.
#pragma unroll
    for (int i = 0; i < 1024 / (64 * kAttnWaves); ++i) {
      const int c = tid + 64 * kAttnWaves * i;
      *reinterpret_cast<u32x4*>(&sm.qs[(c >> 6) * kXPitch + 8 * (c & 63)]) = qreg[i];
    }
    __syncthreads();
  }

  // ---- 2. dequantise, stage in LDS, and S^T[row][head] on MFMA
  f32x4 s = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int t = 0; t < 16; ++t) {
    u32x4 x;
    if (!kSwa) {
      const uint32_t sword = (t < 8) ? s8.x : s8.y;
      x = dequant8(raw[t >> 2][t & 3], e4m3_value((sword >> (8 * ((t >> 1) & 3))) & 0xFFu));
    } else {
      x = raw[t];
    }
    if (!ok) x = u32x4{0u, 0u, 0u, 0u};
    *reinterpret_cast<u32x4*>(&sm.xs[row_local * kXPitch + 128 * g + 8 * t]) = x;
    const u32x4 qv = *reinterpret_cast<const u32x4*>(&sm.qs[n * kXPitch + 128 * g + 8 * t]);
    s = mfma16x16x32(as_bf16x8(x), as_bf16x8(qv), s);
  }
  const uint64_t rows_ok = __ballot(ok);  // bit n (lanes 0..15) = row n of this wavefront
  float z[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) z[j] = ((rows_ok >> (4 * g + j)) & 1) ? s[j] * scale_log2 : kNegInf;

  // ---- 3. softmax statistics of the chunk, per head n, against the
  // running max (online softmax across the workgroup's chunks)
  float m = fmaxf(fmaxf(z[0], z[1]), fmaxf(z[2], z[3]));
  m = fmaxf(m, __shfl_xor(m, 16));
  m = fmaxf(m, __shfl_xor(m, 32));
  if (g == 0) sm.red_m[wave][n] = m;
  __syncthreads();
  float M = st.m_run;
#pragma unroll
  for (int w = 0; w < kAttnWaves; ++w) M = fmaxf(M, sm.red_m[w][n]);
  float lsum = 0.f;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const float p = (z[j] == kNegInf) ? 0.f : exp2f(z[j] - M);
    lsum += p;
    const uint32_t hi = f32_to_bf16_rne(p);
    const uint32_t lo = f32_to_bf16_rne(p - bf16_to_f32(hi));
    sm.ps[0][n * kPPitch + wave * 16 + 4 * g + j] = (uint16_t)hi;
    sm.ps[1][n * kPPitch + wave * 16 + 4 * g + j] = (uint16_t)lo;
  }
  lsum += __shfl_xor(lsum, 16);
  lsum += __shfl_xor(lsum, 32);
  if (g == 0) sm.red_l[wave][n] = lsum;
  if (tid < 16) sm.alpha[tid] = (st.m_run == kNegInf) ? 0.f : exp2f(st.m_run - M);
  const float alpha_n = (st.m_run == kNegInf) ? 0.f : exp2f(st.m_run - M);
  st.m_run = M;
  __syncthreads();

  // ---- 4. O[head][ch] for channels 64*wave .. +64 as 4 column tiles:
  // column tile c holds channels 64*wave + 4*n + c.
  if (!first) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const float a = sm.alpha[4 * g + j];
#pragma unroll
      for (int c = 0; c < 4; ++c) st.o[c][j] *= a;
    }
  }
  if (tid < 16) {
    float l = 0.f;
#pragma unroll
    for (int w = 0; w < kAttnWaves; ++w) l += sm.red_l[w][tid];
    st.l_run = st.l_run * alpha_n + l;
  }
#pragma unroll
  for (int ks = 0; ks < kAttnRows / 32; ++ks) {
    const bf16x8 ph = as_bf16x8(*reinterpret_cast<const u32x4*>(&sm.ps[0][n * kPPitch + 32 * ks + 8 * g]));
    const bf16x8 pl = as_bf16x8(*reinterpret_cast<const u32x4*>(&sm.ps[1][n * kPPitch + 32 * ks + 8 * g]));
    uint2 R[8];
#pragma unroll
    for (int i = 0; i < 8; ++i)
      R[i] = *reinterpret_cast<const uint2*>(&sm.xs[(32 * ks + 8 * g + i) * kXPitch + 64 * wave + 4 * n]);
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      u32x4 bc;
#pragma unroll
      for (int p = 0; p < 4; ++p) {
        const uint32_t a0 = (c < 2) ? R[2 * p].x : R[2 * p].y;
        const uint32_t a1 = (c < 2) ? R[2 * p + 1].x : R[2 * p + 1].y;
        bc[p] = (c & 1) ? byte_perm(a1, a0, 0x07060302u) : byte_perm(a1, a0, 0x05040100u);
      }
      st.o[c] = mfma16x16x32(ph, as_bf16x8(bc), st.o[c]);
      st.o[c] = mfma16x16x32(pl, as_bf16x8(bc), st.o[c]);
    }
  }
}

// One workgroup = chunks [split * per_split, ...) of query blockIdx.y.  With
// one split the workgroup covers the whole query and writes the normalised
// output; otherwise it writes its unnormalised O and (max, sum) per head
// for the combine kernel.
__global__ __launch_bounds__(64 * kAttnWaves) void attn_kernel(
    const uint16_t* __restrict__ q, const uint8_t* __restrict__ codes,
    const uint8_t* __restrict__ scales, int64_t cap, int32_t q_per_seq,
    const int32_t* __restrict__ idx, int32_t k_idx, const uint16_t* __restrict__ swa,
    int64_t swa_q_stride_rows, const int32_t* __restrict__ swa_len, int32_t swa_max,
    float scale_log2, int32_t per_split, float* __restrict__ part_o, float2* __restrict__ part_ml,
    int32_t n_split, float* __restrict__ out) {
  __shared__ __attribute__((aligned(16))) AttnSmem sm;
  const int qb = blockIdx.y, split = blockIdx.x;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int n = lane & 15, g = lane >> 4;
  // Main Q first: its loads overlap the index and row loads.
  u32x4 qreg[1024 / (64 * kAttnWaves)];
  {
    const u32x4* qp = reinterpret_cast<const u32x4*>(q + (int64_t)qb * 16 * CSA2_LATENT);
#pragma unroll
    for (int i = 0; i < 1024 / (64 * kAttnWaves); ++i) qreg[i] = qp[tid + 64 * kAttnWaves * i];
  }
  const int32_t n_swa = min(swa_len[qb], swa_max);
  // The query's tiles: FP4 tiles of 16 selected rows and window tiles of 16
  // rows, the window tiles spread evenly over the chunks so that every
  // chunk moves about the same bytes.  Each wavefront owns one tile of a chunk.
  const int fp4_tiles = (k_idx + 15) / 16, swa_tiles = (swa_max + 15) / 16;
  const int n_tiles = fp4_tiles + swa_tiles;
  const int n_chunks = (n_tiles + kAttnWaves - 1) / kAttnWaves;
  const int c_begin = split * per_split, c_end = min(n_chunks, c_begin + per_split);
  AttnState st;
#pragma unroll
  for (int c = 0; c < 4; ++c) st.o[c] = f32x4{0.f, 0.f, 0.f, 0.f};
  st.m_run = kNegInf;
  st.l_run = 0.f;
  for (int ch = c_begin; ch < c_end; ++ch) {
    if (ch != c_begin) __syncthreads();  // the previous chunk's LDS reads are done
    const int tile = ch * kAttnWaves + wave;
    const int swa_before = (int)(((int64_t)tile * swa_tiles) / n_tiles);
    const bool in_range = tile < n_tiles;
    const bool swa_tile = in_range && ((int64_t)(tile + 1) * swa_tiles) / n_tiles > swa_before;
    if (swa_tile)
      attn_chunk<true>(sm, st, ch == c_begin, qreg, codes, scales, cap, q_per_seq, idx, k_idx, swa,
                       swa_q_stride_rows, n_swa, swa_before * 16, in_range, scale_log2);
    else
      attn_chunk<false>(sm, st, ch == c_begin, qreg, codes, scales, cap, q_per_seq, idx, k_idx, swa,
                        swa_q_stride_rows, n_swa, (tile - swa_before) * 16, in_range, scale_log2);
  }

  if (n_split == 1) {
    if (tid < 16) sm.l_fin[tid] = st.l_run;
    __syncthreads();
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int head = 4 * g + j;
      const float l = sm.l_fin[head];
      const float inv = l > 0.f ? 1.f / l : 0.f;
      *reinterpret_cast<f32x4*>(out + ((int64_t)qb * 16 + head) * CSA2_LATENT + 64 * wave + 4 * n) =
          f32x4{st.o[0][j] * inv, st.o[1][j] * inv, st.o[2][j] * inv, st.o[3][j] * inv};
    }
    return;
  }
  float* po = part_o + ((int64_t)qb * n_split + split) * (16 * CSA2_LATENT);
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int head = 4 * g + j;
    *reinterpret_cast<f32x4*>(po + head * CSA2_LATENT + 64 * wave + 4 * n) =
        f32x4{st.o[0][j], st.o[1][j], st.o[2][j], st.o[3][j]};
  }
  if (tid < 16) part_ml[((int64_t)qb * n_split + split) * 16 + tid] = make_float2(st.m_run, st.l_run);
}

// Merge the chunks of one (head, query) with log-sum-exp weights:
//   o_h = sum_c 2^(m_c - M) O_c / sum_c 2^(m_c - M) l_c,  M = max_c m_c.
// One 128-thread workgroup per (head, query), one float4 of the head's 512
// channels per thread; the chunks' loads are issued together.
__global__ __launch_bounds__(128) void attn_combine_kernel(const float* __restrict__ part_o,
                                                           const float2* __restrict__ part_ml,
                                                           int32_t n_split, float* __restrict__ out) {
  const int h = blockIdx.x, qb = blockIdx.y, tid = threadIdx.x;
  const float2* ml = part_ml + (int64_t)qb * n_split * 16 + h;
  float Mq = kNegInf;
  for (int c = 0; c < n_split; ++c) Mq = fmaxf(Mq, ml[c * 16].x);
  const f32x4* pall = reinterpret_cast<const f32x4*>(part_o + (int64_t)qb * n_split * (16 * CSA2_LATENT) + h * CSA2_LATENT) + tid;
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  float den = 0.f;
  constexpr int kB = 16;
  for (int c0 = 0; c0 < n_split; c0 += kB) {
    f32x4 v[kB];
    float2 m[kB];
#pragma unroll
    for (int cb = 0; cb < kB; ++cb) {  // clamped: all loads in flight together
      const int c = min(c0 + cb, n_split - 1);
      v[cb] = pall[(int64_t)c * (16 * CSA2_LATENT / 4)];
      m[cb] = ml[c * 16];
    }
#pragma unroll
    for (int cb = 0; cb < kB; ++cb) {
      const float e = (c0 + cb >= n_split || m[cb].x == kNegInf) ? 0.f : exp2f(m[cb].x - Mq);
      den += e * m[cb].y;
      acc += e * v[cb];
    }
  }
  const float inv = den > 0.f ? 1.f / den : 0.f;
  reinterpret_cast<f32x4*>(out + ((int64_t)qb * 16 + h) * CSA2_LATENT)[tid] = acc * inv;
}

}  // namespace

// Workgroups per query: enough to fill the chip when there are few
// queries (split-K over chunks + a combine kernel), one per query otherwise
// (no partials).
static void attn_split_plan(int32_t n_q, int32_t k_idx, int32_t swa_max, int* splits, int* per_split) {
  const int n_chunks = attn_splits(k_idx, swa_max);
  const int want = std::max(1, std::min(n_chunks, (int)((1024 + (int64_t)n_q - 1) / std::max(1, n_q))));
  *per_split = (n_chunks + want - 1) / want;
  *splits = (n_chunks + *per_split - 1) / *per_split;
}

size_t attn_workspace_bytes(int32_t n_q, int32_t k_idx, int32_t swa_max) {
  int splits, per_split;
  attn_split_plan(n_q, k_idx, swa_max, &splits, &per_split);
  if (splits == 1) return 0;
  const size_t o_bytes = (size_t)n_q * splits * 16 * CSA2_LATENT * sizeof(float);
  const size_t ml_bytes = (size_t)n_q * splits * 16 * sizeof(float2);
  return o_bytes + ml_bytes;
}

csa2_status attn_launch(const uint16_t* q, int32_t n_q, const csa2_fp4_kv& kv, int32_t q_per_seq,
                        const int32_t* idx, int32_t k_idx, const uint16_t* swa, int64_t swa_q_stride_rows,
                        const int32_t* swa_len, int32_t swa_max, float sm_scale, float* out, void* ws,
                        hipStream_t stream) {
  if (n_q == 0) return CSA2_OK;
  int splits, per_split;
  attn_split_plan(n_q, k_idx, swa_max, &splits, &per_split);
  float* part_o = nullptr;
  float2* part_ml = nullptr;
  if (splits > 1) {
    char* base = reinterpret_cast<char*>(ws);
    part_o = reinterpret_cast<float*>(base);
    base += (size_t)n_q * splits * 16 * CSA2_LATENT * sizeof(float);
    part_ml = reinterpret_cast<float2*>(base);
  }
  const float scale_log2 = sm_scale * 1.4426950408889634f;
  hipLaunchKernelGGL(attn_kernel, dim3(splits, n_q), dim3(64 * kAttnWaves), 0, stream, q, kv.codes, kv.scales,
                     kv.cap, q_per_seq, idx, k_idx, swa, swa_q_stride_rows, swa_len, swa_max, scale_log2,
                     per_split, part_o, part_ml, splits, out);
  if (splits > 1)
    hipLaunchKernelGGL(attn_combine_kernel, dim3(16, n_q), dim3(128), 0, stream, part_o, part_ml, splits, out);
  return launch_status("csa2_sparse_attn");
}

}  // namespace csa2
