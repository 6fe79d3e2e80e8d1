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
// rows, then swa_max window rows) are cut into chunks of 64; one 256-thread
// workgroup handles one chunk of one query:
//   1. each wavefront owns 16 rows; lane (n = l%16, g = l/16) loads row n's
//      channels 128g..128g+127 (FP4: 64 code bytes + 8 scale bytes; SWA: 256
//      bytes of bf16) and dequantises in registers: E2M1 magnitude and E4M3
//      scale are expanded to binary32, multiplied (exact) and truncated to
//      bf16 (exact: the product has at most 6 significant bits);
//   2. S^T = X Q^T on v_mfma_f32_16x16x32_bf16 (16 steps over 512 channels),
//      the dequantised registers being the A operand directly; the rows also
//      go to LDS for the second product;
//   3. softmax statistics per head over the chunk (max, then exp2 and sum);
//      P is split into bf16 hi + lo parts (P ~ hi + lo to 2^-16) so the PV
//      product keeps fp32-level accuracy on bf16 MFMA;
//   4. O = P X: wavefront w computes channels 128w..128w+127 as 8 column
//      tiles whose B operands come from 16-byte LDS reads of 8 rows, split
//      into per-column vectors;
//   5. the chunk writes its unnormalised O and (max, sum) per head.
// A second kernel combines the chunks of each query (log-sum-exp merge).
//
// Citation keys: [P1] "DeepSeek AI Released DeepSeek-V4.1-Flash with 1M
// Context, FP4 KV Cache, and Cross-Layer Attention Reuse"; [P3]
// "DeepSeek-V4.1 Flash: Pushing the Limits of KV Cache Compression".
#include "common.hpp"

namespace csa2 {

constexpr int kAttnRows = 64;                  // rows per workgroup chunk
constexpr int kXPitch = CSA2_LATENT + 8;       // LDS row pitch, bf16 elements
constexpr int kPPitch = kAttnRows + 8;         // LDS P pitch, bf16 elements
constexpr int kMaxSplits = 128;

inline int attn_splits(int32_t k_idx, int32_t swa_max) {
  return (k_idx + swa_max + kAttnRows - 1) / kAttnRows;
}

namespace {

// Dequantise 8 channels (one code dword) with scale s into 4 bf16 pairs.
__device__ __forceinline__ u32x4 dequant8(uint32_t dw, float s) {
  u32x4 r;
#pragma unroll
  for (int p = 0; p < 4; ++p) {
    uint32_t h[2];
#pragma unroll
    for (int e = 0; e < 2; ++e) {
      const uint32_t code = (dw >> (4 * (2 * p + e))) & 15u;
      const float v = e2m1_mag_value(code & 7u) * s;
      h[e] = (__builtin_bit_cast(uint32_t, v) >> 16) ^ ((code & 8u) << 12);
    }
    r[p] = h[0] | (h[1] << 16);
  }
  return r;
}

// E4M3FN scale byte as binary32 (sign, NaN for S.1111.111).
__device__ __forceinline__ float e4m3_value(uint32_t c) {
  const uint32_t mag = c & 0x7Fu;
  const float v = (mag == 0x7Fu) ? __builtin_nanf("") : e4m3_pos_value(mag);
  return (c & 0x80u) ? -v : v;
}

__global__ __launch_bounds__(256) void attn_chunk_kernel(
    const uint16_t* __restrict__ q, const uint8_t* __restrict__ codes,
    const uint8_t* __restrict__ scales, int64_t cap, int32_t q_per_seq,
    const int32_t* __restrict__ idx, int32_t k_idx, const uint16_t* __restrict__ swa,
    int64_t swa_q_stride_rows, const int32_t* __restrict__ swa_len, int32_t swa_max,
    float scale_log2, float* __restrict__ part_o, float2* __restrict__ part_ml, int32_t n_split) {
  __shared__ __attribute__((aligned(16))) uint16_t xs[kAttnRows * kXPitch];
  __shared__ __attribute__((aligned(16))) uint16_t ps[2][16 * kPPitch];
  __shared__ float red_m[4][16];
  __shared__ float red_l[4][16];

  const int qb = blockIdx.y, split = blockIdx.x;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int n = lane & 15, g = lane >> 4;
  const int row_local = wave * 16 + n;
  const int64_t r = (int64_t)split * kAttnRows + row_local;
  const int32_t n_swa = min(swa_len[qb], swa_max);

  // ---- 1. load and dequantise this lane's quarter of row r
  u32x4 xr[16];
  bool ok = false;
  if (r < k_idx) {
    const int32_t id = idx[(int64_t)qb * k_idx + r];
    if (id >= 0 && id < cap) {
      ok = true;
      const int64_t row = (int64_t)(qb / q_per_seq) * cap + id;
      const u32x4* cp = reinterpret_cast<const u32x4*>(codes + row * CSA2_CODE_BYTES + 64 * g);
      const uint2 s8 = *reinterpret_cast<const uint2*>(scales + row * CSA2_SCALE_BYTES + 8 * g);
      u32x4 c[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) c[i] = cp[i];
#pragma unroll
      for (int t = 0; t < 16; ++t) {
        const uint32_t sword = (t < 8) ? s8.x : s8.y;
        const float s = e4m3_value((sword >> (8 * ((t >> 1) & 3))) & 0xFFu);
        xr[t] = dequant8(c[t >> 2][t & 3], s);
      }
    }
  } else {
    const int64_t j = r - k_idx;
    if (j < n_swa) {
      ok = true;
      const u32x4* sp = reinterpret_cast<const u32x4*>(
          swa + ((int64_t)qb * swa_q_stride_rows + j) * CSA2_LATENT + 128 * g);
#pragma unroll
      for (int t = 0; t < 16; ++t) xr[t] = sp[t];
    }
  }
  if (!ok) {
#pragma unroll
    for (int t = 0; t < 16; ++t) xr[t] = u32x4{0, 0, 0, 0};
  }
  // Query operand: head n, channels 128g + 8t .. +8.
  u32x4 qv[16];
  {
    const u32x4* qp = reinterpret_cast<const u32x4*>(q + ((int64_t)qb * 16 + n) * CSA2_LATENT + 128 * g);
#pragma unroll
    for (int t = 0; t < 16; ++t) qv[t] = qp[t];
  }
#pragma unroll
  for (int t = 0; t < 16; ++t)
    *reinterpret_cast<u32x4*>(&xs[row_local * kXPitch + 128 * g + 8 * t]) = xr[t];

  // ---- 2. logits S^T[row][head] for the wavefront's 16 rows
  f32x4 s = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int t = 0; t < 16; ++t) s = mfma16x16x32(as_bf16x8(xr[t]), as_bf16x8(qv[t]), s);
  const uint64_t rows_ok = __ballot(ok);  // bit n (lanes 0..15) = row n of this wavefront
  float z[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) z[j] = ((rows_ok >> (4 * g + j)) & 1) ? s[j] * scale_log2 : kNegInf;

  // ---- 3. softmax statistics of the chunk, per head n
  float m = fmaxf(fmaxf(z[0], z[1]), fmaxf(z[2], z[3]));
  m = fmaxf(m, __shfl_xor(m, 16));
  m = fmaxf(m, __shfl_xor(m, 32));
  if (g == 0) red_m[wave][n] = m;
  __syncthreads();
  const float M = fmaxf(fmaxf(red_m[0][n], red_m[1][n]), fmaxf(red_m[2][n], red_m[3][n]));
  float lsum = 0.f;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const float p = (z[j] == kNegInf) ? 0.f : exp2f(z[j] - M);
    lsum += p;
    const uint32_t hi = f32_to_bf16_rne(p);
    const uint32_t lo = f32_to_bf16_rne(p - bf16_to_f32(hi));
    ps[0][n * kPPitch + wave * 16 + 4 * g + j] = (uint16_t)hi;
    ps[1][n * kPPitch + wave * 16 + 4 * g + j] = (uint16_t)lo;
  }
  lsum += __shfl_xor(lsum, 16);
  lsum += __shfl_xor(lsum, 32);
  if (g == 0) red_l[wave][n] = lsum;
  __syncthreads();

  // ---- 4. O[head][ch] for channels 128*wave .. +128 as 8 column tiles
  f32x4 o[8];
#pragma unroll
  for (int c = 0; c < 8; ++c) o[c] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int ks = 0; ks < kAttnRows / 32; ++ks) {
    const bf16x8 ph = as_bf16x8(*reinterpret_cast<const u32x4*>(&ps[0][n * kPPitch + 32 * ks + 8 * g]));
    const bf16x8 pl = as_bf16x8(*reinterpret_cast<const u32x4*>(&ps[1][n * kPPitch + 32 * ks + 8 * g]));
    u32x4 R[8];
#pragma unroll
    for (int i = 0; i < 8; ++i)
      R[i] = *reinterpret_cast<const u32x4*>(&xs[(32 * ks + 8 * g + i) * kXPitch + 128 * wave + 8 * n]);
#pragma unroll
    for (int c = 0; c < 8; ++c) {
      u32x4 bc;
#pragma unroll
      for (int p = 0; p < 4; ++p) {
        const uint32_t a0 = R[2 * p][c >> 1], a1 = R[2 * p + 1][c >> 1];
        bc[p] = (c & 1) ? ((a0 >> 16) | (a1 & 0xFFFF0000u)) : ((a0 & 0xFFFFu) | (a1 << 16));
      }
      o[c] = mfma16x16x32(ph, as_bf16x8(bc), o[c]);
      o[c] = mfma16x16x32(pl, as_bf16x8(bc), o[c]);
    }
  }

  // ---- 5. chunk results: unnormalised O and (max, sum) per head
  float* po = part_o + ((int64_t)qb * n_split + split) * (16 * CSA2_LATENT);
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int head = 4 * g + j;
    f32x4 v0 = {o[0][j], o[1][j], o[2][j], o[3][j]};
    f32x4 v1 = {o[4][j], o[5][j], o[6][j], o[7][j]};
    f32x4* dst = reinterpret_cast<f32x4*>(po + head * CSA2_LATENT + 128 * wave + 8 * n);
    dst[0] = v0;
    dst[1] = v1;
  }
  if (threadIdx.x < 16) {
    const int h = threadIdx.x;
    part_ml[((int64_t)qb * n_split + split) * 16 + h] =
        make_float2(M, red_l[0][h] + red_l[1][h] + red_l[2][h] + red_l[3][h]);
  }
}

// Merge the chunks of one query: o_h = sum_c 2^(m_c - M) O_c / sum_c 2^(m_c - M) l_c.
__global__ __launch_bounds__(256) void attn_combine_kernel(const float* __restrict__ part_o,
                                                           const float2* __restrict__ part_ml,
                                                           int32_t n_split, float* __restrict__ out) {
  __shared__ float wgt[16][kMaxSplits];
  const int qb = blockIdx.x;
  const float2* ml = part_ml + (int64_t)qb * n_split * 16;
  if (threadIdx.x < 16) {
    const int h = threadIdx.x;
    float M = kNegInf;
    for (int c = 0; c < n_split; ++c) M = fmaxf(M, ml[c * 16 + h].x);
    float den = 0.f;
    for (int c = 0; c < n_split; ++c) {
      const float2 v = ml[c * 16 + h];
      const float e = (v.x == kNegInf) ? 0.f : exp2f(v.x - M);
      wgt[h][c] = e;
      den += e * v.y;
    }
    const float inv = den > 0.f ? 1.f / den : 0.f;
    for (int c = 0; c < n_split; ++c) wgt[h][c] *= inv;
  }
  __syncthreads();
  const float* po = part_o + (int64_t)qb * n_split * (16 * CSA2_LATENT);
  float* ob = out + (int64_t)qb * 16 * CSA2_LATENT;
  for (int e = threadIdx.x; e < 16 * CSA2_LATENT / 4; e += 256) {
    const int h = (4 * e) / CSA2_LATENT;
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
    for (int c = 0; c < n_split; ++c) {
      const f32x4 v = reinterpret_cast<const f32x4*>(po + (int64_t)c * 16 * CSA2_LATENT)[e];
      acc += wgt[h][c] * v;
    }
    reinterpret_cast<f32x4*>(ob)[e] = acc;
  }
}

}  // namespace

size_t attn_workspace_bytes(int32_t n_q, int32_t k_idx, int32_t swa_max) {
  const size_t splits = (size_t)attn_splits(k_idx, swa_max);
  const size_t o_bytes = (size_t)n_q * splits * 16 * CSA2_LATENT * sizeof(float);
  const size_t ml_bytes = (size_t)n_q * splits * 16 * sizeof(float2);
  return o_bytes + ml_bytes;
}

csa2_status attn_launch(const uint16_t* q, int32_t n_q, const csa2_fp4_kv& kv, int32_t q_per_seq,
                        const int32_t* idx, int32_t k_idx, const uint16_t* swa, int64_t swa_q_stride_rows,
                        const int32_t* swa_len, int32_t swa_max, float sm_scale, float* out, void* ws,
                        hipStream_t stream) {
  if (n_q == 0) return CSA2_OK;
  const int splits = attn_splits(k_idx, swa_max);
  float* part_o = reinterpret_cast<float*>(ws);
  float2* part_ml = reinterpret_cast<float2*>(
      reinterpret_cast<char*>(ws) + (size_t)n_q * splits * 16 * CSA2_LATENT * sizeof(float));
  const float scale_log2 = sm_scale * 1.4426950408889634f;
  hipLaunchKernelGGL(attn_chunk_kernel, dim3(splits, n_q), dim3(256), 0, stream, q, kv.codes,
                     kv.scales, kv.cap, q_per_seq, idx, k_idx, swa, swa_q_stride_rows, swa_len,
                     swa_max, scale_log2, part_o, part_ml, splits);
  hipLaunchKernelGGL(attn_combine_kernel, dim3(n_q), dim3(256), 0, stream, part_o, part_ml, splits,
                     out);
  return launch_status("csa2_sparse_attn");
}

}  // namespace csa2
