// Step (a): FP4 quantisation of 512-d latent rows, bulk and append.
//
// Format [P1 "FP4 KV, Bounded Replay, and Other Extensions"]: E2M1 values,
// one E4M3 scale per 16 channels, NVFP4 without its global scale.  One
// wavefront quantises one row: lane l owns channels 8l..8l+7 (one 16-byte
// load), lanes 2g and 2g+1 form scale group g.  Both decisions -- the scale
// code and each magnitude code -- are taken by exact binary32 comparisons
// against products of short significands, so they equal round-to-nearest-
// even of the exact ratios for every finite bf16 input (no division and no
// reciprocal is involved).
//
// Citation key: [P1] "DeepSeek AI Released DeepSeek-V4.1-Flash with 1M
// Context, FP4 KV Cache, and Cross-Layer Attention Reuse".
#include "common.hpp"

namespace csa2 {
namespace {

// E4M3 code of amax/6, round-to-nearest-even, saturating at 448 (0x7E).
// Binary search for the largest code c with 6*v(c) <= amax (exact: 6*v(c)
// has at most 6 significant bits), then compare amax with 6 times the
// midpoint to the next code (also exact); a tie takes the even code.
__device__ __forceinline__ uint32_t scale_code(float amax) {
  uint32_t lo = 0, hi = 126;  // invariant: 6*v(lo) <= amax (v(0) = 0)
  while (lo < hi) {
    const uint32_t mid = (lo + hi + 1) >> 1;
    if (6.0f * e4m3_pos_value(mid) <= amax) lo = mid; else hi = mid - 1;
  }
  if (lo == 126) return 126;
  const float t = 3.0f * (e4m3_pos_value(lo) + e4m3_pos_value(lo + 1));  // 6 * midpoint
  if (amax > t) return lo + 1;
  if (amax == t) return (lo & 1u) ? lo + 1 : lo;
  return lo;
}

// Magnitude code of |x| under scale s > 0: thresholds at the midpoints
// 0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5 (times s, exact products); at a
// midpoint the even code wins, so the comparison is strict below an odd
// code and non-strict below an even one.
__device__ __forceinline__ uint32_t mag_code(float ax, float s) {
  uint32_t m = 0;
  m += ax > 0.25f * s;
  m += ax >= 0.75f * s;
  m += ax > 1.25f * s;
  m += ax >= 1.75f * s;
  m += ax > 2.5f * s;
  m += ax >= 3.5f * s;
  m += ax > 5.0f * s;
  return m;
}

// E4M3 code of one bf16 value (bits b): round-to-nearest-even of x onto
// the E4M3FN grid, saturating at +-448 (0x7E), sign copied (also for 0),
// NaN kept (S.1111.111).  Same exact search as scale_code with factor 1:
// the largest code c with v(c) <= |x|, then |x| against the midpoint.
__device__ __forceinline__ uint32_t fp8_code(uint32_t b) {
  const uint32_t sign = (b >> 8) & 0x80u;
  const float ax = bf16_to_f32(b & 0x7FFFu);
  if (ax != ax) return sign | 0x7Fu;
  uint32_t lo = 0, hi = 126;  // invariant: v(lo) <= ax (v(0) = 0)
  while (lo < hi) {
    const uint32_t mid = (lo + hi + 1) >> 1;
    if (e4m3_pos_value(mid) <= ax) lo = mid; else hi = mid - 1;
  }
  uint32_t c = lo;
  if (lo < 126) {
    const float t = 0.5f * (e4m3_pos_value(lo) + e4m3_pos_value(lo + 1));  // exact midpoint
    if (ax > t || (ax == t && (lo & 1u))) c = lo + 1;
  }
  return sign | c;
}

// FP8 window rows: 8 channels per thread (16 bytes in, 8 bytes out).
__global__ __launch_bounds__(256) void quant_fp8_kernel(const uint16_t* __restrict__ src, int64_t n_vec,
                                                        uint8_t* __restrict__ dst) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= n_vec) return;
  const u32x4 raw = reinterpret_cast<const u32x4*>(src)[i];
  uint32_t lo = 0, hi = 0;
#pragma unroll
  for (int k = 0; k < 2; ++k) {
    lo |= fp8_code(raw[k] & 0xFFFFu) << (16 * k);
    lo |= fp8_code(raw[k] >> 16) << (16 * k + 8);
    hi |= fp8_code(raw[k + 2] & 0xFFFFu) << (16 * k);
    hi |= fp8_code(raw[k + 2] >> 16) << (16 * k + 8);
  }
  reinterpret_cast<uint2*>(dst)[i] = make_uint2(lo, hi);
}

// Quantise the 512 bf16 values at src into one packed row (one wavefront).
__device__ __forceinline__ void quant_row_wave(const uint16_t* __restrict__ src,
                                               uint8_t* __restrict__ codes,
                                               uint8_t* __restrict__ scales, int lane) {
  const u32x4 raw = *reinterpret_cast<const u32x4*>(src + 8 * lane);
  uint32_t bits[8];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    bits[2 * i] = raw[i] & 0xFFFFu;
    bits[2 * i + 1] = raw[i] >> 16;
  }
  float amax = 0.0f;
#pragma unroll
  for (int i = 0; i < 8; ++i) amax = fmaxf(amax, bf16_to_f32(bits[i] & 0x7FFFu));
  amax = fold1_max(amax);
  const uint32_t sc = scale_code(amax);
  const float s = e4m3_pos_value(sc);
  uint32_t packed = 0;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const uint32_t m = (sc == 0) ? 0u : mag_code(bf16_to_f32(bits[i] & 0x7FFFu), s);
    const uint32_t code = ((bits[i] >> 12) & 8u) | m;
    packed |= code << (4 * i);
  }
  reinterpret_cast<uint32_t*>(codes)[lane] = packed;
  if ((lane & 1) == 0) scales[lane >> 1] = (uint8_t)sc;
}

__global__ __launch_bounds__(256) void quant_rows_kernel(const uint16_t* __restrict__ src,
                                                         int64_t n_rows, uint8_t* __restrict__ codes,
                                                         uint8_t* __restrict__ scales) {
  const int lane = threadIdx.x & 63;
  const int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= n_rows) return;
  quant_row_wave(src + row * CSA2_LATENT, codes + row * CSA2_CODE_BYTES,
                 scales + row * CSA2_SCALE_BYTES, lane);
}

__global__ __launch_bounds__(64) void quant_append_kernel(const uint16_t* __restrict__ src,
                                                          uint8_t* __restrict__ codes,
                                                          uint8_t* __restrict__ scales, int64_t cap,
                                                          int32_t* __restrict__ lens,
                                                          int32_t* __restrict__ err_flag) {
  const int b = blockIdx.x;
  const int lane = threadIdx.x;
  const int64_t row = lens[b];
  if (row < 0 || row >= cap) {
    if (lane == 0 && err_flag) atomicOr(err_flag, 1);
    return;
  }
  const int64_t r = (int64_t)b * cap + row;
  quant_row_wave(src + (int64_t)b * CSA2_LATENT, codes + r * CSA2_CODE_BYTES,
                 scales + r * CSA2_SCALE_BYTES, lane);
  if (lane == 0) lens[b] = (int32_t)(row + 1);
}

}  // namespace

csa2_status quant_rows_launch(const uint16_t* src, int64_t n_rows, uint8_t* codes, uint8_t* scales,
                              hipStream_t stream) {
  if (n_rows == 0) return CSA2_OK;
  const int64_t blocks = (n_rows + 3) / 4;
  CSA2_REQUIRE(blocks <= 0x7FFFFFFF, CSA2_ESHAPE, "csa2_quant_rows: too many rows for one launch");
  hipLaunchKernelGGL(quant_rows_kernel, dim3((uint32_t)blocks), dim3(256), 0, stream, src, n_rows,
                     codes, scales);
  return launch_status("csa2_quant_rows");
}

csa2_status quant_fp8_launch(const uint16_t* src, int64_t n_rows, uint8_t* dst, hipStream_t stream) {
  if (n_rows == 0) return CSA2_OK;
  const int64_t n_vec = n_rows * (CSA2_LATENT / 8);
  const int64_t blocks = (n_vec + 255) / 256;
  CSA2_REQUIRE(blocks <= 0x7FFFFFFF, CSA2_ESHAPE, "csa2_quant_fp8_rows: too many rows for one launch");
  hipLaunchKernelGGL(quant_fp8_kernel, dim3((uint32_t)blocks), dim3(256), 0, stream, src, n_vec, dst);
  return launch_status("csa2_quant_fp8_rows");
}

csa2_status quant_append_launch(const uint16_t* src, const csa2_fp4_kv& kv, int32_t* lens,
                                int32_t* err_flag, hipStream_t stream) {
  if (kv.n_seq == 0) return CSA2_OK;
  hipLaunchKernelGGL(quant_append_kernel, dim3(kv.n_seq), dim3(64), 0, stream, src, kv.codes,
                     kv.scales, kv.cap, lens, err_flag);
  return launch_status("csa2_quant_append");
}

}  // namespace csa2
