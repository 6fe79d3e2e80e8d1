// Row conversions shared by the attention kernels: FP4 main-KV rows and
// bf16 / E4M3 window rows to f16 operands of the MFMA products.
#pragma once

#include "common.hpp"

namespace csa2 {

// Selected rows per query that the many-query attention kernel takes (its
// row ids are staged in LDS); more go to the workgroup kernels.
constexpr int kAttnManyMaxIdx = 512;

// Dequantise 8 channels -- code dword dw, channel i in nibble i (byte j =
// channels 2j (low nibble) and 2j+1) -- with the scale as an f16 pair s2:
// four FP4-pair conversions at scale 1 (exact E2M1 values), each followed
// by one packed f16 multiply (exact).  Returns 4 f16 pairs, channel order.
__device__ __forceinline__ u32x4 dequant8_f16(uint32_t dw, f16x2 s2) {
  u32x4 r;
  r[0] = __builtin_bit_cast(uint32_t, __builtin_bit_cast(f16x2, __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(dw, 1.0f, 0)) * s2);
  r[1] = __builtin_bit_cast(uint32_t, __builtin_bit_cast(f16x2, __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(dw, 1.0f, 1)) * s2);
  r[2] = __builtin_bit_cast(uint32_t, __builtin_bit_cast(f16x2, __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(dw, 1.0f, 2)) * s2);
  r[3] = __builtin_bit_cast(uint32_t, __builtin_bit_cast(f16x2, __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(dw, 1.0f, 3)) * s2);
  return r;
}

// Two bf16 values (one dword) as an f16 pair, rounding toward zero
// (v_cvt_pkrtz_f16_f32: exact for |x| in [2^-14, 65504], saturating above).
__device__ __forceinline__ uint32_t bf16x2_to_f16x2(uint32_t u) {
  const float lo = __builtin_bit_cast(float, u << 16), hi = __builtin_bit_cast(float, u & 0xFFFF0000u);
  return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_pkrtz(lo, hi));
}

__device__ __forceinline__ u32x4 bf16x8_to_f16x8(u32x4 v) {
  return u32x4{bf16x2_to_f16x2(v[0]), bf16x2_to_f16x2(v[1]), bf16x2_to_f16x2(v[2]), bf16x2_to_f16x2(v[3])};
}

// Eight E4M3 bytes (two dwords) as four f16 pairs (exact).
__device__ __forceinline__ u32x4 fp8x8_to_f16x8(uint32_t d0, uint32_t d1) {
  return u32x4{__builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(d0, 1.0f, false)),
               __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(d0, 1.0f, true)),
               __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(d1, 1.0f, false)),
               __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(d1, 1.0f, true))};
}

// The E4M3 scale of channel group k (8 channels) of a lane's 128, splat
// into both halves of an f16 pair: sc[i] holds the lane's scale bytes 2i
// (low half) and 2i + 1 as f16, and group k uses scale byte k / 2.
__device__ __forceinline__ f16x2 scale_pair(const uint32_t (&sc)[4], int k) {
  const uint32_t w = sc[k >> 2];
  return __builtin_bit_cast(f16x2, ((k >> 1) & 1) ? byte_perm(w, w, 0x03020302u) : byte_perm(w, w, 0x01000100u));
}

// A lane's 8 scale bytes (s8x: bytes 0..3, s8y: 4..7) as f16 pairs (exact
// E4M3 conversions, two per instruction).
__device__ __forceinline__ void scales_f16(uint32_t s8x, uint32_t s8y, uint32_t (&sc)[4]) {
  sc[0] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(s8x, 1.0f, false));
  sc[1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(s8x, 1.0f, true));
  sc[2] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(s8y, 1.0f, false));
  sc[3] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(s8y, 1.0f, true));
}

}  // namespace csa2
