// Internal helpers shared by the HIP kernels and the C ABI of libcsa2.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <string>

#include "csa2.h"

namespace csa2 {

// ---------------------------------------------------------------- errors
void set_error(const std::string& msg);
void clear_error();

#define CSA2_REQUIRE(cond, code, msg)      \
  do {                                     \
    if (!(cond)) {                         \
      ::csa2::set_error(msg);              \
      return (code);                       \
    }                                      \
  } while (0)

// Status after a kernel launch: CSA2_EHIP with the runtime's message.
csa2_status launch_status(const char* what);

inline hipStream_t as_stream(void* s) { return reinterpret_cast<hipStream_t>(s); }

// ---------------------------------------------------------------- vectors
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 v) { return __builtin_bit_cast(bf16x8, v); }
__device__ __forceinline__ f16x8 as_f16x8(u32x4 v) { return __builtin_bit_cast(f16x8, v); }

// D = A(16x32) * B(32x16) + C on one wavefront (gfx950).  Lane l holds
// A[l%16][8*(l/16) .. +7], B[8*(l/16) .. +7][l%16] and returns
// C[4*(l/16) .. +3][l%16].
__device__ __forceinline__ f32x4 mfma16x16x32(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// The same shape with f16 operands (v_mfma_f32_16x16x32_f16).
__device__ __forceinline__ f32x4 mfma16x16x32_f16(f16x8 a, f16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}

// --------------------------------------------------------------- bf16/f32
__host__ __device__ __forceinline__ float bf16_to_f32(uint32_t b) {
  return __builtin_bit_cast(float, b << 16);
}
// Round-to-nearest-even to bf16 (finite inputs).
__host__ __device__ __forceinline__ uint32_t f32_to_bf16_rne(float f) {
  uint32_t u = __builtin_bit_cast(uint32_t, f);
  return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}

// ----------------------------------------------------------------- E4M3FN
// Value of a non-negative E4M3FN code c in 0..126: exponent field 0 is
// subnormal (m * 2^-9), otherwise (1 + m/8) * 2^(e-7).
__host__ __device__ __forceinline__ float e4m3_pos_value(uint32_t c) {
  const uint32_t e = (c >> 3) & 15u, m = c & 7u;
  if (e == 0) return (float)m * 0.001953125f;  // 2^-9
  return __builtin_bit_cast(float, ((e + 120u) << 23) | (m << 20));
}

// ----------------------------------------------------------------- E2M1
// E2M1 magnitude code m (0..7) as binary32: codes 2..7 are normal numbers
// 2^(e-1)(1 + mant/2) whose binary32 pattern is (m << 22) + 0x3F000000;
// code 1 is 0.5 and code 0 is 0.
__host__ __device__ __forceinline__ float e2m1_mag_value(uint32_t m) {
  const float normal = __builtin_bit_cast(float, (m << 22) + 0x3F000000u);
  return m >= 2u ? normal : 0.5f * (float)m;
}

// Byte permute (v_perm_b32): result byte i = byte sel_i of the 8-byte value
// hi:lo (selector 0..3 = bytes of lo, 4..7 = bytes of hi, 12 = zero byte).
__device__ __forceinline__ uint32_t byte_perm(uint32_t hi, uint32_t lo, uint32_t sel) {
  return __builtin_amdgcn_perm(hi, lo, sel);
}

// Workgroup barrier for an LDS hand-off only: waits for this wavefront's
// LDS operations, then for every wavefront, but leaves its global loads in
// flight (__syncthreads() also waits for all outstanding global memory
// operations, which would drain a prefetch).  The memory clobber keeps the
// compiler from moving memory accesses across it.
// Cross-lane folds on VALU moves instead of LDS-crossbar shuffles: lane i
// gets op(x[i], x[i ^ d]) for d = 16 (v_permlane16_swap: odd and even rows of
// 16 lanes exchanged), d = 32 (v_permlane32_swap: the halves exchanged) and
// d = 1 (DPP quad_perm [1, 0, 3, 2]).  The swaps return both exchanged
// copies, and op is commutative, so the result is that of the shuffle.
__device__ __forceinline__ float fold16_max(float x) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float fold32_max(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float fold16_add(float x) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ __forceinline__ float fold32_add(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ __forceinline__ float fold1_max(float x) {
  return fmaxf(x, __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), 0xB1, 0xF, 0xF, false)));
}

__device__ __forceinline__ void lds_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

// Scores that are not candidates.
constexpr float kNegInf = -__builtin_huge_valf();

// Element type of the window rows handed to the attention kernels.
constexpr int kWinBf16 = 0;  // bf16, converted to f16 toward zero in the kernel
constexpr int kWinE4m3 = 1;  // OCP E4M3FN bytes

}  // namespace csa2
