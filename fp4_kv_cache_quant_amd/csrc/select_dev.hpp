// Workgroup-wide building blocks of the radix selections (internal; used by
// the Top-k kernels and by the scoring kernel's per-workgroup selection).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace csa2 {

__device__ __forceinline__ int lane_id() { return threadIdx.x & 63; }

// Inclusive prefix sum over the 64 lanes of a wavefront on DPP moves (no
// LDS round trips): shifts right by 1, 2, 4 and 8 lanes inside each row of
// 16 lanes (lanes shifted in from outside the row add 0), then the last
// lane of row 0 is added to row 1 and that of row 2 to row 3 (row_bcast:15),
// then the last lane of row 1 to rows 2 and 3 (row_bcast:31).
__device__ __forceinline__ uint32_t wave_inclusive_scan(uint32_t v) {
  int x = (int)v;
  x += __builtin_amdgcn_update_dpp(0, x, 0x111, 0xF, 0xF, true);   // row_shr:1
  x += __builtin_amdgcn_update_dpp(0, x, 0x112, 0xF, 0xF, true);   // row_shr:2
  x += __builtin_amdgcn_update_dpp(0, x, 0x114, 0xF, 0xF, true);   // row_shr:4
  x += __builtin_amdgcn_update_dpp(0, x, 0x118, 0xF, 0xF, true);   // row_shr:8
  x += __builtin_amdgcn_update_dpp(0, x, 0x142, 0xA, 0xF, false);  // row_bcast:15 into rows 1, 3
  x += __builtin_amdgcn_update_dpp(0, x, 0x143, 0xC, 0xF, false);  // row_bcast:31 into rows 2, 3
  return (uint32_t)x;
}

// Exclusive prefix sum over a workgroup of NT threads in thread order.
template <int NT>
__device__ __forceinline__ uint32_t block_exclusive_scan(uint32_t v, uint32_t* wave_sum, uint32_t* total) {
  constexpr int kW = NT / 64;
  const int lane = lane_id(), wave = threadIdx.x >> 6;
  const uint32_t x = wave_inclusive_scan(v);
  if (lane == 63) wave_sum[wave] = x;
  __syncthreads();
  uint32_t before = 0, all = 0;
#pragma unroll
  for (int i = 0; i < kW; ++i) {
    const uint32_t s = wave_sum[i];
    before += (i < wave) ? s : 0u;
    all += s;
  }
  __syncthreads();
  *total = all;
  return before + x - v;
}

// The same scan with a single barrier: wave_sum (kW words) must not be
// written again by this workgroup -- each call site owns its slot.
template <int NT>
__device__ __forceinline__ uint32_t block_exclusive_scan_once(uint32_t v, uint32_t* wave_sum, uint32_t* total) {
  constexpr int kW = NT / 64;
  const int lane = lane_id(), wave = threadIdx.x >> 6;
  const uint32_t x = wave_inclusive_scan(v);
  if (lane == 63) wave_sum[wave] = x;
  __syncthreads();
  uint32_t before = 0, all = 0;
#pragma unroll
  for (int i = 0; i < kW; ++i) {
    const uint32_t s = wave_sum[i];
    before += (i < wave) ? s : 0u;
    all += s;
  }
  *total = all;
  return before + x - v;
}

// Two exclusive prefix sums at once (a.x and a.y), one barrier; wave_sum
// holds 2 * NT / 64 words owned by the call site as above.
template <int NT>
__device__ __forceinline__ uint2 block_exclusive_scan2_once(uint2 v, uint32_t* wave_sum, uint2* total) {
  constexpr int kW = NT / 64;
  const int lane = lane_id(), wave = threadIdx.x >> 6;
  const uint32_t x = wave_inclusive_scan(v.x), y = wave_inclusive_scan(v.y);
  if (lane == 63) wave_sum[wave] = x, wave_sum[kW + wave] = y;
  __syncthreads();
  uint2 before = make_uint2(0u, 0u), all = make_uint2(0u, 0u);
#pragma unroll
  for (int i = 0; i < kW; ++i) {
    const uint32_t sx = wave_sum[i], sy = wave_sum[kW + i];
    before.x += (i < wave) ? sx : 0u;
    before.y += (i < wave) ? sy : 0u;
    all.x += sx;
    all.y += sy;
  }
  *total = all;
  return make_uint2(before.x + x - v.x, before.y + y - v.y);
}

// Largest bin B of hist[0..nbins) with (count of bins >= B) >= need, and the
// count of bins > B, written to out[0], out[1]; requires 1 <= need <= total.
template <int NT>
__device__ void find_threshold_bin(const uint32_t* hist, int nbins, uint32_t need, uint32_t* wave_sum,
                                   uint32_t* out) {
  const int per = (nbins + NT - 1) / NT;
  const int t = threadIdx.x;
  const int hi = nbins - t * per;  // thread t owns bins [hi - per, hi), top bins first
  const int lo = hi - per > 0 ? hi - per : 0;
  uint32_t mine = 0;
  for (int i = lo; i < hi; ++i) mine += hist[i];
  uint32_t total;
  const uint32_t above = block_exclusive_scan<NT>(hi > 0 ? mine : 0u, wave_sum, &total);
  if (hi > 0 && above < need && above + mine >= need) {
    uint32_t acc = above;
    for (int i = hi - 1; i >= lo; --i) {
      if (acc + hist[i] >= need) {
        out[0] = (uint32_t)i;
        out[1] = acc;
        break;
      }
      acc += hist[i];
    }
  }
  __syncthreads();
}

// find_threshold_bin in two barriers: wave_sum (NT / 64 words) is owned by
// the call site and never reused in the workgroup.
template <int NT>
__device__ void find_threshold_bin_once(const uint32_t* hist, int nbins, uint32_t need, uint32_t* wave_sum,
                                        uint32_t* out) {
  const int per = (nbins + NT - 1) / NT;
  const int t = threadIdx.x;
  const int hi = nbins - t * per;
  const int lo = hi - per > 0 ? hi - per : 0;
  uint32_t mine = 0;
  for (int i = lo; i < hi; ++i) mine += hist[i];
  uint32_t total;
  const uint32_t above = block_exclusive_scan_once<NT>(hi > 0 ? mine : 0u, wave_sum, &total);
  if (hi > 0 && above < need && above + mine >= need) {
    uint32_t acc = above;
    for (int i = hi - 1; i >= lo; --i) {
      if (acc + hist[i] >= need) {
        out[0] = (uint32_t)i;
        out[1] = acc;
        break;
      }
      acc += hist[i];
    }
  }
  __syncthreads();
}

// Largest (smallest) of a wavefront's 64 values, on VALU moves: DPP quad_perm swaps of
// neighbours and pairs, row_half_mirror and row_mirror (lane i with 7 - i
// and 15 - i of its 8 / 16 lanes), then v_permlane16_swap / 32_swap.
template <bool kMax>
__device__ __forceinline__ uint32_t wave_reduce_u32(uint32_t v) {
  auto op = [](uint32_t a, uint32_t b) { return kMax ? max(a, b) : min(a, b); };
  int x = (int)v;
  x = (int)op((uint32_t)x, (uint32_t)__builtin_amdgcn_mov_dpp(x, 0xB1, 0xF, 0xF, false));   // quad_perm [1,0,3,2]
  x = (int)op((uint32_t)x, (uint32_t)__builtin_amdgcn_mov_dpp(x, 0x4E, 0xF, 0xF, false));   // quad_perm [2,3,0,1]
  x = (int)op((uint32_t)x, (uint32_t)__builtin_amdgcn_mov_dpp(x, 0x141, 0xF, 0xF, false));  // row_half_mirror
  x = (int)op((uint32_t)x, (uint32_t)__builtin_amdgcn_mov_dpp(x, 0x140, 0xF, 0xF, false));  // row_mirror
  const auto r16 = __builtin_amdgcn_permlane16_swap((uint32_t)x, (uint32_t)x, false, false);
  x = (int)op((uint32_t)r16[0], (uint32_t)r16[1]);
  const auto r32 = __builtin_amdgcn_permlane32_swap((uint32_t)x, (uint32_t)x, false, false);
  return op((uint32_t)r32[0], (uint32_t)r32[1]);
}
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) { return wave_reduce_u32<true>(v); }
__device__ __forceinline__ uint32_t wave_min_u32(uint32_t v) { return wave_reduce_u32<false>(v); }

// The score whose order key (order_key in topk_ws.hpp) is key != 0.
__device__ __forceinline__ float order_key_value(uint32_t key) {
  return __builtin_bit_cast(float, (key & 0x80000000u) ? (key & 0x7FFFFFFFu) : ~key);
}

}  // namespace csa2
