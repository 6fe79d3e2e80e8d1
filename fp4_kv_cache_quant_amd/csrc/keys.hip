// Indexer-key and block-key maintenance on append.
//
// [P1 "Compressed Sparse Attention 2 (CSA2)"]: a Full layer projects indexer
// K for its positions, and the hierarchical indexer keeps a pool of blocks
// of 8 positions, which needs a key per block; the pages do not say how a
// block key is formed.  READING: the sum of the indexer keys of the block's
// existing positions, in bf16.  A bulk kernel forms the keys of the blocks
// of a prefilled cache; the append kernel writes an appended position's
// indexer key and adds it to its block's key (the first position of a
// block starts it).  The running sum is rounded to bf16 after every add,
// which equals the once-rounded sum whenever the partial sums are exact in
// bf16 (integer-valued keys with |sum| <= 256).
//
// Citation key: [P1] "DeepSeek AI Released DeepSeek-V4.1-Flash with 1M
// Context, FP4 KV Cache, and Cross-Layer Attention Reuse".
#include "common.hpp"

namespace csa2 {
namespace {

// One thread per (block, dimension): blk_k[b][j][d] = bf16(sum of the keys
// of positions blk*j .. blk*j+blk-1 below lens[b]); blocks at or past
// ceil(lens[b]/blk) are written as 0.
__global__ __launch_bounds__(256) void block_keys_kernel(const uint16_t* __restrict__ idx_k, int64_t key_cap,
                                                         const int32_t* __restrict__ lens, int32_t blk,
                                                         uint16_t* __restrict__ blk_k, int64_t blk_cap) {
  const int b = blockIdx.y;
  const int64_t t = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (t >= blk_cap * CSA2_IDX_DIM) return;
  const int64_t j = t / CSA2_IDX_DIM;
  const int d = (int)(t % CSA2_IDX_DIM);
  const int64_t L = min((int64_t)lens[b], key_cap);
  const uint16_t* kb = idx_k + (int64_t)b * key_cap * CSA2_IDX_DIM;
  float acc = 0.f;
  for (int i = 0; i < blk; ++i) {
    const int64_t p = j * blk + i;
    if (p < L) acc += bf16_to_f32(kb[p * CSA2_IDX_DIM + d]);
  }
  blk_k[((int64_t)b * blk_cap + j) * CSA2_IDX_DIM + d] = (uint16_t)f32_to_bf16_rne(acc);
}

// One 64-thread workgroup per sequence, one thread per dimension.  The
// position is lens[b] (read before the latent append advances it).
__global__ __launch_bounds__(64) void append_keys_kernel(const uint16_t* __restrict__ new_k,
                                                         uint16_t* __restrict__ idx_k, int64_t key_cap,
                                                         uint16_t* __restrict__ blk_k, int64_t blk_cap,
                                                         int32_t blk, const int32_t* __restrict__ lens,
                                                         int32_t* __restrict__ err_flag) {
  const int b = blockIdx.x, d = threadIdx.x;
  const int64_t row = lens[b];
  const int64_t j = row / blk;
  if (row < 0 || row >= key_cap || (blk_k && j >= blk_cap)) {
    if (d == 0 && err_flag) atomicOr(err_flag, 2);
    return;
  }
  const uint16_t k = new_k[(int64_t)b * CSA2_IDX_DIM + d];
  idx_k[((int64_t)b * key_cap + row) * CSA2_IDX_DIM + d] = k;
  if (blk_k) {
    uint16_t* bk = blk_k + ((int64_t)b * blk_cap + j) * CSA2_IDX_DIM + d;
    *bk = (row % blk == 0) ? k : (uint16_t)f32_to_bf16_rne(bf16_to_f32(*bk) + bf16_to_f32(k));
  }
}

}  // namespace

csa2_status block_keys_launch(const uint16_t* idx_k, int64_t key_cap, const int32_t* lens, int32_t blk,
                              uint16_t* blk_k, int64_t blk_cap, int32_t n_seq, hipStream_t stream) {
  if (n_seq == 0 || blk_cap == 0) return CSA2_OK;
  const int64_t blocks = (blk_cap * CSA2_IDX_DIM + 255) / 256;
  CSA2_REQUIRE(blocks <= 0x7FFFFFFF && n_seq <= 65535, CSA2_ESHAPE, "csa2_block_keys: too large for one launch");
  hipLaunchKernelGGL(block_keys_kernel, dim3((uint32_t)blocks, n_seq), dim3(256), 0, stream, idx_k, key_cap, lens,
                     blk, blk_k, blk_cap);
  return launch_status("csa2_block_keys");
}

csa2_status append_keys_launch(const uint16_t* new_k, uint16_t* idx_k, int64_t key_cap, uint16_t* blk_k,
                               int64_t blk_cap, int32_t blk, const int32_t* lens, int32_t* err_flag, int32_t n_seq,
                               hipStream_t stream) {
  if (n_seq == 0) return CSA2_OK;
  hipLaunchKernelGGL(append_keys_kernel, dim3(n_seq), dim3(64), 0, stream, new_k, idx_k, key_cap, blk_k, blk_cap,
                     blk, lens, err_flag);
  return launch_status("csa2_append_index_keys");
}

}  // namespace csa2
