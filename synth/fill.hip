// Device side of the seeded synthetic-input generator (see synth/__init__.py).
//
// Element i of tensor `tid` is the (i+1)-th output of Vigna's splitmix64
// generator whose state starts at mix((seed << 32) ^ tid).  Row-structured
// tensors use the flat index ((b << 24) + row) * dim + d.  INT9 maps the
// output h to (h mod 9) - 4 as bf16; NORMAL maps it to ntab[h >> 48], a table
// built and uploaded by the host.  No step of the attention method lives here.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

__host__ __device__ inline uint64_t mix64(uint64_t z) {
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
  return z ^ (z >> 31);
}

__constant__ uint16_t kInt9Bf16[9] = {0xC080, 0xC040, 0xC000, 0xBF80, 0x0000,
                                      0x3F80, 0x4000, 0x4040, 0x4080};

__global__ void fill_rows_kernel(uint16_t* __restrict__ dst, int64_t bstride, int64_t rstride,
                                 int32_t nb, int64_t n_rows, int32_t dim, int32_t b0,
                                 int64_t row0, uint64_t key, int32_t kind,
                                 const uint16_t* __restrict__ ntab) {
  const int64_t per_b = n_rows * dim;
  const int64_t total = per_b * nb;
  for (int64_t e = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; e < total;
       e += (int64_t)gridDim.x * blockDim.x) {
    const int64_t bi = e / per_b;
    const int64_t rem = e - bi * per_b;
    const int64_t r = rem / dim;
    const int64_t d = rem - r * dim;
    const uint64_t idx = ((((uint64_t)(b0 + bi)) << 24) + (uint64_t)(row0 + r)) * (uint64_t)dim + (uint64_t)d;
    const uint64_t h = mix64(key + (idx + 1) * 0x9E3779B97F4A7C15ull);
    const uint16_t v = (kind == 0) ? kInt9Bf16[h % 9] : ntab[h >> 48];
    dst[bi * bstride + r * rstride + d] = v;
  }
}

}  // namespace

extern "C" int32_t synth_fill_rows(void* dst, int64_t bstride, int64_t rstride, int32_t nb,
                                   int64_t n_rows, int32_t dim, int32_t b0, int64_t row0,
                                   uint64_t seed, uint32_t tid, int32_t kind, const void* ntab,
                                   hipStream_t stream) {
  if (!dst || nb < 0 || n_rows < 0 || dim <= 0 || b0 < 0 || row0 < 0) return -1;
  if (kind != 0 && kind != 1) return -1;
  if (kind == 1 && !ntab) return -1;
  if (seed >= (1ull << 32)) return -1;
  const int64_t total = (int64_t)nb * n_rows * dim;
  if (total == 0) return 0;
  const uint64_t key = mix64((seed << 32) ^ (uint64_t)tid);
  int64_t blocks = (total + 255) / 256;
  if (blocks > 65536) blocks = 65536;
  hipLaunchKernelGGL(fill_rows_kernel, dim3((unsigned)blocks), dim3(256), 0, stream,
                     (uint16_t*)dst, bstride, rstride, nb, n_rows, dim, b0, row0, key, kind,
                     (const uint16_t*)ntab);
  return hipGetLastError() == hipSuccess ? 0 : -2;
}
