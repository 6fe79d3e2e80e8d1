/* Host side of the seeded synthetic-input generator (see synth/__init__.py):
 * the same splitmix64 stream and value maps as synth/fill.hip and the numpy
 * definition, in plain C for speed.  No step of the attention method. */
#include <stdint.h>

static uint64_t mix64(uint64_t z) {
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
  return z ^ (z >> 31);
}

static const uint16_t kInt9Bf16[9] = {0xC080, 0xC040, 0xC000, 0xBF80, 0x0000,
                                      0x3F80, 0x4000, 0x4040, 0x4080};

/* out[bi][ri][d] = value at flat index ((bs[bi] << 24) + rows[ri]) * dim + d. */
void synth_gen_rows_host(uint64_t key, int32_t kind, const int64_t* bs, int64_t nb, const int64_t* rows,
                         int64_t nr, int32_t dim, const uint16_t* ntab, uint16_t* out) {
  for (int64_t bi = 0; bi < nb; ++bi)
    for (int64_t ri = 0; ri < nr; ++ri) {
      const uint64_t base = (((uint64_t)bs[bi] << 24) + (uint64_t)rows[ri]) * (uint64_t)dim;
      uint16_t* o = out + (bi * nr + ri) * dim;
      for (int32_t d = 0; d < dim; ++d) {
        const uint64_t h = mix64(key + (base + (uint64_t)d + 1) * 0x9E3779B97F4A7C15ull);
        o[d] = kind == 0 ? kInt9Bf16[h % 9] : ntab[h >> 48];
      }
    }
}
