/*
 * csa2_oracle.c -- TEST INFRASTRUCTURE.  The plain, slow CPU oracle of the
 * CSA2 FP4-KV decode path.  Only the tests, the smoke check and the
 * benchmark's CPU-baseline leg may load it; the product library never does,
 * and it shares no code, header or table with the HIP path.
 *
 * Every function is written from the definition of what it computes, scalar,
 * without blocking or reordering, so that it can be checked by eye.  Floating
 * point is double, rounded once to binary32 where a result is stored as
 * binary32; the quantiser compares exact products.
 *
 * Citations name the page and its section:
 *   [P1] "DeepSeek AI Released DeepSeek-V4.1-Flash with 1M Context, FP4 KV
 *        Cache, and Cross-Layer Attention Reuse" (thecryptopost.io)
 *   [P3] "DeepSeek-V4.1 Flash: Pushing the Limits of KV Cache Compression"
 *        (tldrocket.com)
 *   [P4] "DeepSeek-V4.1-Flash: Pushing the Limits of KV Cache Compression"
 *        (agihunt.info paper page 2609.19969), summary
 *
 * Readings taken where the pages are silent are marked READING and are the
 * same ones the library documents in its header.
 *
 * Build: gcc -O2 -std=c11 -ffp-contract=off -fno-fast-math -shared -fPIC
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define D_LATENT 512   /* [P3]: a 512-dimensional latent shared by key and value */
#define GROUP 16       /* [P1 "FP4 KV, ..."]: one E4M3 scale per 16 channels */
#define N_GROUPS (D_LATENT / GROUP)
#define CODE_BYTES (D_LATENT / 2)
#define IDX_HEADS 8
#define IDX_DIM 64
#define MAIN_HEADS 16

/* ---------------------------------------------------------------- formats */

/* bf16: the upper 16 bits of an IEEE binary32. */
double orc_bf16_value(uint16_t b) {
  uint32_t u = (uint32_t)b << 16;
  float f;
  memcpy(&f, &u, sizeof f);
  return (double)f;
}

/* E4M3 (OCP 8-bit float "E4M3FN"): sign, 4 exponent bits with bias 7,
 * 3 mantissa bits; exponent field 0 is subnormal; no infinities; the
 * all-ones exponent with all-ones mantissa is NaN.  [P1 "FP4 KV, ..."]:
 * the per-16-channel scale is E4M3. READING: the OCP FN variant. */
double orc_e4m3_value(uint8_t c) {
  int s = (c >> 7) & 1, e = (c >> 3) & 15, m = c & 7;
  double v;
  if (e == 15 && m == 7) return NAN;
  if (e == 0)
    v = ldexp((double)m / 8.0, -6);
  else
    v = ldexp(1.0 + (double)m / 8.0, e - 7);
  return s ? -v : v;
}

/* E2M1 (4-bit float): sign, 2 exponent bits with bias 1, 1 mantissa bit;
 * exponent field 0 is subnormal (0 or 0.5).  [P1 "FP4 KV, ..."]. */
double orc_e2m1_value(uint8_t c) {
  int s = (c >> 3) & 1, e = (c >> 1) & 3, m = c & 1;
  double v;
  if (e == 0)
    v = 0.5 * (double)m;
  else
    v = ldexp(1.0 + (double)m / 2.0, e - 1);
  return s ? -v : v;
}

/* Round num/den to the nearest of the ascending values vals[0..n-1],
 * ties to the even index, saturating past the last value.  Compares num
 * with den * (midpoint of two neighbours); both operands of every
 * comparison are exact doubles (short significands), so the result is the
 * exact round-to-nearest-even of the rational num/den. */
static int nearest_even_index(double num, double den, const double* vals, int n) {
  for (int c = 0; c + 1 < n; ++c) {
    double mid = den * (0.5 * (vals[c] + vals[c + 1]));
    if (num < mid) return c;
    if (num == mid) return (c % 2 == 0) ? c : c + 1;
  }
  return n - 1;
}

static double g_e4m3_pos[127]; /* codes 0x00..0x7E, ascending */
static double g_e2m1_pos[8];   /* codes 0..7, ascending */

/* Filled once when the library is loaded, before any thread can call in. */
__attribute__((constructor)) static void tables_init(void) {
  for (int c = 0; c < 127; ++c) g_e4m3_pos[c] = orc_e4m3_value((uint8_t)c);
  for (int c = 0; c < 8; ++c) g_e2m1_pos[c] = orc_e2m1_value((uint8_t)c);
}

/* Scale code of one 16-channel group with absolute maximum `amax`:
 * E4M3 round-to-nearest-even of amax / 6 (6 = the largest E2M1 magnitude,
 * the NVFP4 convention that [P1 "FP4 KV, ..."] says is followed, without
 * its second-level global scale).  Saturates at 448. */
uint8_t orc_scale_code(double amax) {
  return (uint8_t)nearest_even_index(amax, 6.0, g_e4m3_pos, 127);
}

/* E2M1 code of one value x under the group scale s: magnitude is
 * round-to-nearest-even of |x| / s onto {0,0.5,1,1.5,2,3,4,6}, saturating at
 * 6; the sign bit is the sign bit of x (READING: also for magnitude 0).
 * A zero scale gives magnitude 0.  `neg` is the sign bit of x. */
uint8_t orc_e2m1_code(double absx, int neg, double s) {
  int m = 0;
  if (s > 0.0) m = nearest_even_index(absx, s, g_e2m1_pos, 8);
  return (uint8_t)((neg ? 8 : 0) | m);
}

/* Quantise one 512-channel bf16 latent row [P1 "FP4 KV, ..."]:
 * 32 groups of 16 channels, one E4M3 scale byte per group, one E2M1 code per
 * channel.  READING (byte layout, not on the pages): code byte j holds
 * channel 2j in its low nibble and channel 2j+1 in its high nibble; scale
 * byte g belongs to channels 16g..16g+15. */
void orc_quant_row(const uint16_t* x, uint8_t* codes, uint8_t* scales) {
  uint8_t c[D_LATENT];
  for (int g = 0; g < N_GROUPS; ++g) {
    double amax = 0.0;
    for (int i = 0; i < GROUP; ++i) {
      double a = fabs(orc_bf16_value(x[g * GROUP + i]));
      if (a > amax) amax = a;
    }
    uint8_t sc = orc_scale_code(amax);
    double s = orc_e4m3_value(sc);
    scales[g] = sc;
    for (int i = 0; i < GROUP; ++i) {
      uint16_t b = x[g * GROUP + i];
      c[g * GROUP + i] = orc_e2m1_code(fabs(orc_bf16_value(b)), (b >> 15) & 1, s);
    }
  }
  for (int j = 0; j < CODE_BYTES; ++j) codes[j] = (uint8_t)(c[2 * j] | (c[2 * j + 1] << 4));
}

void orc_quant_rows(const uint16_t* x, int64_t n, uint8_t* codes, uint8_t* scales) {
  for (int64_t r = 0; r < n; ++r)
    orc_quant_row(x + r * D_LATENT, codes + r * CODE_BYTES, scales + r * N_GROUPS);
}

/* Dequantise one row: value = E2M1(code) * E4M3(scale) (exact). */
void orc_dequant_row(const uint8_t* codes, const uint8_t* scales, double* out) {
  for (int d = 0; d < D_LATENT; ++d) {
    uint8_t byte = codes[d / 2];
    uint8_t code = (d % 2 == 0) ? (byte & 15) : (byte >> 4);
    out[d] = orc_e2m1_value(code) * orc_e4m3_value(scales[d / GROUP]);
  }
}

/* ------------------------------------------------------------ indexer score */

/* Indexer score of one key [P1 "Compressed Sparse Attention 2 (CSA2)"]: the
 * pages name an indexer Q scored against indexer K but print no formula.
 * READING: per indexer head h, r_h = max(0, q_h . k); score = sum_h w_h r_h
 * (w == NULL: every w_h = 1), the real sum rounded once to binary32.
 * Every bf16 product is exact in double and so is each w_h r_h (a binary32
 * weight times an r_h of at most 17 significant bits for integer-valued
 * inputs); the double sums below are exact whenever the terms span fewer
 * than 53 bits, which holds for integer-valued q, k and for weights with
 * short significands -- the inputs for which the library claims exact
 * scores.  No order of summation is implied by the definition. */
float orc_index_score_one(const uint16_t* q, const float* w, const uint16_t* k) {
  double s = 0.0;
  for (int h = 0; h < IDX_HEADS; ++h) {
    double dot = 0.0;
    for (int d = 0; d < IDX_DIM; ++d)
      dot += orc_bf16_value(q[h * IDX_DIM + d]) * orc_bf16_value(k[d]);
    const double r = dot > 0.0 ? dot : 0.0;
    s += (w ? (double)w[h] : 1.0) * r;
  }
  return (float)s;
}

/* Scores of n keys given by row ids into a key array [*][64]. */
void orc_index_score(const uint16_t* q, const float* w, const uint16_t* keys,
                     const int64_t* ids, int64_t n, float* out) {
  for (int64_t i = 0; i < n; ++i) out[i] = orc_index_score_one(q, w, keys + ids[i] * IDX_DIM);
}

/* --------------------------------------------------------------- selection */

typedef struct {
  float score;
  int64_t id;
} cand_t;

/* Larger score first; equal scores (-0 == +0 under these comparisons): lower
 * id first (READING: ties go to the lower position; the pages give no tie
 * rule). */
static int cand_order(const void* pa, const void* pb) {
  const cand_t* a = (const cand_t*)pa;
  const cand_t* b = (const cand_t*)pb;
  if (a->score > b->score) return -1;
  if (a->score < b->score) return 1;
  return (a->id < b->id) ? -1 : (a->id > b->id) ? 1 : 0;
}

static int id_order(const void* pa, const void* pb) {
  int64_t a = *(const int64_t*)pa, b = *(const int64_t*)pb;
  return (a < b) ? -1 : (a > b) ? 1 : 0;
}

/* Top-k of n candidates [P1 "Compressed Sparse Attention 2 (CSA2)"]: keep the
 * min(k, #candidates) best by (score desc, id asc); write their ids ascending
 * into out[0..k-1], padding with -1 (READING: output order and padding).
 * READING (non-candidates): a NaN or -inf score never takes part -- it marks
 * a slot with nothing to select (a position past the sequence, an empty pool
 * block) -- and -0 equals +0.  Returns the number selected. */
int64_t orc_select(const float* scores, const int64_t* ids, int64_t n, int64_t k, int64_t* out) {
  cand_t* c = (cand_t*)malloc((size_t)(n > 0 ? n : 1) * sizeof(cand_t));
  int64_t m = 0;
  for (int64_t i = 0; i < n; ++i) {
    if (isnan(scores[i]) || scores[i] == -INFINITY) continue;
    c[m].score = scores[i];
    c[m].id = ids[i];
    ++m;
  }
  const int64_t take = m < k ? m : k;
  qsort(c, (size_t)m, sizeof(cand_t), cand_order);
  for (int64_t i = 0; i < take; ++i) out[i] = c[i].id;
  qsort(out, (size_t)take, sizeof(int64_t), id_order);
  for (int64_t i = take; i < k; ++i) out[i] = -1;
  free(c);
  return take;
}

/* Flat Full layer [P1 "Compressed Sparse Attention 2 (CSA2)"]: score all L
 * positions with the layer's indexer Q and select a fresh Top-k. */
int64_t orc_flat_select(const uint16_t* q, const float* w, const uint16_t* tok_keys, int64_t L,
                        int64_t k, int64_t* out) {
  int64_t* ids = (int64_t*)malloc((size_t)(L > 0 ? L : 1) * sizeof(int64_t));
  float* sc = (float*)malloc((size_t)(L > 0 ? L : 1) * sizeof(float));
  for (int64_t i = 0; i < L; ++i) ids[i] = i;
  orc_index_score(q, w, tok_keys, ids, L, sc);
  int64_t r = orc_select(sc, ids, L, k, out);
  free(ids);
  free(sc);
  return r;
}

/* Pool of a hierarchical Full layer [P1 "Compressed Sparse Attention 2
 * (CSA2)"]: the decoder's Full layer builds a candidate pool of up to
 * n_pool_blocks blocks of `blk` positions.  Block b covers positions
 * blk*b .. blk*b+blk-1 and is a candidate iff blk*b < L (READING: a partial
 * last block is a candidate).  Blocks are ranked by their block key's score
 * (READING: block keys are given inputs).  Writes the kept block ids
 * ascending, -1 padded. */
int64_t orc_pool_blocks(const uint16_t* q, const float* w, const uint16_t* blk_keys, int64_t L,
                        int64_t blk, int64_t n_pool_blocks, int64_t* pool_out) {
  int64_t nb = (L + blk - 1) / blk;
  return orc_flat_select(q, w, blk_keys, nb, n_pool_blocks, pool_out);
}

/* Token-level selection inside a pool: the candidates are the positions
 * blk*b + j (j < blk) of every pool block b >= 0 that lie below L; each is
 * scored with the given indexer Q on the token indexer K.  Used by the
 * hierarchical Full layer (its own Q) and by Reindex layers (their own Q,
 * [P1 "Compressed Sparse Attention 2 (CSA2)"]: rescore with own indexer Q). */
int64_t orc_pool_select(const uint16_t* q, const float* w, const uint16_t* tok_keys, int64_t L,
                        const int64_t* pool, int64_t n_pool_blocks, int64_t blk, int64_t k,
                        int64_t* out) {
  int64_t cap = n_pool_blocks * blk, n = 0;
  int64_t* ids = (int64_t*)malloc((size_t)(cap > 0 ? cap : 1) * sizeof(int64_t));
  float* sc = (float*)malloc((size_t)(cap > 0 ? cap : 1) * sizeof(float));
  for (int64_t p = 0; p < n_pool_blocks; ++p) {
    if (pool[p] < 0) continue;
    for (int64_t j = 0; j < blk; ++j) {
      int64_t pos = pool[p] * blk + j;
      if (pos < L) ids[n++] = pos;
    }
  }
  orc_index_score(q, w, tok_keys, ids, n, sc);
  int64_t r = orc_select(sc, ids, n, k, out);
  free(ids);
  free(sc);
  return r;
}

/* ---------------------------------------------------------------- attention */

/* Sparse + SWA attention of one query token in one layer.
 * [P1 "Compressed Sparse Attention 2 (CSA2)"]: each layer attends with its
 * own main Q over the selected main-KV positions; [P1 "Causal
 * Encoder-Decoder: Half the Prefill"]: a 128-token sliding window runs in
 * every layer; [P3]: keys and values share one 512-d latent.
 * The attended set is the dequantised rows idx[i] >= 0 of the FP4 cache
 * (codes [*][256], scales [*][32]) followed by the first swa_len bf16 SWA rows
 * (READING: one softmax over the concatenation, no de-duplication).
 * For each head h: z_j = sm_scale * (q_h . x_j), p = softmax(z),
 * o_h = sum_j p_j x_j, rounded to binary32.  An empty set gives o_h = 0. */
/* Attention of 16 heads over n value rows x [n][512] (double): for each
 * head h, z_j = sm_scale * (q_h . x_j), p = softmax(z), o_h = sum_j p_j x_j,
 * rounded to binary32; an empty set gives o_h = 0. */
static void attn_over_rows(const uint16_t* q, const double* x, int64_t n, double sm_scale, float* out) {
  double* z = (double*)malloc((size_t)(n > 0 ? n : 1) * sizeof(double));
  for (int h = 0; h < MAIN_HEADS; ++h) {
    double zmax = -INFINITY, denom = 0.0;
    for (int64_t j = 0; j < n; ++j) {
      double dot = 0.0;
      for (int d = 0; d < D_LATENT; ++d) dot += orc_bf16_value(q[h * D_LATENT + d]) * x[j * D_LATENT + d];
      z[j] = sm_scale * dot;
      if (z[j] > zmax) zmax = z[j];
    }
    for (int64_t j = 0; j < n; ++j) {
      z[j] = exp(z[j] - zmax);
      denom += z[j];
    }
    for (int d = 0; d < D_LATENT; ++d) {
      double acc = 0.0;
      for (int64_t j = 0; j < n; ++j) acc += z[j] * x[j * D_LATENT + d];
      out[h * D_LATENT + d] = (n > 0) ? (float)(acc / denom) : 0.0f;
    }
  }
  free(z);
}

/* The selected rows idx[i] >= 0 of the FP4 cache, dequantised, into x;
 * returns how many. */
static int64_t gather_rows(const uint8_t* codes, const uint8_t* scales, const int64_t* idx, int64_t n_idx,
                           double* x) {
  int64_t r = 0;
  for (int64_t i = 0; i < n_idx; ++i) {
    if (idx[i] < 0) continue;
    orc_dequant_row(codes + idx[i] * CODE_BYTES, scales + idx[i] * N_GROUPS, x + r * D_LATENT);
    ++r;
  }
  return r;
}

static int64_t count_selected(const int64_t* idx, int64_t n_idx) {
  int64_t n_sel = 0;
  for (int64_t i = 0; i < n_idx; ++i) n_sel += idx[i] >= 0;
  return n_sel;
}

void orc_sparse_attn(const uint16_t* q, const uint8_t* codes, const uint8_t* scales,
                     const int64_t* idx, int64_t n_idx, const uint16_t* swa, int64_t swa_len,
                     double sm_scale, float* out) {
  const int64_t n = count_selected(idx, n_idx) + (swa_len > 0 ? swa_len : 0);
  double* x = (double*)malloc((size_t)(n > 0 ? n : 1) * D_LATENT * sizeof(double));
  int64_t r = gather_rows(codes, scales, idx, n_idx, x);
  for (int64_t j = 0; j < swa_len; ++j, ++r)
    for (int d = 0; d < D_LATENT; ++d) x[r * D_LATENT + d] = orc_bf16_value(swa[j * D_LATENT + d]);
  attn_over_rows(q, x, n, sm_scale, out);
  free(x);
}

/* ------------------------------------------------ context-parallel shares */

/* One rank's share of steps (d)+(e) when the attended rows are split over
 * ranks (one sequence longer than a GPU holds: each rank holds some of the
 * selected rows, the rank with the tail also the window).  READING (the
 * pages do not describe a split): the share is the unnormalised softmax
 * over the rank's rows in base-2 units, per head h:
 *   z_j = sm_scale * log2(e) * (q_h . x_j),  m_h = max_j z_j,
 *   l_h = sum_j 2^(z_j - m_h),  o_h = sum_j 2^(z_j - m_h) x_j,
 * and an empty share is m = -inf, l = 0, o = 0.  o [16][512], ml [16][2]
 * (m, l), both double.  The rows are those of orc_sparse_attn. */
void orc_sparse_attn_partial(const uint16_t* q, const uint8_t* codes, const uint8_t* scales,
                             const int64_t* idx, int64_t n_idx, const uint16_t* swa, int64_t swa_len,
                             double sm_scale, double* o, double* ml) {
  const double log2e = 1.0 / log(2.0);
  const int64_t n = count_selected(idx, n_idx) + (swa_len > 0 ? swa_len : 0);
  double* x = (double*)malloc((size_t)(n > 0 ? n : 1) * D_LATENT * sizeof(double));
  double* z = (double*)malloc((size_t)(n > 0 ? n : 1) * sizeof(double));
  int64_t r = gather_rows(codes, scales, idx, n_idx, x);
  for (int64_t j = 0; j < swa_len; ++j, ++r)
    for (int d = 0; d < D_LATENT; ++d) x[r * D_LATENT + d] = orc_bf16_value(swa[j * D_LATENT + d]);
  for (int h = 0; h < MAIN_HEADS; ++h) {
    double m = -INFINITY, l = 0.0;
    for (int64_t j = 0; j < n; ++j) {
      double dot = 0.0;
      for (int d = 0; d < D_LATENT; ++d) dot += orc_bf16_value(q[h * D_LATENT + d]) * x[j * D_LATENT + d];
      z[j] = sm_scale * log2e * dot;
      if (z[j] > m) m = z[j];
    }
    for (int64_t j = 0; j < n; ++j) {
      z[j] = exp2(z[j] - m);
      l += z[j];
    }
    for (int d = 0; d < D_LATENT; ++d) {
      double acc = 0.0;
      for (int64_t j = 0; j < n; ++j) acc += z[j] * x[j * D_LATENT + d];
      o[h * D_LATENT + d] = acc;
    }
    ml[2 * h] = m;
    ml[2 * h + 1] = l;
  }
  free(z);
  free(x);
}

/* The softmax over the union of n_parts shares (the arithmetic after the
 * ranks exchange them): per head, M = max_s m_s, then
 *   out = sum_s 2^(m_s - M) o_s / sum_s 2^(m_s - M) l_s,
 * shares with m_s = -inf contributing nothing; no rows at all gives 0.
 * o [n_parts][16][512], ml [n_parts][16][2]; out [16][512] float. */
void orc_attn_merge(const double* o, const double* ml, int64_t n_parts, float* out) {
  for (int h = 0; h < MAIN_HEADS; ++h) {
    double M = -INFINITY;
    for (int64_t s = 0; s < n_parts; ++s)
      if (ml[(s * MAIN_HEADS + h) * 2] > M) M = ml[(s * MAIN_HEADS + h) * 2];
    double den = 0.0;
    for (int64_t s = 0; s < n_parts; ++s) {
      const double ms = ml[(s * MAIN_HEADS + h) * 2];
      if (ms != -INFINITY) den += exp2(ms - M) * ml[(s * MAIN_HEADS + h) * 2 + 1];
    }
    for (int d = 0; d < D_LATENT; ++d) {
      double acc = 0.0;
      for (int64_t s = 0; s < n_parts; ++s) {
        const double ms = ml[(s * MAIN_HEADS + h) * 2];
        if (ms != -INFINITY) acc += exp2(ms - M) * o[(s * MAIN_HEADS + h) * D_LATENT + d];
      }
      out[h * D_LATENT + d] = den > 0.0 ? (float)(acc / den) : 0.0f;
    }
  }
}

/* ------------------------------------------------------------ FP8 window */

/* [P4] summary: the sliding-window KV is kept in FP8.  READING: OCP E4M3FN
 * elements, one byte per channel, no scale: the E4M3 round-to-nearest-even
 * of the bf16 value with ties to the even code, saturating at +-448; the
 * sign bit is copied (also for zero); NaN stays NaN (S.1111.111). */
uint8_t orc_fp8_code(uint16_t b) {
  const double x = orc_bf16_value(b);
  const int neg = (b >> 15) & 1;
  if (isnan(x)) return (uint8_t)((neg << 7) | 0x7F);
  return (uint8_t)((neg << 7) | nearest_even_index(fabs(x), 1.0, g_e4m3_pos, 127));
}

void orc_fp8_rows(const uint16_t* x, int64_t n_rows, uint8_t* out) {
  for (int64_t i = 0; i < n_rows * D_LATENT; ++i) out[i] = orc_fp8_code(x[i]);
}

/* orc_sparse_attn with FP8 window rows: window row j's channel d is
 * E4M3(swa8[j][d]) (exact). */
void orc_sparse_attn_fp8w(const uint16_t* q, const uint8_t* codes, const uint8_t* scales,
                          const int64_t* idx, int64_t n_idx, const uint8_t* swa8, int64_t swa_len,
                          double sm_scale, float* out) {
  const int64_t n = count_selected(idx, n_idx) + (swa_len > 0 ? swa_len : 0);
  double* x = (double*)malloc((size_t)(n > 0 ? n : 1) * D_LATENT * sizeof(double));
  int64_t r = gather_rows(codes, scales, idx, n_idx, x);
  for (int64_t j = 0; j < swa_len; ++j, ++r)
    for (int d = 0; d < D_LATENT; ++d) x[r * D_LATENT + d] = orc_e4m3_value(swa8[j * D_LATENT + d]);
  attn_over_rows(q, x, n, sm_scale, out);
  free(x);
}

/* ------------------------------------------------- block-key maintenance */

/* Key of block b (positions blk*b .. blk*b + blk-1) over the first L
 * positions of indexer K tok_keys [*][64].  The pages say the hierarchical
 * pool needs a key per block of 8 but not how it is formed ([P1 "Compressed
 * Sparse Attention 2 (CSA2)"]).  READING: the sum of the indexer keys of the
 * block's positions that exist (< L), rounded once to bf16 (RNE); for
 * integer-valued keys with |sum| <= 256 the sum is exact. */
void orc_block_key(const uint16_t* tok_keys, int64_t L, int64_t blk, int64_t b, uint16_t* out) {
  for (int d = 0; d < IDX_DIM; ++d) {
    double acc = 0.0;
    for (int64_t i = blk * b; i < blk * (b + 1) && i < L; ++i) acc += orc_bf16_value(tok_keys[i * IDX_DIM + d]);
    float f = (float)acc;
    uint32_t u;
    memcpy(&u, &f, sizeof u);
    u = (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16; /* RNE to bf16 (finite) */
    out[d] = (uint16_t)u;
  }
}
