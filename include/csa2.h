/*
 * csa2.h -- C ABI of the CSA2 FP4-KV decode path for AMD Instinct MI355X
 * (gfx950).
 *
 * The path (one decode step of a stack of CSA2 layers):
 *   (a) append a 512-d latent row to the FP4 main KV cache (E2M1 values, one
 *       E4M3 scale per 16 channels);
 *   (b) score an indexer query against indexer keys;
 *   (c) keep the Top-K positions, under the static Full / Reindex / Reuse
 *       layer modes and the hierarchical pool of 2,048 blocks of 8;
 *   (d) gather and dequantise the selected FP4 rows;
 *   (e) attend over them together with the layer's bf16 128-row sliding
 *       window, with online softmax.
 *
 * Citations name the page and its section:
 *   [P1] "DeepSeek AI Released DeepSeek-V4.1-Flash with 1M Context, FP4 KV
 *        Cache, and Cross-Layer Attention Reuse" (thecryptopost.io)
 *   [P3] "DeepSeek-V4.1 Flash: Pushing the Limits of KV Cache Compression"
 *        (tldrocket.com)
 *   [P4] "DeepSeek-V4.1-Flash: Pushing the Limits of KV Cache Compression"
 *        (agihunt.info paper page 2609.19969), summary
 *
 * Conventions for every call:
 *   - Pointers to tensors are DEVICE pointers owned by the caller; the
 *     library never frees them.  Arrays of pointers inside descriptors are
 *     host memory.  Shapes are given in the comments, row-major, last index
 *     contiguous.  bf16 values travel as uint16_t bit patterns.
 *   - `stream` is a hipStream_t passed as void* (NULL = the null stream).
 *     Every call only enqueues work on that stream, never synchronises the
 *     host, and allocates nothing, except csa2_sched_create/_destroy and
 *     csa2_sched_check.  Calls are therefore capturable in a HIP graph.
 *   - Return value: CSA2_OK (0) or a negative csa2_status.  On error nothing
 *     was enqueued and csa2_last_error() returns a message (thread-local).
 *     Argument errors are detected on the host; device-side conditions
 *     (appending past capacity) are reported through a device flag.
 *   - Numerics: quantised bytes, scores of integer-valued indexer inputs and
 *     selected indices are exact and deterministic.  Attention runs on f16
 *     matrix-core inputs with fp32 accumulation: dequantised FP4 values are
 *     exact in f16; main Q and window rows are rounded to f16 toward zero
 *     (exact for |x| in [2^-14, 65504]; larger magnitudes saturate).
 */
#ifndef CSA2_H
#define CSA2_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef int32_t csa2_status;
#define CSA2_OK 0
#define CSA2_EINVAL (-1)    /* null pointer or invalid argument value */
#define CSA2_ESHAPE (-2)    /* a size outside what the call supports */
#define CSA2_ECAPACITY (-3) /* a buffer is too small */
#define CSA2_EMODE (-4)     /* invalid layer table */
#define CSA2_EHIP (-5)      /* the HIP runtime reported an error */
#define CSA2_ENOMEM (-6)    /* device allocation failed (create only) */

#define CSA2_LATENT 512     /* [P3]: 512-d latent shared by key and value */
#define CSA2_GROUP 16       /* [P1 "FP4 KV, ..."]: one scale per 16 channels */
#define CSA2_CODE_BYTES 256 /* 512 E2M1 codes, two per byte */
#define CSA2_SCALE_BYTES 32 /* 32 E4M3 scales */
#define CSA2_HEADS 16       /* main query heads */
#define CSA2_IDX_HEADS 8    /* indexer heads */
#define CSA2_IDX_DIM 64     /* indexer head dimension */
#define CSA2_SWA_MAX 128    /* [P1 "Causal Encoder-Decoder..."]: 128-token window */
#define CSA2_TOPK_MAX 2048  /* largest k of one csa2_topk call */
#define CSA2_TOPK_NMAX 1048576 /* most candidates per sequence of one csa2_topk call */

/* Message of the last failing call on this thread ("" if none). */
const char* csa2_last_error(void);
/* Version of this ABI (bumped on any signature or struct change; 2 added
 * the FP8 window, 3 the key maintenance on append, 4 the per-layer indexer
 * K of flat Full layers and csa2_flat_select, 5 the stream argument of
 * csa2_sched_check, the per-step window rows of csa2_step_io and
 * csa2_pool_select; 6 csa2_prefill_select; 7 csa2_sparse_attn_partial
 * and csa2_attn_merge). */
int32_t csa2_abi_version(void);

/* ------------------------------------------------------------ FP4 cache
 * One FP4 main-KV tensor [P1 "FP4 KV, Bounded Replay, and Other
 * Extensions"]: E2M1 elements with one E4M3 (OCP E4M3FN) scale per 16
 * channels, no second-level scale.  Planar layout:
 *   codes  [n_seq][cap][256] uint8: byte j holds channel 2j (low nibble)
 *                                   and channel 2j+1 (high nibble);
 *                                   nibble = sign<<3 | E2M1 magnitude code
 *   scales [n_seq][cap][32]  uint8: E4M3 scale of channels 16g..16g+15
 * 288 bytes per row.  Value of channel d = E2M1(code_d) * E4M3(scale_{d/16}). */
typedef struct {
  uint8_t* codes;
  uint8_t* scales;
  int64_t cap;   /* rows per sequence */
  int32_t n_seq; /* sequences */
} csa2_fp4_kv;

/* Quantise n_rows bf16 rows src [n_rows][512] into codes [n_rows][256] and
 * scales [n_rows][32] (the caller offsets the pointers to the first
 * destination row).  Per 16-channel group with absolute maximum a: scale =
 * E4M3 round-to-nearest-even of a/6, saturating at 448 (the NVFP4 recipe the
 * pages say is followed, [P1 "FP4 KV, ..."]); each channel's magnitude is
 * the round-to-nearest-even of |x|/scale onto {0,.5,1,1.5,2,3,4,6},
 * saturating at 6, with ties to the even code; the sign bit is copied from
 * x (also for magnitude 0); a zero scale gives magnitude 0.  Exact for
 * every finite bf16 input. */
csa2_status csa2_quant_rows(const uint16_t* src, int64_t n_rows, uint8_t* codes, uint8_t* scales,
                            void* stream);

/* Step (a): append one new latent row per sequence.  For each sequence b:
 * row = lens[b]; if row < kv.cap, quantise src[b] (as csa2_quant_rows) into
 * row `row` of sequence b and set lens[b] = row + 1; otherwise leave the
 * cache and lens[b] unchanged and OR 1 into *err_flag (if err_flag is not
 * NULL).  src [kv.n_seq][512] bf16; lens [kv.n_seq] int32 (device). */
csa2_status csa2_quant_append(const uint16_t* src, csa2_fp4_kv kv, int32_t* lens, int32_t* err_flag,
                              void* stream);

/* Step (b): indexer scores [P1 "Compressed Sparse Attention 2 (CSA2)"]:
 * a layer scores its indexer Q against indexer K (Full: all positions or a
 * block pool; Reindex: rescoring with its own Q).  The pages print no
 * formula; the score of key k is
 *     score = sum_h w_h * max(0, q_h . k),   h < 8 indexer heads,
 * (w == NULL means w_h = 1).  The result is the real sum rounded once to
 * binary32 -- exact -- when q, k are integer-valued (|q_h . k| < 2^24) and,
 * with w, every product w_h r_h and every partial sum is representable in
 * binary32 (e.g. weights that are small multiples of 1/8); with other
 * weights the sum is a binary32 sum in an unspecified order.
 *   q      [n_seq][8][64] bf16; w [n_seq][8] f32 or NULL
 *   keys   [n_seq][key_cap][64] bf16
 *   lens   [n_seq] int32 (device): positions per sequence
 *   scores [n_seq][n_out] f32 out; a slot that is not a candidate gets -inf.
 * Flat mode (pool == NULL): slot i scores key row i; it is a candidate iff
 *   i < ceil(lens[b] / len_div) (len_div = 1 for position keys, 8 for the
 *   keys of blocks of 8 positions).  Requires n_out <= key_cap.
 * Pool mode (pool != NULL): pool [n_seq][n_pool] int32 block ids (-1 =
 *   empty); n_out must be n_pool * blk; slot p scores key row
 *   pool[b][p/blk]*blk + p%blk, a candidate iff the block id is >= 0 and
 *   the row is < lens[b] and < key_cap. */
csa2_status csa2_index_score(const uint16_t* q, const float* w, const uint16_t* keys, int64_t key_cap,
                             const int32_t* lens, int32_t len_div, const int32_t* pool, int32_t n_pool,
                             int32_t blk, float* scores, int64_t n_out, int32_t n_seq, void* stream);

/* Step (c): Top-k [P1 "Compressed Sparse Attention 2 (CSA2)"]: a fresh
 * Top-512 (and the 2,048-block pool of the hierarchical indexer).  Among the
 * candidate slots of scores [n_seq][n] -- slots i < ceil(lens[b]/len_div)
 * if lens != NULL (else all n) whose score is neither -inf nor NaN --
 * keep the min(k, #candidates) best by (score descending, slot ascending:
 * ties go to the lower position), and write their ids in ascending order to
 * out [n_seq][k], padding with -1.  The id of slot i is i, or with a pool
 * pool[b][i/blk]*blk + i%blk (pool [n_seq][n_pool], n == n_pool*blk,
 * n_pool <= CSA2_TOPK_MAX; pool ids ascending makes slot order = id order).
 * -0 and +0 are equal.
 * ws: device workspace of csa2_topk_workspace_size(n, n_seq) bytes,
 * 16-byte aligned, zero-filled before its first use; every call leaves it
 * ready for the next one (calls sharing a workspace must not overlap).
 * Limits: 1 <= k <= CSA2_TOPK_MAX, n <= CSA2_TOPK_NMAX. */
size_t csa2_topk_workspace_size(int64_t n, int32_t n_seq);
csa2_status csa2_topk(const float* scores, int64_t n, const int32_t* lens, int32_t len_div, int32_t k,
                      const int32_t* pool, int32_t n_pool, int32_t blk, int32_t* out, void* ws,
                      size_t ws_bytes, int32_t n_seq, void* stream);

/* Steps (b)+(c) of a flat Full layer in one call [P1 "Compressed Sparse
 * Attention 2 (CSA2)"]: a fresh Top-k over all positions.  The result equals
 * csa2_index_score (flat, len_div 1, n_out = key_cap) followed by csa2_topk
 * (n = key_cap, lens): out [n_seq][k] int32, ascending positions, -1
 * padded.  With G = ceil(key_cap / 8,192) and G * k <= 65,536, for
 * key_cap > 65,536, or for G >= 4 and G * n_seq >= 256, the scores are not
 * written out: every scoring workgroup keeps the Top-k
 * (score descending, position ascending) of its 8,192 positions, and one
 * selection runs over those candidates; otherwise the scores go through
 * csa2_topk's passes.
 *   q [n_seq][8][64] bf16, w [n_seq][8] f32 or NULL, keys [n_seq][key_cap][64]
 *   bf16 (q, keys 16-byte aligned), lens [n_seq] int32 (device)
 *   ws: csa2_flat_select_workspace_size(key_cap, k, n_seq) bytes, 256-byte
 *   aligned, zero-filled before its first use and left ready for the next
 *   call (calls sharing it must not overlap).
 * Limits: 1 <= k <= CSA2_TOPK_MAX, 1 <= key_cap <= CSA2_TOPK_NMAX. */
size_t csa2_flat_select_workspace_size(int64_t key_cap, int32_t k, int32_t n_seq);
csa2_status csa2_flat_select(const uint16_t* q, const float* w, const uint16_t* keys, int64_t key_cap,
                             const int32_t* lens, int32_t k, int32_t* out, void* ws, size_t ws_bytes, int32_t n_seq,
                             void* stream);

/* Steps (b)+(c) of a hierarchical layer's pool in one call [P1 "Compressed
 * Sparse Attention 2 (CSA2)"]: the hierarchical Full layer and the Reindex
 * layers after it keep a fresh Top-k among the positions of a pool of up to
 * 2,048 blocks of blk positions.  The result equals csa2_index_score (pool
 * mode, n_out = n_pool * blk) followed by csa2_topk (the same pool, lens =
 * NULL): out [n_seq][k] int32, the ascending positions, -1 padded.  For
 * n_pool * blk <= 16,384 the scoring also leaves a lower bound of each
 * sequence's k-th score (every wavefront's j-th largest of its 128 slots,
 * j = ceil(k / tiles), the least of them), and the selection keeps only the
 * scores at or above it.
 *   q [n_seq][8][64] bf16, w [n_seq][8] f32 or NULL, keys [n_seq][key_cap][64]
 *   bf16 (q, keys 16-byte aligned), lens [n_seq] int32 (device), pool
 *   [n_seq][n_pool] int32 ascending block ids (-1 = empty)
 *   ws: csa2_pool_select_workspace_size(n_pool, blk, n_seq) bytes, 256-byte
 *   aligned, zero-filled before its first use and left ready for the next
 *   call (calls sharing it must not overlap).
 * Limits: 1 <= k <= CSA2_TOPK_MAX, 1 <= n_pool <= CSA2_TOPK_MAX,
 * n_pool * blk <= CSA2_TOPK_NMAX. */
size_t csa2_pool_select_workspace_size(int32_t n_pool, int32_t blk, int32_t n_seq);
csa2_status csa2_pool_select(const uint16_t* q, const float* w, const uint16_t* keys, int64_t key_cap,
                             const int32_t* lens, const int32_t* pool, int32_t n_pool, int32_t blk, int32_t k,
                             int32_t* out, void* ws, size_t ws_bytes, int32_t n_seq, void* stream);

/* Steps (d)+(e): sparse + SWA attention of n_q queries.
 * [P1 "Compressed Sparse Attention 2 (CSA2)"]: each layer attends with its
 * own main Q over the selected main-KV rows; [P1 "Causal Encoder-Decoder:
 * Half the Prefill"]: a 128-token sliding window runs in every layer; [P3]:
 * key and value are the same 512-d latent.  For query b the attended set
 * is the FP4 rows idx[b][i] (0 <= id < kv->cap; other entries are skipped)
 * of cache sequence b / q_per_seq, dequantised (step d), followed by SWA
 * rows swa[b*swa_q_stride_rows + j] for j < swa_len[b]; one softmax over the
 * whole set per head:  o_h = sum_j softmax_j(sm_scale * q_h . x_j) x_j.
 * An empty set gives o_h = 0.
 *   q   [n_q][16][512] bf16;  idx [n_q][k_idx] int32
 *   swa [*][512] bf16 rows;   swa_len [n_q] int32 (device), each <= swa_max
 *   swa_q_stride_rows >= 0: rows between the windows of consecutive queries
 *       (swa_max for separate windows, 1 for the overlapping windows of
 *       consecutive prefill tokens); a negative stride is rejected
 *   out [n_q][16][512] f32
 *   ws  device workspace of csa2_sparse_attn_workspace_size(...) bytes,
 *       16-byte aligned; no initialisation needed.  Calls that share a
 *       workspace must not overlap in time.
 * Limits: 1 <= k_idx + swa_max <= 8192, swa_max <= 4096, n_q <= 65535;
 * q, kv->codes, swa, out and ws 16-byte aligned, kv->scales 8-byte. */
size_t csa2_sparse_attn_workspace_size(int32_t n_q, int32_t k_idx, int32_t swa_max);
csa2_status csa2_sparse_attn(const uint16_t* q, int32_t n_q, const csa2_fp4_kv* kv, int32_t q_per_seq,
                             const int32_t* idx, int32_t k_idx, const uint16_t* swa,
                             int64_t swa_q_stride_rows, const int32_t* swa_len, int32_t swa_max,
                             float sm_scale, float* out, void* ws, size_t ws_bytes, void* stream);

/* The context-parallel split of steps (d)+(e): one sequence longer than a
 * GPU holds, its positions sharded over ranks.  Each selecting layer: every
 * rank selects among its own positions with global ids, the ranks exchange
 * (score, id) pairs and derive the same global Top-512, each rank attends
 * over the selected rows it holds (the rank with the tail also over the
 * window), and the ranks' shares are merged.  The pages describe no split:
 * the share and the merge are the plain log-sum-exp decomposition of the
 * softmax of csa2_sparse_attn ([P1 "Compressed Sparse Attention 2 (CSA2)"]:
 * one softmax over the selected rows and the window).  The exchange itself
 * (RCCL all-gather over xGMI) is the caller's.
 *
 * csa2_sparse_attn_partial: a rank's share -- csa2_sparse_attn's arguments
 * and rows (bf16 window rows; swa_max = 0 or swa_len 0 on ranks without the
 * window), the softmax left unnormalised:
 *   out_o  [n_q][16][512] f32: o_h = sum_j 2^(z_j - m_h) x_j
 *   out_ml [n_q][16][2]  f32: (m_h, l_h), m_h = max_j z_j, l_h = sum_j 2^(z_j - m_h)
 * with z_j = sm_scale * log2(e) * (q_h . x_j) (base-2 units); a query with no
 * row gives m = -inf, l = 0, o = 0.  ws: csa2_sparse_attn_workspace_size bytes,
 * as for csa2_sparse_attn.  out_o 16-byte and out_ml 8-byte aligned.
 *
 * csa2_attn_merge: the softmax over the union of n_parts shares, per query
 * and head: M = max_s m_s, out = sum_s 2^(m_s - M) o_s / sum_s 2^(m_s - M) l_s
 * (0 where no share has a row).  parts_o [n_parts][n_q][16][512],
 * parts_ml [n_parts][n_q][16][2] (the shares of the ranks, stacked in any
 * order), out [n_q][16][512] f32.  n_parts >= 1, n_q <= 65535; parts_o and
 * out 16-byte, parts_ml 8-byte aligned. */
csa2_status csa2_sparse_attn_partial(const uint16_t* q, int32_t n_q, const csa2_fp4_kv* kv, int32_t q_per_seq,
                                     const int32_t* idx, int32_t k_idx, const uint16_t* swa,
                                     int64_t swa_q_stride_rows, const int32_t* swa_len, int32_t swa_max,
                                     float sm_scale, float* out_o, float* out_ml, void* ws, size_t ws_bytes,
                                     void* stream);
csa2_status csa2_attn_merge(const float* parts_o, const float* parts_ml, int32_t n_parts, int32_t n_q, float* out,
                            void* stream);

/* csa2_sparse_attn for callers that cannot allocate device memory (code
 * under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc): the same computation and arguments without a workspace.  The
 * split partials live in a static scratch array of 16 MiB per GPU (held
 * until the process ends); a call whose csa2_sparse_attn_workspace_size
 * exceeds it fails with CSA2_ECAPACITY before anything is enqueued (batch
 * 16 at 512 selected + 128 window rows needs about 2.6 MB).  Allocates
 * nothing.  Every call on one GPU uses that GPU's one scratch array, so
 * calls that overlap in time on one GPU (concurrent streams, threads)
 * race; calls in order on one stream do not. */
csa2_status csa2_sparse_attn_noalloc(const uint16_t* q, int32_t n_q, const csa2_fp4_kv* kv, int32_t q_per_seq,
                                     const int32_t* idx, int32_t k_idx, const uint16_t* swa,
                                     int64_t swa_q_stride_rows, const int32_t* swa_len, int32_t swa_max,
                                     float sm_scale, float* out, void* stream);

/* FP8 window rows ([P4] summary: the sliding-window KV is kept in FP8).
 * READING: OCP E4M3FN elements, one byte per channel, no scale; a bf16 value
 * becomes its round-to-nearest-even E4M3 code (ties to the even code),
 * saturating at +-448, with the sign copied (also for zero) and NaN kept.
 * csa2_quant_fp8_rows converts src [n_rows][512] bf16 into dst [n_rows][512]
 * E4M3 (exact decisions); csa2_sparse_attn_f8w is csa2_sparse_attn with the
 * window rows swa [*][512] given as those E4M3 bytes (dequantised exactly).
 * src 16-byte, dst 8-byte aligned. */
csa2_status csa2_quant_fp8_rows(const uint16_t* src, int64_t n_rows, uint8_t* dst, void* stream);
csa2_status csa2_sparse_attn_f8w(const uint16_t* q, int32_t n_q, const csa2_fp4_kv* kv, int32_t q_per_seq,
                                 const int32_t* idx, int32_t k_idx, const uint8_t* swa,
                                 int64_t swa_q_stride_rows, const int32_t* swa_len, int32_t swa_max,
                                 float sm_scale, float* out, void* ws, size_t ws_bytes, void* stream);

/* Indexer-key and block-key maintenance ([P1 "Compressed Sparse Attention 2
 * (CSA2)"]: the hierarchical pool needs a key per block of blk positions;
 * the pages do not say how it is formed).  READING: a block's key is the
 * sum of the indexer keys of its existing positions, in bf16.
 *   csa2_block_keys: blk_k [n_seq][blk_cap][64] = the key of every block of
 *     idx_k [n_seq][key_cap][64] over its first lens[b] positions (summed in
 *     binary32, rounded once to bf16); blocks past the last are written 0.
 *   csa2_append_index_keys: for each sequence b, with row = lens[b] (read
 *     before csa2_quant_append advances it): idx_k[b][row] = new_k[b], and
 *     if blk_k != NULL the key of block row/blk becomes new_k[b] (first
 *     position of the block) or its previous value + new_k[b], rounded to
 *     bf16.  The running sum equals the once-rounded sum while every
 *     partial sum is exact in bf16 (integer-valued keys, |sum| <= 256).
 *     A row past key_cap (or a block past blk_cap) writes nothing and ORs 2
 *     into *err_flag (if not NULL).
 * new_k [n_seq][64] bf16; lens [n_seq] int32 (device). */
csa2_status csa2_block_keys(const uint16_t* idx_k, int64_t key_cap, const int32_t* lens, int32_t blk,
                            uint16_t* blk_k, int64_t blk_cap, int32_t n_seq, void* stream);
csa2_status csa2_append_index_keys(const uint16_t* new_k, uint16_t* idx_k, int64_t key_cap, uint16_t* blk_k,
                                   int64_t blk_cap, int32_t blk, const int32_t* lens, int32_t* err_flag,
                                   int32_t n_seq, void* stream);

/* ------------------------------------------------------------ scheduler
 * Static layer-mode table [P1 "Compressed Sparse Attention 2 (CSA2)"]:
 *   Full    computes its own selection: a fresh Top-k over all positions,
 *           or (hierarchical) Top-pool_blocks blocks by block key, then a
 *           Top-k over the pool's positions;
 *   Reindex rescores with its own indexer Q the keys of the last Full layer
 *           (its pool when that layer is hierarchical, else all positions);
 *   Reuse   reuses the latest Full/Reindex indices and skips the indexer.
 * Every layer attends with its own main Q and SWA window over the main-KV
 * tensor kv_id.  Layer 0 must be Full; Reindex needs an earlier Full; Reuse
 * needs an earlier Full or Reindex (else CSA2_EMODE). */
#define CSA2_FULL 0
#define CSA2_REINDEX 1
#define CSA2_REUSE 2

typedef struct {
  int32_t mode;         /* CSA2_FULL / CSA2_REINDEX / CSA2_REUSE */
  int32_t kv_id;        /* main-KV tensor attended over (index into io.kv) */
  int32_t hierarchical; /* Full only: 1 = select through the block pool */
} csa2_layer;

typedef struct {
  int32_t n_seq;
  int32_t n_layers;
  const csa2_layer* layers; /* host [n_layers], copied at create */
  int64_t key_cap;          /* rows per sequence of indexer K (>= every lens) */
  int64_t blk_cap;          /* rows per sequence of block keys (hierarchical) */
  int32_t topk;             /* positions kept (512) */
  int32_t pool_blocks;      /* blocks kept by a hierarchical Full layer (2048) */
  int32_t blk;              /* positions per block (8) */
  int32_t swa_max;          /* rows per sequence of each SWA buffer (128) */
  float sm_scale;           /* softmax scale (READING: 1/sqrt(512)) */
  int32_t swa_fp8;          /* 1: window rows are E4M3 bytes (see csa2_quant_fp8_rows) */
} csa2_sched_desc;

/* Per-step inputs/outputs.  Arrays marked "host" hold device pointers. */
typedef struct {
  int32_t n_kv;
  const csa2_fp4_kv* kv;        /* host [n_kv]; each n_seq = desc.n_seq */
  int32_t* lens;                /* [n_seq] positions, shared by all tensors */
  const uint16_t* new_row;      /* [n_seq][512] bf16 row to append, or NULL */
  int32_t append_kv;            /* tensor that receives the appended row */
  uint16_t* idx_k;              /* [n_seq][key_cap][64] bf16 indexer K (written with new_idx_k) */
  uint16_t* blk_k;              /* [n_seq][blk_cap][64] bf16 block keys, or NULL (written with
                                   new_idx_k) */
  const uint16_t* const* idx_q; /* host [n_layers]: [n_seq][8][64] (Reuse: ignored) */
  const float* const* idx_w;    /* host [n_layers] of [n_seq][8] f32 or NULL; NULL array = all 1 */
  const uint16_t* const* main_q; /* host [n_layers]: [n_seq][16][512] bf16 */
  const void* const* swa;       /* host [n_layers]: [n_seq][swa_max][512] bf16, or E4M3
                                   bytes when desc.swa_fp8 */
  const int32_t* swa_len;       /* [n_seq] valid SWA rows (<= swa_max) */
  float* const* out;            /* host [n_layers]: [n_seq][16][512] f32 */
  const uint16_t* new_idx_k;    /* [n_seq][64] bf16 indexer key of the appended position, or
                                   NULL: with it the step first appends the key to idx_k and
                                   its block's key (csa2_append_index_keys) */
  const uint16_t* const* layer_idx_k; /* host [n_layers] or NULL: entry l = the own indexer K
                                   [n_seq][key_cap][64] bf16 of flat Full layer l (each Full
                                   layer projects its keys); the Reindex layers after it rescore
                                   the same keys.  A NULL array or entry means idx_k; entries of
                                   other layers must be NULL (else CSA2_EINVAL), and hierarchical
                                   Full layers always use idx_k with blk_k. */
  const void* const* new_swa_row; /* host [n_layers] or NULL: entry l = [n_seq][512] window row of
                                   the step's token for layer l (bf16, or E4M3 bytes when
                                   desc.swa_fp8), 16-byte aligned.  READING: each window is a ring
                                   of swa_max rows, position p in slot p % swa_max, and the step's
                                   token is position lens[b] - 1 (after the step's append).  Layer
                                   l's attention reads this row in place of that slot and stores it
                                   there, so that it joins the window as the layer runs; a slot at
                                   or past swa_len[b] is neither read nor written.  NULL: the
                                   windows are read as they are. */
} csa2_step_io;

typedef struct csa2_sched csa2_sched;

/* Validate the table and allocate the scheduler's device workspace on the
 * current device; csa2_sched_decode_step and csa2_sched_check must be called
 * with that device current (else CSA2_EINVAL). */
csa2_status csa2_sched_create(const csa2_sched_desc* desc, csa2_sched** out);
/* One decode step on `stream`: the key append (if io.new_idx_k), the
 * latent append (if io.new_row), then every layer in table order.
 * Asynchronous; capturable in a HIP graph.  Device flags (csa2_sched_check):
 * bit 0 an append found a full cache, bit 1 a key append found one. */
csa2_status csa2_sched_decode_step(csa2_sched* s, const csa2_step_io* io, void* stream);
/* Device pointer to the indices [n_seq][topk] int32 that layer `layer`
 * attended over in the last step (Reuse layers share their source's
 * buffer), or NULL if out of range. */
const int32_t* csa2_sched_indices(const csa2_sched* s, int32_t layer);
/* Device pointer to the pool [n_seq][pool_blocks] int32 built by the last
 * hierarchical Full layer, or NULL if the table has none. */
const int32_t* csa2_sched_pool(const csa2_sched* s);
/* Blocking: on `stream` (the stream the steps ran on), read and clear the
 * device error flags (bit 0: a latent append found a full cache; bit 1: a
 * key append did), then wait for the stream.  The flags reflect every step
 * enqueued on that stream before the call; steps still running on other
 * streams are not waited for.  Returns CSA2_OK and stores the flags in
 * *flags.  Not capturable (it synchronises). */
csa2_status csa2_sched_check(csa2_sched* s, int32_t* flags, void* stream);
void csa2_sched_destroy(csa2_sched* s);

/* ------------------------------------------------------------ prefill
 * A causal prefill chunk of an encoder layer group over compressed entries
 * [P1 "Compressed Sparse Attention 2 (CSA2)"]: the encoder layers run CSA2
 * at compression ratio 2 in groups of one Full and five Reuse layers; [P3]:
 * the encoder merges adjacent positions.  READING: compressed entry e
 * merges tokens ratio*e .. ratio*e + ratio-1 and is visible to the query at
 * token t iff its last token is <= t, so query t sees entries
 * e < vis(t) = min(n_entries, (t + 1) / ratio); its window is the 128
 * tokens t-127 .. t.  Query i of a chunk sits at token t0 + i.  Every
 * query selects on its own. */

/* Indexer scores of the chunk's n_q queries against all entries (the
 * formula of csa2_index_score, on MFMA with both operands dense):
 *   q      [n_q][8][64] bf16; w [n_q][8] f32 or NULL (all 1)
 *   keys   [n_entries][64] bf16 indexer K of the entries
 *   scores [n_q][n_entries] f32 out, 16-byte aligned: scores[i][e] for
 *          e < vis(t0 + i), -inf for the entries query i cannot see
 *   n_vis  [n_q] int32 out (device): vis(t0 + i), usable as the `lens` of
 *          csa2_topk (len_div 1) over these scores.
 * Requires ratio >= 1, t0 >= 0, 1 <= n_q <= 2,097,120, n_entries <= 2^30. */
csa2_status csa2_prefill_index_score(const uint16_t* q, const float* w, const uint16_t* keys,
                                     int64_t n_entries, int64_t t0, int32_t ratio, int32_t n_q,
                                     float* scores, int32_t* n_vis, void* stream);

/* The selection of a chunk's queries, as a Full or Reindex layer of
 * csa2_prefill_chunk takes it: query i's Top-k of its indexer scores over
 * its visible entries ([P1 "Compressed Sparse Attention 2 (CSA2)"]: the
 * indexer picks each query's own top entries), in csa2_topk's order
 * (score descending, the lower entry first among equal scores, ids
 * ascending, -1 padded).
 *   q, w, keys, n_entries, t0, ratio, n_q: as csa2_prefill_index_score
 *   k      entries kept per query, 1 .. 2048
 *   idx    [n_q][k] int32 out (device)
 *   n_vis  [n_q] int32 out (device): vis(t0 + i)
 *   ws     csa2_prefill_select_workspace_size(n_entries, n_q, k) bytes,
 *          256-byte aligned, zero-filled before its first use and left
 *          ready for the next call (calls sharing it must not overlap).
 * For 32,769 .. 65,536 entries, n_q >= 256 and k <= 512 the selection is
 * filtered while scoring: only the scores at or above a per-query
 * threshold estimated from 1,024 sampled entries leave the scoring kernel,
 * and a query whose candidates cannot give its Top-k exactly is scored
 * again in full; otherwise all scores are written and selected.  The
 * result is the same either way.  Requires 1 <= n_q <= 65535,
 * 1 <= n_entries <= 1,048,576, ratio >= 1, t0 >= 0, q and keys 16-byte
 * aligned.  Asynchronous on `stream`; allocates nothing. */
size_t csa2_prefill_select_workspace_size(int64_t n_entries, int32_t n_q, int32_t k);
csa2_status csa2_prefill_select(const uint16_t* q, const float* w, const uint16_t* keys, int64_t n_entries,
                                int64_t t0, int32_t ratio, int32_t n_q, int32_t k, int32_t* idx,
                                int32_t* n_vis, void* ws, size_t ws_bytes, void* stream);

typedef struct {
  int32_t n_layers;
  const csa2_layer* layers; /* host [n_layers]; Full / Reindex (flat) / Reuse */
  int64_t n_entries;        /* compressed entries in the cache and indexer K */
  int32_t ratio;            /* tokens per entry (2 in the encoder) */
  int32_t n_q;              /* queries of the chunk */
  int64_t t0;               /* token of query 0; needs t0 >= swa - 1 */
  int32_t topk;             /* entries kept per query (512) */
  int32_t swa;              /* window tokens per query (128) */
  float sm_scale;
} csa2_prefill_desc;

typedef struct {
  int32_t n_kv;
  const csa2_fp4_kv* kv;          /* host [n_kv]; each n_seq = 1, cap >= n_entries */
  const uint16_t* entry_k;        /* [n_entries][64] bf16 indexer K */
  const uint16_t* const* idx_q;   /* host [n_layers]: [n_q][8][64] bf16 (Reuse: ignored) */
  const float* const* idx_w;      /* host [n_layers] of [n_q][8] f32 or NULL; NULL array = all 1 */
  const uint16_t* const* main_q;  /* host [n_layers]: [n_q][16][512] bf16 */
  const uint16_t* const* swa;     /* host [n_layers]: [n_q + swa - 1][512] bf16, row j = token
                                     t0 - swa + 1 + j */
  float* const* out;              /* host [n_layers]: [n_q][16][512] f32 */
  int32_t* const* idx;            /* host [n_layers]: [n_q][topk] int32 out for Full / Reindex
                                     layers (ascending entry ids, -1 padded); Reuse: ignored */
} csa2_prefill_io;

/* Workspace of csa2_prefill_chunk (scores [n_q][n_entries] f32 and, when the
 * selection is filtered while scoring, candidate lists of 2 KiB per query
 * and 512 entries dominate). */
size_t csa2_prefill_workspace_size(const csa2_prefill_desc* desc);
/* Run the layer table over the chunk: a Full or Reindex layer scores all
 * visible entries with its own indexer Q and keeps a Top-`topk` per query
 * (csa2_topk's order: score descending, lower entry first, ids ascending,
 * -1 padded); a Reuse layer reuses the latest selection; every layer
 * attends (csa2_sparse_attn) with its own main Q over its query's selected
 * entries of tensor kv_id followed by the query's window rows.
 * ws: csa2_prefill_workspace_size bytes, 256-byte aligned, zero-filled
 * before its first use and left ready for the next call (calls sharing it
 * must not overlap).  Asynchronous on `stream`; allocates nothing. */
csa2_status csa2_prefill_chunk(const csa2_prefill_desc* desc, const csa2_prefill_io* io, void* ws,
                               size_t ws_bytes, void* stream);

#ifdef __cplusplus
}
#endif
#endif /* CSA2_H */
