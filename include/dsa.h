/*
 * dsa.h -- C ABI of the MI355X (gfx950) DeepSeek Sparse Attention hot path.
 *
 * Three calls make one decode step (or one prefill) of DeepSeek Sparse
 * Attention, as the method is described on the pages
 *   "DeepSeek fixes RoPE mismatch in the V3.2-Exp inference demo"
 *   "DeepSeek-V3.2-Exp . RoPE coefficients"
 *   "DeepSeek-V3.2-Exp -- Sparse latent attention"
 *   "DeepSeek-V3.2-Exp . Rotate first features"
 *   "DeepSeek-V3.2-Exp . Similarities"
 *
 *   dsa_indexer     lightning-indexer score on block-FP8 q and k with
 *                   non-interleaved RoPE (also appends the new keys)
 *   dsa_topk        per-query causal top-k selection (up to 2048 positions)
 *   dsa_sparse_mla  sparse latent attention in absorbed (MQA) form
 *
 * plus dsa_rope_table, which builds the rotary tables, and dsa_mla_append,
 * which writes new latent / rotary-key rows into the caches call 3 reads.
 *
 * The prefill can also run in the multi-head (non-absorbed) form:
 *   dsa_mla_kv_up     per-head keys and values up-projected from the latent
 *   dsa_sparse_mha    sparse attention over them under the index and causal
 *                     masks
 * and the absorbed form's projections around call 3 are dsa_mla_absorb_q
 * (query into the latent space) and dsa_mla_absorb_o (latent output back to
 * each head's values).
 *
 * Conventions shared by every call:
 *  - Every pointer in an args struct is a DEVICE pointer unless stated.
 *    The caller owns every buffer; the library allocates nothing, frees
 *    nothing and never synchronises. Its only state across calls is
 *    one-time set-up, kept per device under a lock: which kernels have been
 *    opted in to more than 64 KiB of LDS, and where the static scratch of
 *    dsa_sparse_mla_noalloc lives.
 *  - Work is enqueued on `stream` in order; results are ready when the
 *    stream reaches the end of the call's work. Calls on one stream see each
 *    other's results in order.
 *  - All arguments are validated on the host before anything is launched;
 *    on any error nothing is launched and no memory is touched. Values that
 *    live in device memory (positions, indices) cannot be checked on the
 *    host: the kernels bound-check them instead and treat an out-of-range
 *    position as an empty row and an out-of-range index as "not selected".
 *  - dsa_status 0 means success. A failed launch reports DSA_ERR_HIP.
 *    Device-side faults surface at the caller's next synchronisation.
 *  - bf16 data is passed as uint16 bit patterns.
 *  - Paged caches. Every call that reads or writes a per-position cache
 *    (k_cache/k_scale, latent/rope) takes the same four optional fields:
 *      block_table  int32 [B][max_pages] (NULL: dense caches)
 *      page_size    positions per page, a power of two in [1, 65536]
 *      max_pages    row length of block_table, >= ceil(Lmax / page_size)
 *      num_pages    pages in the pool, >= 1
 *    Position p of batch row b then lives in pool row
 *    block_table[b][p / page_size] * page_size + p % page_size, and the
 *    cache pointers address the pool (batch strides are ignored). A table
 *    entry outside [0, num_pages) marks the page as not present: the
 *    indexer scores such a key -inf and appends nothing there, the attention
 *    skips it, dsa_mla_append writes nothing there. The pages name paged
 *    variants of the indexer kernels without giving their layout; this is
 *    the plain block-table reading.
 */
#ifndef DSA_H
#define DSA_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

#define DSA_ABI_VERSION 3

/* Fixed head geometry (page "Sparse latent attention": 64 indexer heads of
 * 128 features, one shared 128-feature key per position, a 512-feature
 * latent plus a 64-feature rotary key cached per position). */
#define DSA_INDEX_DIM 128     /* indexer head dim; also the FP8 block size */
#define DSA_INDEX_ROPE 64     /* rotated features of an indexer row */
#define DSA_MAX_INDEX_HEADS 64
#define DSA_LATENT_DIM 512
#define DSA_ROPE_DIM 64
#define DSA_MAX_ATTN_HEADS 128
#define DSA_MAX_TOPK 2048

typedef enum dsa_status {
    DSA_OK = 0,
    DSA_ERR_NULL = 1,        /* a required pointer is NULL */
    DSA_ERR_SHAPE = 2,       /* a size or stride is out of its range */
    DSA_ERR_UNSUPPORTED = 3, /* unknown dtype or flag */
    DSA_ERR_WORKSPACE = 4,   /* workspace missing or smaller than required */
    DSA_ERR_ALIGN = 5,       /* a pointer or stride is not 16-byte aligned */
    DSA_ERR_HIP = 6,         /* a HIP launch failed */
    DSA_ERR_SCRATCH = 7      /* the no-allocation call's static scratch is too small */
} dsa_status;

enum { DSA_DTYPE_F32 = 0, DSA_DTYPE_BF16 = 1 };

/* dsa_indexer_args.flags */
#define DSA_INDEXER_APPEND_ONLY 1u  /* run step 1 only: append keys, no scores */
#define DSA_INDEXER_HADAMARD 2u     /* rotate q and k rows by H_128/sqrt(128) before quantising */
#define DSA_INDEXER_POW2_SCALE 4u   /* round block scales up to a power of two */

/* ------------------------------------------------------------------------
 * Rotary table. Page "RoPE coefficients" (precompute_freqs_cis excerpt):
 * theta_i = theta^(-2i/64) for i < 32 in float32; with yarn != 0 the YaRN
 * blend theta_i/factor*(1-smooth_i) + theta_i*smooth_i, smooth = 1 - ramp,
 * with the ramp and correction range of the YaRN paper (Peng et al. 2023)
 * over [low, high] from beta_fast/beta_slow and orig_len. Entry [p][i] is
 * (cos, sin) of the float32 product p*theta_i, rounded to float32.
 * Output: cos_out, sin_out float32 [P][32], row-major.
 * ---------------------------------------------------------------------- */
typedef struct dsa_rope_table_args {
    int32_t P;          /* positions, >= 1 */
    int32_t yarn;       /* 0: plain frequencies, 1: YaRN blend */
    int32_t orig_len;   /* original training length (YaRN only), >= 1 */
    float theta;        /* rotary base, > 1 */
    float factor;       /* YaRN interpolation factor, >= 1 */
    float beta_fast;    /* YaRN ramp bounds, beta_fast > beta_slow > 0 */
    float beta_slow;
    float* cos_out;     /* [P][32] */
    float* sin_out;     /* [P][32] */
} dsa_rope_table_args;

dsa_status dsa_rope_table(const dsa_rope_table_args* args, hipStream_t stream);

/* ------------------------------------------------------------------------
 * Call 1: lightning-indexer score.
 * Pages: the aipricedb digest's indexer formula
 *   I[t,s] = sum_j w[t,j] * ReLU(q[t,j] . k[s]);
 * "Sparse latent attention", equation S^I; "Rotate first features"
 * (Indexer.forward: non-interleaved RoPE on the first 64 of 128 features in
 * float32, cast back to the input type, block-FP8 quantisation with one
 * float32 scale per 128-element block, keys written to the cache before
 * scoring). Optional per the flags: the Hadamard rotation the pages apply
 * before quantisation ("Sparse latent attention": q and k times
 * H_128/sqrt(128); "Rotate first features": rotate_activation), and
 * power-of-two block scales (the act_quant scale_fmt option).
 *
 * Per query row r = (b, s) at position p = pos[b][s]:
 *  1. if k_raw != NULL: key row k_raw[b][s] is rotated with table row p,
 *     rounded to the activation dtype, quantised, and written to
 *     k_cache[b][p] / k_scale[b][p];
 *  2. the H query rows q_raw[b][s][h] are rotated with row p, rounded,
 *     quantised (to q_fp8/q_scale when given, else to the workspace);
 *  3. for every key 0 <= s' <= p (n_valid = p + 1):
 *       scores[r][s'] = k_scale[b][s'] * sum_h w[r][h] * q_scale[r][h] *
 *                       ReLU(sum_d q8[r][h][d] * k8[b][s'][d])
 *     with q8/k8 the E4M3 code values; entries s' > p are not written.
 * w carries every constant factor (H^-0.5, the 128^-0.5 score scale): the
 * call applies none.
 * Codes: OCP E4M3 (max 448), round to nearest even, saturating; scale =
 * amax/448 (float32 division), 1 for an all-zero row.
 * DSA_INDEXER_HADAMARD: after the RoPE step every q and k row is replaced by
 * H_128 x / sqrt(128) (fast Walsh-Hadamard transform in float32, butterfly
 * strides 1, 2, ..., 64, then one multiplication by fl32(128^-0.5)) and
 * rounded to the activation dtype. Exact scores are unchanged (H/sqrt(128)
 * is orthonormal); the FP8 codes change.
 * DSA_INDEXER_POW2_SCALE: scale = the smallest power of two >= amax/448.
 * With either flag a single-row decode call runs as three launches
 * (prepare k, prepare q, score) instead of the fused one, and needs the
 * workspace dsa_indexer_workspace() reports when q_fp8 is not given.
 *
 * Layouts (row-major, contiguous):
 *   q_raw   [B][S][H][128]  act_dtype         k_raw  [B][S][128] act_dtype
 *   pos     [B][S] int32                      w      [B][S][H] float32
 *   rope_cos/rope_sin [P][32] float32 (dsa_rope_table's output)
 *   k_cache [B][Lmax][128] uint8 (in/out)     k_scale [B][Lmax] float32 (in/out)
 *   q_fp8   [B][S][H][128] uint8 (out, optional)
 *   q_scale [B][S][H] float32 (out, optional; given iff q_fp8 is)
 *   scores  row r at scores + r*ld_scores, float32, ld_scores >= Lmax
 * Alignment: q_raw, k_raw, k_cache, q_fp8, rope_cos and rope_sin 16 bytes;
 * the other arrays 4.
 * Limits: 1 <= H <= 64, B, S >= 1, 1 <= Lmax, P >= 1. A row whose position
 * lies outside [0, min(Lmax, P)) is skipped (nothing appended or scored).
 * With S > 1 every row's key is appended before any row is scored, so a
 * prefill row sees the keys of earlier rows of the same call. Rows of one
 * batch row must have distinct positions (their cache rows are written
 * concurrently).
 * flags: 0, or DSA_INDEXER_APPEND_ONLY to run step 1 alone (fills the key
 * cache, the pages' k_cache/k_scale_cache write); then k_raw is required and
 * q_raw, w, q_fp8, q_scale, scores and the workspace are ignored (may be
 * NULL).
 * Workspace: dsa_indexer_workspace() bytes, 256-byte aligned; 0 when both
 * q_fp8 and q_scale are given.
 * ---------------------------------------------------------------------- */
typedef struct dsa_indexer_args {
    int32_t B, S, H, Lmax, P;
    int32_t act_dtype;           /* DSA_DTYPE_F32 or DSA_DTYPE_BF16 */
    const void* q_raw;
    const void* k_raw;           /* NULL: append nothing */
    const int32_t* pos;
    const float* rope_cos;
    const float* rope_sin;
    const float* w;
    uint8_t* k_cache;
    float* k_scale;
    uint8_t* q_fp8;              /* optional */
    float* q_scale;              /* optional */
    float* scores;
    int64_t ld_scores;
    uint32_t flags;              /* 0 or DSA_INDEXER_APPEND_ONLY */
    void* workspace;
    size_t workspace_bytes;
    const int32_t* block_table;  /* paged k_cache/k_scale (see the conventions) */
    int32_t page_size, max_pages, num_pages;
} dsa_indexer_args;

dsa_status dsa_indexer_workspace(const dsa_indexer_args* args, size_t* bytes);
dsa_status dsa_indexer(const dsa_indexer_args* args, hipStream_t stream);

/* ------------------------------------------------------------------------
 * Call 2: causal top-k. Pages: "Sparse latent attention" (a lightning
 * indexer chooses up to 2,048 positions per query; selection mask over
 * top_2048 of the causally masked score); "Rotate first features"
 * (topk(min(index_topk, end_pos))).
 * Row r = (b, s) has n_valid = pos[b][s] + 1 candidates scores[r][0..n_valid)
 * (0 when the position is outside [0, Lmax)). It selects
 * k_eff = min(K, n_valid) positions under the order (score descending,
 * position ascending) -- equal scores keep the lower position; -0.0 and
 * +0.0 are equal -- and writes them to idx[r][0..k_eff) in ascending
 * position order, then -1 in idx[r][k_eff..K). count[r] = k_eff if given.
 * Scores must be finite (NaN is not ordered).
 * Layouts: scores row r at scores + r*ld_scores (ld_scores >= Lmax),
 *   pos [B][S] int32, idx [B][S][K] int32, count [B][S] int32 (optional).
 * Limits: 1 <= K <= 2048, B, S >= 1, 1 <= Lmax <= 2^21, and
 *   B*S*ceil(Lmax/16384) < 2^31.
 * Workspace: dsa_topk_workspace() bytes (0 when Lmax <= 16384), 256-byte
 * aligned. Rows longer than 16,384 are selected in levels (the top k of each
 * 16,384-score chunk, then of merged groups of those lists); the workspace
 * carries the intermediate candidate lists between the call's launches. Its
 * contents on entry do not matter and are left undefined. Calls that
 * overlap in time need their own.
 * ---------------------------------------------------------------------- */
typedef struct dsa_topk_args {
    int32_t B, S, Lmax, K;
    const float* scores;
    int64_t ld_scores;
    const int32_t* pos;
    int32_t* idx;
    int32_t* count;              /* optional */
    void* workspace;
    size_t workspace_bytes;
} dsa_topk_args;

dsa_status dsa_topk_workspace(const dsa_topk_args* args, size_t* bytes);
dsa_status dsa_topk(const dsa_topk_args* args, hipStream_t stream);

/* ------------------------------------------------------------------------
 * Call 3: sparse latent attention, absorbed (MQA) form. Pages:
 * "Similarities" (MLA decode excerpt: scores = (q_nope_absorbed . kv_cache
 * + q_pe . pe_cache) * softmax_scale, index mask, softmax, scores .
 * kv_cache); "Sparse latent attention" (S' = S m^2/sqrt(192), softmax,
 * O = AV; attention runs over the selected positions alone).
 * For row r = (b, s) and head h, over the selected positions
 * p = idx[r][j] with 0 <= p < Lmax (other entries, e.g. -1, are skipped):
 *   z_j = scale * (q[r][h][0:512] . latent[b][p] + q[r][h][512:576] . rope[b][p])
 *   out[r][h][:] = sum_j softmax(z)_j * latent[b][p_j]       (bf16)
 *   lse[r][h]    = log sum_j exp(z_j)                         (float32)
 * Products and sums in float32; the probabilities are rounded to bf16 for
 * the value product. A row with no selected position gives out = 0 and
 * lse = -inf. q's 64 trailing features and the rope cache are used as
 * given (already rotated by the caller, interleaved pairing).
 * Layouts: q [B][S][Hq][576] bf16 contiguous; latent row p of batch b at
 *   latent + b*latent_batch_stride + p*latent_row_stride (elements, 512
 *   bf16 per row); rope likewise (64 bf16 per row) -- one fused 576-wide
 *   cache row works by pointing rope at latent + 512; idx [B][S][K] int32;
 *   out [B][S][Hq][512] bf16; lse [B][S][Hq] float32 (optional).
 * Limits: 1 <= Hq <= 128, 1 <= K <= 2048, B, S, Lmax >= 1; pointers 16-byte
 * aligned, strides multiples of 8 elements. scale > 0 and finite.
 * Workspace: dsa_sparse_mla_workspace() bytes (key-split partial results).
 * ---------------------------------------------------------------------- */
typedef struct dsa_mla_args {
    int32_t B, S, Hq, Lmax, K;
    const uint16_t* q;
    const uint16_t* latent;
    int64_t latent_row_stride;
    int64_t latent_batch_stride;
    const uint16_t* rope;
    int64_t rope_row_stride;
    int64_t rope_batch_stride;
    const int32_t* idx;
    float scale;
    uint16_t* out;
    float* lse;                  /* optional */
    void* workspace;
    size_t workspace_bytes;
    const int32_t* block_table;  /* paged latent/rope (see the conventions) */
    int32_t page_size, max_pages, num_pages;
} dsa_mla_args;

dsa_status dsa_sparse_mla_workspace(const dsa_mla_args* args, size_t* bytes);
dsa_status dsa_sparse_mla(const dsa_mla_args* args, hipStream_t stream);

/* ------------------------------------------------------------------------
 * dsa_sparse_mla without allocation or workspace. For callers that cannot
 * allocate device memory or hand over a workspace: code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc.
 * Same arguments, kernels and results as dsa_sparse_mla (bit for bit); the
 * workspace fields are ignored. The key-split partial results go to a
 * static device array of DSA_MLA_NOALLOC_MAX_BYTES that every GPU the
 * library runs on holds from the library's load until the process ends.
 * Its address is looked up once per device, on the first call with that
 * device current. The call itself allocates and frees nothing.
 * Limit: the call needs dsa_sparse_mla_workspace() bytes of that array; a
 * larger need (221 to 255 query rows B*S at 128 heads and K = 2048; every
 * call with at most 220 rows, or at least 256, fits) is rejected with
 * DSA_ERR_SCRATCH before anything is launched.
 * Concurrency: every call on one GPU shares that GPU's array, and nothing
 * in it needs to start at any value. Calls that overlap on one GPU (on
 * different streams, or from different host threads without ordering)
 * race on it; calls ordered on one stream do not.
 * ---------------------------------------------------------------------- */
#define DSA_MLA_NOALLOC_MAX_BYTES ((size_t)56 << 20)
dsa_status dsa_sparse_mla_noalloc(const dsa_mla_args* args, hipStream_t stream);

/* ------------------------------------------------------------------------
 * MLA-side cache append (the step that fills the caches call 3 reads).
 * Pages: "RoPE coefficients" (MLA prefill excerpt: new latent rows are
 * written to the latent cache and the rotated rotary keys to the rope cache
 * at their positions); the aipricedb digest's update note of 2025.11.17
 * (MLA's rotary embedding pairs features 2j and 2j+1, interleaved, unlike
 * the indexer's j / j+32).
 * For query row r = (b, s) at position p = pos[b][s] (rows with p < 0,
 * p >= Lmax or p >= P are skipped entirely):
 *   latent[b][p][0:512] = latent_new[b][s][0:512]
 *   rope[b][p][2j], rope[b][p][2j+1] = bf16(a*c - b*s), bf16(a*s + b*c)
 *     for j < 32, (a, b) = kpe_new[b][s][2j], kpe_new[b][s][2j+1] and
 *     (c, s) = (rope_cos[p][j], rope_sin[p][j]); float32 products, each sum
 *     or difference rounded once (no fused multiply-add), then bf16 (RNE);
 *   if q != NULL: q[b][s][h][512 + 2j], q[...][512 + 2j + 1] are rotated in
 *     place the same way for every head h < Hq (q's latent part untouched).
 * Layouts: latent_new [B][S][512] bf16, kpe_new [B][S][64] bf16, pos [B][S]
 *   int32, rope_cos/sin [P][32] float32 (dsa_rope_table), the caches as in
 *   dsa_mla_args (element strides), q [B][S][Hq][576] bf16.
 * Limits: B, S, Lmax, P >= 1; 1 <= Hq <= 128 when q is given; every
 * pointer 16-byte aligned, cache strides multiples of 8 elements.
 * ---------------------------------------------------------------------- */
typedef struct dsa_mla_append_args {
    int32_t B, S, Hq, Lmax, P;
    const uint16_t* latent_new;
    const uint16_t* kpe_new;
    const int32_t* pos;
    const float* rope_cos;
    const float* rope_sin;
    uint16_t* latent;            /* in/out */
    int64_t latent_row_stride;
    int64_t latent_batch_stride;
    uint16_t* rope;              /* in/out */
    int64_t rope_row_stride;
    int64_t rope_batch_stride;
    uint16_t* q;                 /* optional, rotated in place */
    const int32_t* block_table;  /* paged latent/rope (see the conventions) */
    int32_t page_size, max_pages, num_pages;
} dsa_mla_append_args;

dsa_status dsa_mla_append(const dsa_mla_append_args* args, hipStream_t stream);

/* ------------------------------------------------------------------------
 * MLA projections: the key/value up-projection of the multi-head prefill
 * form and the two absorption products of the absorbed form.
 * Pages: "RoPE coefficients" (MLA prefill excerpt: wkv_b applied to the
 * latent rows, its output viewed per head as k_nope (128) then v (128));
 * "Similarities" (MQA decode excerpt: q_nope times W_UK[h] is the latent
 * query, the latent attention output times W_UV[h]^T the head's output).
 * wkv_b [Hq][256][512] bf16 row-major: rows 0..127 of head h are W_UK[h],
 * rows 128..255 are W_UV[h].
 *   dsa_mla_kv_up     y[b][s][256h + d] = sum_c wkv_b[h][d][c] * x[b][s][c]
 *                     (x rows of 512 features, y rows of Hq*256)
 *   dsa_mla_absorb_q  y[b][s][h][c] = sum_d x[b][s][h][d] * W_UK[h][d][c]
 *                     (x head rows of 128, y head rows of 512: only those
 *                     512 elements are written, so y may be the 576-wide
 *                     query of dsa_sparse_mla)
 *   dsa_mla_absorb_o  y[b][s][h][d] = sum_c x[b][s][h][c] * W_UV[h][d][c]
 *                     (x head rows of 512, y head rows of 128)
 * Products accumulate in float32 (bf16 MFMA); the result is rounded to bf16
 * once (nearest even).
 * Addressing, element strides: row s of batch b of x starts at
 * x + b*x_batch_stride + s*x_row_stride, head h of it at + h*x_head_stride;
 * y likewise. dsa_mla_kv_up ignores the head strides. Output heads, rows and
 * batches must not overlap (checked from the strides); y must not overlap x
 * or wkv_b.
 * Limits: B >= 1, 1 <= rows <= 2^24, 1 <= Hq <= 128, B (kv_up) or B*Hq
 * (absorption) <= 65535; every pointer 16-byte aligned, strides
 * non-negative multiples of 8 elements. No workspace.
 * ---------------------------------------------------------------------- */
typedef struct dsa_mla_proj_args {
    int32_t B, rows, Hq;
    const uint16_t* wkv_b;
    const uint16_t* x;
    int64_t x_row_stride, x_batch_stride, x_head_stride;
    uint16_t* y;
    int64_t y_row_stride, y_batch_stride, y_head_stride;
} dsa_mla_proj_args;

dsa_status dsa_mla_kv_up(const dsa_mla_proj_args* args, hipStream_t stream);
dsa_status dsa_mla_absorb_q(const dsa_mla_proj_args* args, hipStream_t stream);
dsa_status dsa_mla_absorb_o(const dsa_mla_proj_args* args, hipStream_t stream);

/* ------------------------------------------------------------------------
 * Sparse attention in the multi-head (non-absorbed) prefill form.
 * Page "RoPE coefficients" (MLA prefill excerpt): per-head keys
 * [k_nope ; k_pe] and values from the up-projection; scores scaled, the
 * index mask scattered from the top-k list and the causal mask added,
 * softmax over positions, product with the values.
 * For row r = (b, s) and head h, over the positions p that appear in idx[r]
 * (a repeated entry counts once), with 0 <= p < Lmax and, when pos is given,
 * p <= pos[b][s]:
 *   z_p = scale * (q[r][h][0:128] . kv[b][p][h][0:128] + q[r][h][128:192] . rope[b][p])
 *   out[r][h][:] = sum_p softmax(z)_p * kv[b][p][h][128:256]       (bf16)
 * Products and sums in float32; the probabilities are rounded to bf16 for
 * the value product. A row with no such position gives 0.
 * Layouts: q [B][S][Hq][192] bf16 (q_nope, then q_pe already rotated);
 *   kv [B][Lmax][Hq][256] bf16 contiguous (dsa_mla_kv_up with rows = Lmax);
 *   rope row p of batch b at rope + b*rope_batch_stride + p*rope_row_stride
 *   (64 bf16, dense caches only); idx [B][S][K] int32; pos [B][S] int32 or
 *   NULL (no causal mask); out [B][S][Hq][128] bf16.
 * Cost: every 64-position tile that any of 128 consecutive rows selects is
 * computed for all of them, so the work follows the causal extent (as the
 * pages' dense masked form does), not K as in dsa_sparse_mla.
 * Limits: 1 <= Hq <= 128, 1 <= K <= 2048, 1 <= Lmax <= 65536, B, S >= 1,
 * B*S <= 2^26; pointers 16-byte aligned (idx, pos 4), rope strides multiples
 * of 8 elements. scale > 0 and finite.
 * Workspace: dsa_sparse_mha_workspace() bytes, 256-byte aligned (per-row
 * bit masks, per-128-row key-tile lists and 256 zero bytes the call writes
 * itself); contents on entry do not matter.
 * ---------------------------------------------------------------------- */
typedef struct dsa_mha_args {
    int32_t B, S, Hq, Lmax, K;
    const uint16_t* q;
    const uint16_t* kv;
    const uint16_t* rope;
    int64_t rope_row_stride;
    int64_t rope_batch_stride;
    const int32_t* idx;
    const int32_t* pos;          /* optional */
    float scale;
    uint16_t* out;
    void* workspace;
    size_t workspace_bytes;
} dsa_mha_args;

dsa_status dsa_sparse_mha_workspace(const dsa_mha_args* args, size_t* bytes);
dsa_status dsa_sparse_mha(const dsa_mha_args* args, hipStream_t stream);

/* ------------------------------------------------------------------------
 * Helpers.
 * ---------------------------------------------------------------------- */
const char* dsa_status_str(dsa_status status);   /* static string, never NULL */
int dsa_abi_version(void);                       /* DSA_ABI_VERSION */

#ifdef __cplusplus
}
#endif
#endif /* DSA_H */
