/*
 * oracle.h -- C interface of the CPU oracle for the DeepSeek Sparse Attention
 * (DSA) hot path: lightning-indexer score, causal top-k, sparse latent
 * attention in absorbed (MQA) form.
 *
 * TEST INFRASTRUCTURE. This library is the plain, slow, obviously correct
 * reference that the GPU library is checked against. Only the tests, the
 * smoke check and the benchmark's CPU-baseline leg may load it. It shares no
 * code, header, table or helper with the GPU library, and the GPU library
 * never calls it.
 *
 * Precision: every floating-point reduction is carried out in double. Steps
 * that the pages fix in float32 (the rotary embedding, the quantiser's scale
 * and division) are done in float32 with one IEEE rounding per operation
 * (the library is built with -ffp-contract=off).
 *
 * Parity notes per function are in oracle.c.
 */
#ifndef DSA_ORACLE_H
#define DSA_ORACLE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* OCP 8-bit floating point, E4M3 ("FN": no infinities, max 448). */
double  orc_e4m3_decode(uint8_t code);
uint8_t orc_e4m3_encode(float x);
void    orc_e4m3_encode_array(int64_t n, const float* x, uint8_t* codes);
void    orc_e4m3_decode_array(int64_t n, const uint8_t* codes, double* out);

/* Nearest bfloat16 value (ties to even), returned as a float. */
float orc_round_bf16(float x);
void  orc_round_bf16_array(int64_t n, const float* x, float* out);

/* Rotary table: cos/sin [P][npairs] float32 (npairs = rope_dim/2).
 * yarn != 0 applies the YaRN frequency blend (used when the served length
 * exceeds orig_len). */
void orc_rope_table(int P, int rope_dim, double theta, int yarn, int orig_len,
                    double factor, double beta_fast, double beta_slow,
                    float* cos_out, float* sin_out);
/* Frequencies theta_i as float32, npairs of them (exposed for the tests). */
void orc_rope_freqs(int rope_dim, double theta, int yarn, int orig_len,
                    double factor, double beta_fast, double beta_slow,
                    float* freqs_out);

/* Rotary embedding of nrows rows of width `width` whose first rope_dim
 * features are rotated; row r uses table row pos[r]. interleaved = 0 pairs
 * feature j with j + rope_dim/2 (indexer); interleaved = 1 pairs 2j with
 * 2j+1 (MLA). Output values are float32; out_bf16 != 0 rounds every output
 * element to bfloat16 ("cast back to the input type"). */
void orc_rope_rows(int64_t nrows, int width, int rope_dim, int interleaved,
                   const float* x, const int32_t* pos, const float* cos_tab,
                   const float* sin_tab, int out_bf16, float* y);

/* Block-wise FP8 quantisation of nrows rows of 128 values: one float32
 * scale per row (scale = amax/448, or 1 when amax == 0) and E4M3 codes of
 * x/scale. */
void orc_quantize_rows(int64_t nrows, const float* x, uint8_t* codes, float* scales);
/* As orc_quantize_rows with the scale rounded up to a power of two. */
void orc_quantize_rows_pow2(int64_t nrows, const float* x, uint8_t* codes, float* scales);
/* y = H_128 x / sqrt(128) per 128-feature row: the signed sum in double,
 * rounded once to float32; out_bf16 then rounds that to bfloat16. */
void orc_hadamard_rows(int64_t nrows, const float* x, int out_bf16, float* y);

/* Dequantise: out[r][d] = decode(codes[r][d]) * scales[r] (double). */
void orc_dequantize_rows(int64_t nrows, const uint8_t* codes, const float* scales,
                         double* out);

/* Lightning-indexer score on real-valued q and k:
 *   out[r][s] = sum_h w[r][h] * max(0, sum_d q[r][h][d] * k[b(r)][s][d])
 * for s < n_valid[r]; b(r) = r / S. q [B*S][H][D], w [B*S][H],
 * k [B][Lmax][D], out [B*S][Lmax] (entries s >= n_valid[r] untouched). */
void orc_indexer_scores(int B, int S, int H, int D, int Lmax, const double* q,
                        const double* w, const double* k, const int32_t* n_valid,
                        double* out);

/* Causal top-k: per row, the k_eff = min(K, n_valid[r]) positions with the
 * largest score under (score desc, position asc), written in ascending
 * position order, tail padded with -1. scores row stride = ld. */
void orc_topk(int64_t nrows, int64_t ld, const double* scores, const int32_t* n_valid,
              int K, int32_t* idx);

/* Sparse latent attention, absorbed form. Row r (batch b = r / S) has query
 * q[r][h][0:Dl+Dr]; for each selected position p = idx[r][j] != -1:
 *   z = scale * (q[r][h][0:Dl] . latent[b][p] + q[r][h][Dl:] . kpe[b][p])
 * softmax over the selected set, out[r][h] = sum_j softmax_j * latent[b][p_j],
 * lse[r][h] = log sum_j exp(z_j). */
void orc_sparse_mla(int B, int S, int Hq, int Dl, int Dr, int Lmax, int K,
                    const double* q, const double* latent, const double* kpe,
                    const int32_t* idx, double scale, double* out, double* lse);

/* Non-absorbed (multi-head) form of the same attention over the same
 * selected set: k_nope = W_UK[h] c, v = W_UV[h] c with wkv_b [Hq][Dn+Dv][Dl]
 * (rows 0..Dn-1 are W_UK, rows Dn.. are W_UV);
 *   z = scale * (q_nope[r][h] . k_nope + q_pe[r][h] . kpe[b][p]),
 * out[r][h][0:Dv] = sum softmax * v. */
void orc_mla_mha(int B, int S, int Hq, int Dn, int Dv, int Dl, int Dr, int Lmax,
                 int K, const double* q_nope, const double* q_pe,
                 const double* wkv_b, const double* latent, const double* kpe,
                 const int32_t* idx, double scale, double* out);

/* Multi-head prefill attention over up-projected per-head keys and values,
 * the selection taken as a set (a repeated position counts once) and, when
 * pos is given, causally masked (p <= pos[r]):
 *   z = scale * (q[r][h][0:Dn] . kv[b][p][h][0:Dn] + q[r][h][Dn:] . kpe[b][p]),
 * out[r][h] = sum softmax * kv[b][p][h][Dn:Dn+Dv]; empty rows give 0. */
void orc_sparse_mha(int B, int S, int Hq, int Dn, int Dv, int Dr, int Lmax, int K,
                    const double* q, const double* kv, const double* kpe,
                    const int32_t* idx, const int32_t* pos, double scale, double* out);

int orc_num_threads(void);
void orc_set_num_threads(int n);   /* threads for later calls; n >= 1 */

#ifdef __cplusplus
}
#endif
#endif
