/*
 * oracle.c -- CPU oracle for the DeepSeek Sparse Attention (DSA) hot path.
 *
 * TEST INFRASTRUCTURE, NOT PRODUCT CODE. This is the plain, slow, obviously
 * correct reference the GPU library is checked against. It is loaded only by
 * the tests, by the smoke check and by the benchmark's CPU-baseline leg. It
 * shares no code with the GPU library (sparse_attention_index_amd/csrc) and
 * neither side includes or calls the other.
 *
 * Sources (the pages the method is taken from):
 *  [P1] "DeepSeek fixes RoPE mismatch in the V3.2-Exp inference demo"
 *       (aipricedb news digest): the indexer formula I[t,s], the block-wise
 *       FP8 quantisation with 128-element blocks, the 2025.11.17 note that
 *       the indexer's RoPE is non-interleaved and MLA's is interleaved.
 *  [P2] "DeepSeek-V3.2-Exp . RoPE coefficients": precompute_freqs_cis
 *       excerpt (frequencies, YaRN blend, polar table), ModelArgs defaults,
 *       MLA __init__ excerpt (softmax scale, mscale), MLA prefill excerpt
 *       (non-absorbed form).
 *  [P3] "DeepSeek-V3.2-Exp -- Sparse latent attention": the 43-step
 *       equation list (lightning-indexer score S^I, top-2048 selection mask
 *       M^sel, S' = S m^2/sqrt(192), softmax, O = AV).
 *  [P4] "DeepSeek-V3.2-Exp . Rotate first features": Indexer.forward and
 *       apply_rotary_emb excerpts, "rotate the first 64 of 128 features",
 *       "in float32, cast back to the input type".
 *  [P5] "DeepSeek-V3.2-Exp . Similarities": MLA decode excerpt (absorbed
 *       MQA form over kv_cache and pe_cache), score shape.
 *  [OFP8] OCP 8-bit Floating Point Specification (2023), E4M3 encoding.
 *  [YaRN] Peng et al., "YaRN: Efficient Context Window Extension of Large
 *       Language Models" (2023): correction range and linear ramp, used for
 *       the part of the frequency blend the [P2] excerpt omits.
 *
 * Parity status of each function is stated at the function. "Parity
 * unpinned" marks a step no test ties to something other than this file.
 */
#include "oracle.h"

#include <math.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

int orc_num_threads(void) {
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/* Threads for the following calls (n >= 1); no effect without OpenMP. */
void orc_set_num_threads(int n) {
#ifdef _OPENMP
    if (n >= 1) omp_set_num_threads(n);
#else
    (void)n;
#endif
}

/* ------------------------------------------------------------------------
 * E4M3 codec [OFP8]; the format the indexer's "FP8" means [P1 TileLang
 * kernels paragraph, P4 act_quant call]. Sign bit, 4 exponent bits (bias 7),
 * 3 mantissa bits. Exponent field 0 is subnormal: m * 2^-9. Exponent 15 with
 * mantissa 7 is NaN; there is no infinity; the largest finite value is 448.
 * Pinned by: all 256 codes against the closed form and against PyTorch's
 * float8_e4m3fn, round-to-nearest-even midpoints, saturation.
 * ---------------------------------------------------------------------- */
double orc_e4m3_decode(uint8_t code) {
    int sign = code >> 7;
    int e = (code >> 3) & 0xF;
    int m = code & 0x7;
    double v;
    if (e == 15 && m == 7) return NAN;
    if (e == 0)
        v = ldexp((double)m, -9);
    else
        v = ldexp(1.0 + (double)m / 8.0, e - 7);
    return sign ? -v : v;
}

/* Nearest finite E4M3 value to x, ties to the even code, magnitudes at or
 * beyond 448 saturate to 448. Plain search over the 127 non-negative finite
 * codes, which increase with their magnitude. */
uint8_t orc_e4m3_encode(float x) {
    double a = fabs((double)x);
    uint8_t sign = signbit(x) ? 0x80 : 0x00;
    int c;
    if (a >= 448.0) return (uint8_t)(sign | 0x7E);
    for (c = 1; c <= 0x7E; ++c) {
        double hi = orc_e4m3_decode((uint8_t)c);
        if (hi >= a) {
            double lo = orc_e4m3_decode((uint8_t)(c - 1));
            double dlo = a - lo, dhi = hi - a;
            int pick;
            if (dlo < dhi) pick = c - 1;
            else if (dhi < dlo) pick = c;
            else pick = ((c - 1) % 2 == 0) ? c - 1 : c; /* tie: even code */
            return (uint8_t)(sign | pick);
        }
    }
    return (uint8_t)(sign | 0x7E); /* not reached: a < 448 */
}

void orc_e4m3_encode_array(int64_t n, const float* x, uint8_t* codes) {
    int64_t i;
#pragma omp parallel for schedule(static)
    for (i = 0; i < n; ++i) codes[i] = orc_e4m3_encode(x[i]);
}

void orc_e4m3_decode_array(int64_t n, const uint8_t* codes, double* out) {
    int64_t i;
#pragma omp parallel for schedule(static)
    for (i = 0; i < n; ++i) out[i] = orc_e4m3_decode(codes[i]);
}

/* ------------------------------------------------------------------------
 * bfloat16 rounding: the float32 values whose low 16 bits are zero; pick the
 * nearer of the two neighbours bracketing x, ties to the one whose last kept
 * bit is 0. Used for "cast back to the input type" [P4] when the input is
 * bfloat16. Pinned by: PyTorch's float32 -> bfloat16 conversion.
 * ---------------------------------------------------------------------- */
static float bits_to_f32(uint32_t u) { float f; memcpy(&f, &u, 4); return f; }
static uint32_t f32_to_bits(float f) { uint32_t u; memcpy(&u, &f, 4); return u; }

float orc_round_bf16(float x) {
    uint32_t u = f32_to_bits(x);
    uint32_t down = u & 0xFFFF0000u;          /* toward zero */
    uint32_t up = down + 0x10000u;            /* away from zero */
    double dd, du;
    if ((u & 0xFFFFu) == 0) return x;         /* already a bf16 value */
    if (((u >> 23) & 0xFF) == 0xFF) return x; /* inf/nan: not expected */
    dd = fabs((double)x - (double)bits_to_f32(down));
    if (((up >> 23) & 0xFF) == 0xFF)          /* rounding up overflows */
        du = fabs(ldexp(1.0, 128) * (signbit(x) ? -1.0 : 1.0) - (double)x);
    else
        du = fabs((double)bits_to_f32(up) - (double)x);
    if (dd < du) return bits_to_f32(down);
    if (du < dd) return bits_to_f32(up);
    return ((down >> 16) & 1u) ? bits_to_f32(up) : bits_to_f32(down);
}

void orc_round_bf16_array(int64_t n, const float* x, float* out) {
    int64_t i;
#pragma omp parallel for schedule(static)
    for (i = 0; i < n; ++i) out[i] = orc_round_bf16(x[i]);
}

/* ------------------------------------------------------------------------
 * Rotary table [P2 precompute_freqs_cis excerpt]. theta_i = base^(-2i/dim)
 * for i < dim/2, held in float32. When the served length exceeds the
 * original one, the YaRN blend freqs/factor*(1-smooth) + freqs*smooth
 * applies, smooth = 1 - ramp; the ramp and its correction range are not on
 * the page, they follow [YaRN]:
 *   d(r)  = dim * ln(orig / (2 pi r)) / (2 ln base)
 *   low   = max(floor(d(beta_fast)), 0), high = min(ceil(d(beta_slow)), dim-1)
 *   ramp_i = clamp((i - low) / (high - low), 0, 1)   (high += 0.001 if equal)
 * The table entry for position p and pair i is (cos, sin) of the float32
 * product p * theta_i (the page forms the angles with a float32 outer
 * product), each rounded to float32.
 * Reading: theta and the blend are evaluated in double and rounded once to
 * float32; cos/sin are evaluated in double and rounded to float32.
 * Pinned by: closed-form cos/sin for the plain table; YaRN invariants
 * (ratio 1 at pair 0, 1/factor at the last pair, monotone); the ramp's end
 * points by [YaRN]'s rule in wavelengths (a pair turning more than
 * beta_fast times over the original context is kept, less than beta_slow
 * times fully interpolated, blended in between), which fixes the floor of
 * low and the ceiling of high, and the ramp's linearity in the pair index.
 * ---------------------------------------------------------------------- */
static double yarn_corr_dim(double rotations, int dim, double base, int orig) {
    return (double)dim * log((double)orig / (rotations * 2.0 * acos(-1.0))) / (2.0 * log(base));
}

void orc_rope_freqs(int rope_dim, double theta, int yarn, int orig_len,
                    double factor, double beta_fast, double beta_slow,
                    float* freqs_out) {
    int npairs = rope_dim / 2, i;
    double low = 0, high = 0;
    if (yarn) {
        low = floor(yarn_corr_dim(beta_fast, rope_dim, theta, orig_len));
        high = ceil(yarn_corr_dim(beta_slow, rope_dim, theta, orig_len));
        if (low < 0) low = 0;
        if (high > rope_dim - 1) high = rope_dim - 1;
        if (low == high) high += 0.001;
    }
    for (i = 0; i < npairs; ++i) {
        float f = (float)pow(theta, -(2.0 * i) / (double)rope_dim);
        if (yarn) {
            double ramp = ((double)i - low) / (high - low);
            double smooth;
            if (ramp < 0) ramp = 0;
            if (ramp > 1) ramp = 1;
            smooth = 1.0 - ramp;
            f = (float)((double)f / factor * (1.0 - smooth) + (double)f * smooth);
        }
        freqs_out[i] = f;
    }
}

void orc_rope_table(int P, int rope_dim, double theta, int yarn, int orig_len,
                    double factor, double beta_fast, double beta_slow,
                    float* cos_out, float* sin_out) {
    int npairs = rope_dim / 2, p;
    float freqs[256];
    orc_rope_freqs(rope_dim, theta, yarn, orig_len, factor, beta_fast, beta_slow, freqs);
#pragma omp parallel for schedule(static)
    for (p = 0; p < P; ++p) {
        int i;
        for (i = 0; i < npairs; ++i) {
            float ang = (float)p * freqs[i];
            cos_out[(int64_t)p * npairs + i] = (float)cos((double)ang);
            sin_out[(int64_t)p * npairs + i] = (float)sin((double)ang);
        }
    }
}

/* ------------------------------------------------------------------------
 * Rotary embedding [P4 apply_rotary_emb excerpt and description; P1 update
 * note]. A pair (a, b) is treated as the complex number a + ib and multiplied
 * by cos + i sin in float32:
 *   a' = a*cos - b*sin,   b' = a*sin + b*cos   (each product rounded, then
 *   the sum rounded; no fused multiply-add).
 * Non-interleaved (indexer): pair i is (x[i], x[i + rope_dim/2]).
 * Interleaved (MLA): pair i is (x[2i], x[2i+1]).
 * Features rope_dim..width-1 pass through. With out_bf16 the whole output
 * row is rounded to bfloat16 ("cast back to the input type").
 * Pinned by: a hand-derived worked example (closed form with cos 3, sin 3),
 * the permutation identity between the two pairings, identity at position 0,
 * per-pair norm preservation, relative-position dependence of dot products.
 * ---------------------------------------------------------------------- */
void orc_rope_rows(int64_t nrows, int width, int rope_dim, int interleaved,
                   const float* x, const int32_t* pos, const float* cos_tab,
                   const float* sin_tab, int out_bf16, float* y) {
    int64_t r;
    int half = rope_dim / 2;
#pragma omp parallel for schedule(static)
    for (r = 0; r < nrows; ++r) {
        const float* xr = x + r * width;
        float* yr = y + r * width;
        const float* c = cos_tab + (int64_t)pos[r] * half;
        const float* s = sin_tab + (int64_t)pos[r] * half;
        int i;
        for (i = rope_dim; i < width; ++i) yr[i] = xr[i];
        for (i = 0; i < half; ++i) {
            int ia = interleaved ? 2 * i : i;
            int ib = interleaved ? 2 * i + 1 : i + half;
            float a = xr[ia], b = xr[ib];
            float ac = a * c[i], bs = b * s[i];
            float as = a * s[i], bc = b * c[i];
            yr[ia] = ac - bs;
            yr[ib] = as + bc;
        }
        if (out_bf16)
            for (i = 0; i < width; ++i) yr[i] = orc_round_bf16(yr[i]);
    }
}

/* ------------------------------------------------------------------------
 * Block-wise FP8 quantisation, 128-element blocks, one float32 scale per
 * block [P1 act_quant_kernel; P4 act_quant call; the indexer head dim is 128
 * so one block is one row]. The page does not show the kernel body.
 * Reading: amax = max |x|; scale = amax / 448 (float32 division, the E4M3
 * maximum); scale = 1 when amax == 0 (or when amax/448 rounds to 0);
 * code = E4M3 encode of the float32 quotient x / scale.
 * Pinned by: amax element encodes to +-448, dequantisation error within
 * half an E4M3 step, the codec pins above.
 * ---------------------------------------------------------------------- */
void orc_quantize_rows(int64_t nrows, const float* x, uint8_t* codes, float* scales) {
    int64_t r;
#pragma omp parallel for schedule(static)
    for (r = 0; r < nrows; ++r) {
        const float* xr = x + r * 128;
        float amax = 0.0f, scale;
        int d;
        for (d = 0; d < 128; ++d) {
            float a = fabsf(xr[d]);
            if (a > amax) amax = a;
        }
        scale = amax / 448.0f;
        if (!(scale > 0.0f)) scale = 1.0f;
        for (d = 0; d < 128; ++d) codes[r * 128 + d] = orc_e4m3_encode(xr[d] / scale);
        scales[r] = scale;
    }
}

/* ------------------------------------------------------------------------
 * Power-of-two block scale (the `scale_fmt` variant of act_quant named on
 * page "Rotate first features", Indexer.forward; the pages do not print its
 * rule). Reading: the smallest power of two s with s >= fl32(amax / 448),
 * so no element saturates; s = 1 when amax == 0.
 * Pinned by: s is a power of two, fl32(amax/448) <= s < 2 fl32(amax/448),
 * max |x| / s <= 448.
 * ---------------------------------------------------------------------- */
static float orc_pow2_ceil(float v) {
    int e;
    double m = frexp((double)v, &e);  /* v = m * 2^e, m in [0.5, 1) */
    if (m == 0.5) return v;
    return (float)ldexp(1.0, e);
}

void orc_quantize_rows_pow2(int64_t nrows, const float* x, uint8_t* codes, float* scales) {
    int64_t r;
#pragma omp parallel for schedule(static)
    for (r = 0; r < nrows; ++r) {
        const float* xr = x + r * 128;
        float amax = 0.0f, scale;
        int d;
        for (d = 0; d < 128; ++d) {
            float a = fabsf(xr[d]);
            if (a > amax) amax = a;
        }
        scale = amax / 448.0f;
        scale = (scale > 0.0f) ? orc_pow2_ceil(scale) : 1.0f;
        for (d = 0; d < 128; ++d) codes[r * 128 + d] = orc_e4m3_encode(xr[d] / scale);
        scales[r] = scale;
    }
}

/* ------------------------------------------------------------------------
 * Hadamard rotation of 128-feature rows [page "Sparse latent attention":
 * the indexer's rotated q and k are multiplied by H_128 / sqrt(128) before
 * quantisation; page "Rotate first features": rotate_activation(q),
 * rotate_activation(k) ahead of act_quant]. H_128 is the Sylvester Hadamard
 * matrix (H_1 = [1], H_2n = [[H_n, H_n], [H_n, -H_n]]), whose entry (i, j)
 * is (-1)^popcount(i & j); it is symmetric, so y = H x / sqrt(128) row by
 * row.
 * The definition written out: each output is the double-precision sum of
 * the 128 signed inputs times 1/sqrt(128), rounded once to float32; with
 * out_bf16 that float32 value is then cast to bfloat16 (the activation
 * dtype), like every other step of the indexer's preparation. How a fast
 * transform orders its float32 additions is not on the pages; a GPU result
 * is judged against this one within the rounding bound of its own order.
 * Pinned by: scipy's Hadamard matrix in a float64 product (equal after one
 * rounding), H e_i = column i of H, orthonormality (norm preserved,
 * H H x = x).
 * ---------------------------------------------------------------------- */
static int orc_popcount7(int v) {
    int c = 0;
    while (v) {
        c += v & 1;
        v >>= 1;
    }
    return c;
}

void orc_hadamard_rows(int64_t nrows, const float* x, int out_bf16, float* y) {
    int64_t r;
    const double inv = 1.0 / sqrt(128.0);
#pragma omp parallel for schedule(static)
    for (r = 0; r < nrows; ++r) {
        const float* xr = x + r * 128;
        int i, j;
        for (i = 0; i < 128; ++i) {
            double acc = 0.0;
            float o;
            for (j = 0; j < 128; ++j) {
                double v = (double)xr[j];
                acc += (orc_popcount7(i & j) & 1) ? -v : v;
            }
            o = (float)(acc * inv);
            y[r * 128 + i] = out_bf16 ? orc_round_bf16(o) : o;
        }
    }
}

void orc_dequantize_rows(int64_t nrows, const uint8_t* codes, const float* scales,
                         double* out) {
    int64_t r;
#pragma omp parallel for schedule(static)
    for (r = 0; r < nrows; ++r) {
        int d;
        for (d = 0; d < 128; ++d)
            out[r * 128 + d] = orc_e4m3_decode(codes[r * 128 + d]) * (double)scales[r];
    }
}

/* ------------------------------------------------------------------------
 * Lightning-indexer score [P1 formula I[t,s]; P3 equation S^I; P4
 * Indexer.forward fp8_index call]:
 *   I[t,s] = sum_h w[t,h] * ReLU(q[t,h] . k[s])
 * evaluated in double on the values given (the dequantised FP8 values in
 * the quantised path). Constant factors (H^-0.5, the 128^-0.5 score scale,
 * q's block scale) are the caller's: they are folded into w, as the page
 * folds them into `weights`. Causality: a query at position pos sees keys
 * 0..pos, its own key included (the key is written to the cache before
 * scoring), so n_valid = pos + 1.
 * Pinned by: closed forms for one-hot weights, all-positive dots (a
 * matrix-vector identity), all-negative dots (zero), head/dim permutation
 * invariance, and brute force against an independent formulation.
 * ---------------------------------------------------------------------- */
void orc_indexer_scores(int B, int S, int H, int D, int Lmax, const double* q,
                        const double* w, const double* k, const int32_t* n_valid,
                        double* out) {
    int64_t r, nrows = (int64_t)B * S;
    /* The (row, key) entries are independent. With at least as many rows as
     * threads the rows are shared out; with fewer (a decode step) each row's
     * keys are, so every thread works either way. The arithmetic of an entry
     * is the same in both cases. */
    const int by_rows = nrows >= orc_num_threads();
#pragma omp parallel for schedule(dynamic, 1) if (by_rows)
    for (r = 0; r < nrows; ++r) {
        int64_t b = r / S;
        const double* qr = q + r * H * D;
        const double* wr = w + r * H;
        const double* kb = k + b * (int64_t)Lmax * D;
        int s;
#pragma omp parallel for schedule(static) if (!by_rows)
        for (s = 0; s < n_valid[r]; ++s) {
            const double* ks = kb + (int64_t)s * D;
            double total = 0.0;
            int h;
            for (h = 0; h < H; ++h) {
                double dot = 0.0;
                int d;
                for (d = 0; d < D; ++d) dot += qr[h * D + d] * ks[d];
                if (dot > 0.0) total += wr[h] * dot;
            }
            out[r * (int64_t)Lmax + s] = total;
        }
    }
}

/* ------------------------------------------------------------------------
 * Causal top-k [P3 "a lightning indexer chooses up to 2,048 positions for
 * each query", selection mask M^sel over top_2048; P4 topk(min(index_topk,
 * end_pos))]. Reading: k_eff = min(K, n_valid) for every row (a prefill row
 * t selects among its own t+1 causal keys); the total order is (score
 * descending, position ascending), so equal scores keep the lower position;
 * -0 and +0 compare equal. The selected positions are returned in ascending
 * order (the page only scatters them into a mask, so order carries no
 * meaning) and the row is padded with -1.
 * Pinned by: a full sort from an independent library routine on small rows,
 * all-equal scores, K >= n_valid, duplicate scores, permutation of values.
 * ---------------------------------------------------------------------- */
typedef struct { double v; int32_t i; } scored_pos;

static int by_score_then_pos(const void* pa, const void* pb) {
    const scored_pos* a = (const scored_pos*)pa;
    const scored_pos* b = (const scored_pos*)pb;
    if (a->v > b->v) return -1;
    if (a->v < b->v) return 1;
    return (a->i < b->i) ? -1 : (a->i > b->i) ? 1 : 0;
}

static int by_pos(const void* pa, const void* pb) {
    int32_t a = *(const int32_t*)pa, b = *(const int32_t*)pb;
    return (a < b) ? -1 : (a > b) ? 1 : 0;
}

void orc_topk(int64_t nrows, int64_t ld, const double* scores, const int32_t* n_valid,
              int K, int32_t* idx) {
    int64_t r;
#pragma omp parallel for schedule(dynamic, 1)
    for (r = 0; r < nrows; ++r) {
        int n = n_valid[r], keff = n < K ? n : K, j;
        scored_pos* tmp = (scored_pos*)malloc(sizeof(scored_pos) * (size_t)(n > 0 ? n : 1));
        int32_t* out = idx + r * K;
        for (j = 0; j < n; ++j) {
            tmp[j].v = scores[r * ld + j];
            tmp[j].i = j;
        }
        qsort(tmp, (size_t)n, sizeof(scored_pos), by_score_then_pos);
        for (j = 0; j < keff; ++j) out[j] = tmp[j].i;
        qsort(out, (size_t)keff, sizeof(int32_t), by_pos);
        for (j = keff; j < K; ++j) out[j] = -1;
        free(tmp);
    }
}

/* ------------------------------------------------------------------------
 * Sparse latent attention, absorbed (MQA) form [P5 MLA decode excerpt:
 * scores = (q_nope_absorbed . kv_cache + q_pe . pe_cache) * softmax_scale,
 * index mask, softmax, scores . kv_cache; P3 S' = S m^2/sqrt(192), softmax,
 * O = AV; P3 "attention runs over those alone"]. The index mask makes every
 * non-selected position contribute exp(-inf) = 0, so the softmax is taken
 * over the selected positions only. The output is the latent-space result
 * (before the value up-projection). The scale is the caller's (192^-0.5,
 * times m^2 when the YaRN correction applies). Evaluated in double with the
 * maximum subtracted. A row with no selected position gives out = 0 and
 * lse = -inf.
 * Pinned by: dense recovery against PyTorch's scaled_dot_product_attention
 * when every position is selected, agreement with the non-absorbed form
 * below, equal logits giving the mean, one selected row giving that row,
 * invariance to the order of the indices.
 * ---------------------------------------------------------------------- */
void orc_sparse_mla(int B, int S, int Hq, int Dl, int Dr, int Lmax, int K,
                    const double* q, const double* latent, const double* kpe,
                    const int32_t* idx, double scale, double* out, double* lse) {
    int64_t task, ntask = (int64_t)B * S * Hq;
    int Dq = Dl + Dr;
    (void)Lmax;
#pragma omp parallel for schedule(dynamic, 4)
    for (task = 0; task < ntask; ++task) {
        int64_t r = task / Hq;
        int h = (int)(task % Hq);
        int64_t b = r / S;
        const double* qh = q + (r * Hq + h) * Dq;
        const int32_t* sel = idx + r * K;
        double* z = (double*)malloc(sizeof(double) * (size_t)K);
        double* o = out + (r * Hq + h) * Dl;
        double m = -INFINITY, l = 0.0;
        int j, d;
        for (j = 0; j < K; ++j) {
            const double* c;
            const double* pe;
            double dot = 0.0;
            if (sel[j] < 0) continue;
            c = latent + (b * Lmax + sel[j]) * Dl;
            pe = kpe + (b * Lmax + sel[j]) * Dr;
            for (d = 0; d < Dl; ++d) dot += qh[d] * c[d];
            for (d = 0; d < Dr; ++d) dot += qh[Dl + d] * pe[d];
            z[j] = scale * dot;
            if (z[j] > m) m = z[j];
        }
        for (d = 0; d < Dl; ++d) o[d] = 0.0;
        if (m == -INFINITY) {
            if (lse) lse[r * Hq + h] = -INFINITY;
            free(z);
            continue;
        }
        for (j = 0; j < K; ++j) {
            const double* c;
            double p;
            if (sel[j] < 0) continue;
            c = latent + (b * Lmax + sel[j]) * Dl;
            p = exp(z[j] - m);
            l += p;
            for (d = 0; d < Dl; ++d) o[d] += p * c[d];
        }
        for (d = 0; d < Dl; ++d) o[d] /= l;
        if (lse) lse[r * Hq + h] = m + log(l);
        free(z);
    }
}

/* ------------------------------------------------------------------------
 * Non-absorbed (multi-head) form [P2 MLA prefill excerpt: kv = wkv_b(kv)
 * split into k_nope and v per head, k = [k_nope ; k_pe], scores = q . k *
 * softmax_scale, index mask, softmax, scores . v]. Restricted to the same
 * selected set. Used only to cross-check the absorbed form: applying W_UK to
 * the query and W_UV to the latent output gives the same result.
 * ---------------------------------------------------------------------- */
void orc_mla_mha(int B, int S, int Hq, int Dn, int Dv, int Dl, int Dr, int Lmax,
                 int K, const double* q_nope, const double* q_pe,
                 const double* wkv_b, const double* latent, const double* kpe,
                 const int32_t* idx, double scale, double* out) {
    int64_t task, ntask = (int64_t)B * S * Hq;
#pragma omp parallel for schedule(dynamic, 1)
    for (task = 0; task < ntask; ++task) {
        int64_t r = task / Hq;
        int h = (int)(task % Hq);
        int64_t b = r / S;
        const double* qn = q_nope + (r * Hq + h) * Dn;
        const double* qp = q_pe + (r * Hq + h) * Dr;
        const double* W = wkv_b + (int64_t)h * (Dn + Dv) * Dl; /* [Dn+Dv][Dl] */
        const int32_t* sel = idx + r * K;
        double* z = (double*)malloc(sizeof(double) * (size_t)K);
        double* v = (double*)malloc(sizeof(double) * (size_t)K * Dv);
        double* o = out + (r * Hq + h) * Dv;
        double m = -INFINITY, l = 0.0;
        int j, d, e;
        for (j = 0; j < K; ++j) {
            const double* c;
            const double* pe;
            double dot = 0.0;
            if (sel[j] < 0) continue;
            c = latent + (b * Lmax + sel[j]) * Dl;
            pe = kpe + (b * Lmax + sel[j]) * Dr;
            for (d = 0; d < Dn; ++d) {
                double kn = 0.0;
                for (e = 0; e < Dl; ++e) kn += W[(int64_t)d * Dl + e] * c[e];
                dot += qn[d] * kn;
            }
            for (d = 0; d < Dr; ++d) dot += qp[d] * pe[d];
            for (d = 0; d < Dv; ++d) {
                double vv = 0.0;
                for (e = 0; e < Dl; ++e) vv += W[(int64_t)(Dn + d) * Dl + e] * c[e];
                v[(int64_t)j * Dv + d] = vv;
            }
            z[j] = scale * dot;
            if (z[j] > m) m = z[j];
        }
        for (d = 0; d < Dv; ++d) o[d] = 0.0;
        if (m != -INFINITY) {
            for (j = 0; j < K; ++j) {
                double p;
                if (sel[j] < 0) continue;
                p = exp(z[j] - m);
                l += p;
                for (d = 0; d < Dv; ++d) o[d] += p * v[(int64_t)j * Dv + d];
            }
            for (d = 0; d < Dv; ++d) o[d] /= l;
        }
        free(z);
        free(v);
    }
}

/* ------------------------------------------------------------------------
 * Multi-head (non-absorbed) prefill attention over per-head keys and values
 * that are already up-projected [P2 MLA prefill excerpt: k = [k_nope ;
 * k_pe broadcast over heads], scores = q . k * softmax_scale, plus the index
 * mask (0 at the selected positions, -inf elsewhere, built by scattering the
 * top-k list) and the causal mask, softmax over positions, scores . v].
 * The selection is a set, as the scattered mask makes it: a position listed
 * twice counts once. Position p of row r = (b, s) takes part iff it appears in
 * idx[r], 0 <= p < Lmax, and (when pos is given) p <= pos[r]. A row with no
 * such position gives out = 0.
 * q [B][S][Hq][Dn+Dr] (q_nope then q_pe), kv [B][Lmax][Hq][Dn+Dv] (k_nope
 * then v), kpe [B][Lmax][Dr], idx [B][S][K], pos [B][S] or NULL,
 * out [B][S][Hq][Dv].
 * Pinned by: with kv from the up-projection it equals orc_mla_mha (which
 * equals the absorbed form, itself pinned to PyTorch's attention); masking
 * by position against a dense masked softmax written with PyTorch.
 * ---------------------------------------------------------------------- */
void orc_sparse_mha(int B, int S, int Hq, int Dn, int Dv, int Dr, int Lmax, int K,
                    const double* q, const double* kv, const double* kpe,
                    const int32_t* idx, const int32_t* pos, double scale, double* out) {
    int64_t r, nrows = (int64_t)B * S;
    const int Dq = Dn + Dr, Dkv = Dn + Dv;
#pragma omp parallel for schedule(dynamic, 1)
    for (r = 0; r < nrows; ++r) {
        int64_t b = r / S;
        const int32_t* sel = idx + r * K;
        unsigned char* in_mask = (unsigned char*)calloc((size_t)Lmax, 1);
        double* z = (double*)malloc(sizeof(double) * (size_t)Lmax);
        int j, p, h, d;
        for (j = 0; j < K; ++j) {
            p = sel[j];
            if (p < 0 || p >= Lmax) continue;
            if (pos != NULL && p > pos[r]) continue;
            in_mask[p] = 1;
        }
        for (h = 0; h < Hq; ++h) {
            const double* qh = q + (r * Hq + h) * Dq;
            double* o = out + (r * Hq + h) * Dv;
            double m = -INFINITY, l = 0.0;
            for (p = 0; p < Lmax; ++p) {
                const double* kh;
                const double* pe;
                double dot = 0.0;
                if (!in_mask[p]) continue;
                kh = kv + ((b * Lmax + p) * Hq + h) * Dkv;
                pe = kpe + (b * Lmax + p) * Dr;
                for (d = 0; d < Dn; ++d) dot += qh[d] * kh[d];
                for (d = 0; d < Dr; ++d) dot += qh[Dn + d] * pe[d];
                z[p] = scale * dot;
                if (z[p] > m) m = z[p];
            }
            for (d = 0; d < Dv; ++d) o[d] = 0.0;
            if (m == -INFINITY) continue;
            for (p = 0; p < Lmax; ++p) {
                const double* vh;
                double w;
                if (!in_mask[p]) continue;
                vh = kv + ((b * Lmax + p) * Hq + h) * Dkv + Dn;
                w = exp(z[p] - m);
                l += w;
                for (d = 0; d < Dv; ++d) o[d] += w * vh[d];
            }
            for (d = 0; d < Dv; ++d) o[d] /= l;
        }
        free(z);
        free(in_mask);
    }
}
