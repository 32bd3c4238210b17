// indexer.hip -- lightning-indexer kernels for gfx950.
//
// Method (aipricedb digest, indexer formula; page "Sparse latent
// attention", equation S^I; page "Rotate first features", Indexer.forward):
//   I[t,s] = sum_h w[t,h] * ReLU(q[t,h] . k[s]),   64 heads x 128 features,
// q and k rotated on features 0..63 with the non-interleaved pairing
// (j, j+32) in float32, cast back to the activation dtype, then block-FP8
// quantised (one float32 scale per 128 features, OCP E4M3 codes).
//
// Kernels:
//   prepare_rows_kernel  one wave per 128-feature row: RoPE, cast, amax,
//                        scale, E4M3 encode; q rows go to q_fp8/q_scale,
//                        k rows are appended to k_cache/k_scale at pos.
//   score_rows_kernel    few query rows per batch row: one block per (row,
//                        key block), q codes of the row in registers.
//   score_tile_kernel    many query rows: 64 queries x 128 keys per block,
//                        per-head GEMM tiles on the bf16 MFMA with the key
//                        codes held in registers across all heads.
//   decode_score_kernel  one query row per batch row, fused with prepare.
// Codes are converted exactly to bf16 and multiplied on the bf16 MFMA
// (products of E4M3 values are exact in float32); the epilogue applies ReLU,
// the per-head weight w*q_scale, the head sum and the key's scale.
#include "dsa_common.h"

namespace dsa {

// ---------------------------------------------------------------------------
// prepare: RoPE (non-interleaved, first 64 features) + cast + block FP8.
// Lane l holds features l and l+64 of its row; the rotation pairs feature j
// (lane j) with j+32 (lane j+32), exchanged with one cross-lane swap. Each
// wave handles kPrepRows consecutive rows and issues all their loads (pos,
// then table entries and inputs) together, so the dependent global round
// trips are paid once per kPrepRows rows.
// Options: `had` replaces the rotated row by H_128 x / sqrt(128) (fast
// Walsh-Hadamard transform in float32, butterfly strides 1..32 across lanes
// and 64 inside the lane, then a multiplication by fl32(128^-0.5), rounded
// to the activation dtype); `pow2` rounds the block scale up to a power of
// two.
// ---------------------------------------------------------------------------
constexpr int kPrepRows = 8;
constexpr float kInvSqrt128 = 0.088388347648318440550f;   // fl32(128^-0.5)

// smallest power of two >= v (v > 0, finite)
__device__ __forceinline__ float pow2_ceil(float v) {
    uint32_t u = __float_as_uint(v);
    const uint32_t e = u >> 23, m = u & 0x7FFFFFu;
    if (e == 0u) {                                  // subnormal
        if (m & (m - 1u)) u = 1u << (32 - __clz(static_cast<int>(m)));
    } else if (m != 0u) {
        u = (e + 1u) << 23;
    }
    return __uint_as_float(u);
}

// one stride of the Walsh-Hadamard butterfly on features lane (a) and
// lane + 64 (c): (x[i], x[i+s]) -> (x[i] + x[i+s], x[i] - x[i+s])
__device__ __forceinline__ void wht_step(float& a, float& c, int lane, int s) {
    const float pa = __shfl_xor(a, s), pc = __shfl_xor(c, s);
    const bool upper = (lane & s) != 0;
    a = upper ? pa - a : a + pa;
    c = upper ? pc - c : c + pc;
}

template <bool BF16_IN, bool TO_CACHE>
__global__ __launch_bounds__(256) void prepare_rows_kernel(
    int64_t nrows, int rows_per_pos, int S, int Lmax, int P, const void* __restrict__ x,
    const int32_t* __restrict__ pos, const float* __restrict__ cos_t,
    const float* __restrict__ sin_t, uint8_t* __restrict__ codes_out,
    float* __restrict__ scales_out, int had, int pow2, CacheMap cmap) {
    const int lane = threadIdx.x & 63;
    const int64_t row0 = (static_cast<int64_t>(blockIdx.x) * 4 + (threadIdx.x >> 6)) * kPrepRows;
    if (row0 >= nrows) return;
    const int j = lane & 31;

    int p[kPrepRows];
    float x0[kPrepRows], x1[kPrepRows];
#pragma unroll
    for (int k = 0; k < kPrepRows; ++k) {
        const int64_t row = row0 + k;
        const bool ok = row < nrows;
        p[k] = ok ? pos[row / rows_per_pos] : -1;
        if (BF16_IN) {
            const uint16_t* xr = static_cast<const uint16_t*>(x) + (ok ? row : 0) * 128;
            x0[k] = bf16_bits_to_float(xr[lane]);
            x1[k] = bf16_bits_to_float(xr[lane + 64]);
        } else {
            const float* xr = static_cast<const float*>(x) + (ok ? row : 0) * 128;
            x0[k] = xr[lane];
            x1[k] = xr[lane + 64];
        }
    }
    float cs[kPrepRows], sn[kPrepRows];
#pragma unroll
    for (int k = 0; k < kPrepRows; ++k) {
        const bool ok = p[k] >= 0 && p[k] < Lmax && p[k] < P;
        const int64_t pe = ok ? p[k] : 0;
        cs[k] = cos_t[pe * 32 + j];
        sn[k] = sin_t[pe * 32 + j];
    }
#pragma unroll
    for (int k = 0; k < kPrepRows; ++k) {
        const int64_t row = row0 + k;
        if (row >= nrows) break;                   // wave-uniform
        if (!(p[k] >= 0 && p[k] < Lmax && p[k] < P)) continue;
        const float other = __shfl_xor(x0[k], 32);
        float y0;
        {
#pragma clang fp contract(off)
            // pair (a, b) = (x[j], x[j+32]):  a' = a c - b s,  b' = a s + b c
            if (lane < 32) {
                const float ac = x0[k] * cs[k], bs = other * sn[k];
                y0 = ac - bs;
            } else {
                const float as = other * sn[k], bc = x0[k] * cs[k];
                y0 = as + bc;
            }
        }
        if (BF16_IN) y0 = bf16_bits_to_float(float_to_bf16_bits(y0));   // cast back to bf16
        float y1 = x1[k];
        if (had) {
#pragma unroll
            for (int st = 1; st < 64; st <<= 1) wht_step(y0, y1, lane, st);
            const float t = y0 + y1;
            y1 = y0 - y1;
            y0 = t * kInvSqrt128;
            y1 = y1 * kInvSqrt128;
            if (BF16_IN) {
                y0 = bf16_bits_to_float(float_to_bf16_bits(y0));
                y1 = bf16_bits_to_float(float_to_bf16_bits(y1));
            }
        }

        const float amax = wave_max_dpp(fmaxf(fabsf(y0), fabsf(y1)));
        float scale = amax / 448.0f;
        if (pow2) scale = scale > 0.0f ? pow2_ceil(scale) : 1.0f;
        else if (!(scale > 0.0f)) scale = 1.0f;
        const uint8_t c0 = e4m3_encode(y0 / scale);
        const uint8_t c1 = e4m3_encode(y1 / scale);

        int64_t dst;
        if (TO_CACHE) {
            const int64_t b = (row / rows_per_pos) / S;
            dst = cmap.row(b, p[k]);
            if (dst < 0) continue;                  // page not present: nothing to write
        } else {
            dst = row;
        }
        codes_out[dst * 128 + lane] = c0;
        codes_out[dst * 128 + lane + 64] = c1;
        if (lane == 0) scales_out[dst] = scale;
    }
}

hipError_t launch_prepare(bool bf16_in, bool to_cache, int64_t nrows, int rows_per_pos, int S,
                          int Lmax, int P, const void* x, const int32_t* pos, const float* cos_t,
                          const float* sin_t, uint8_t* codes, float* scales, bool hadamard,
                          bool pow2, CacheMap cmap, hipStream_t stream) {
    if (nrows <= 0) return hipSuccess;
    const dim3 grid(static_cast<unsigned>((nrows + 4 * kPrepRows - 1) / (4 * kPrepRows))),
        block(256);
#define DSA_PREP(B, C)                                                                         \
    hipLaunchKernelGGL((prepare_rows_kernel<B, C>), grid, block, 0, stream, nrows, rows_per_pos, \
                       S, Lmax, P, x, pos, cos_t, sin_t, codes, scales, hadamard ? 1 : 0,       \
                       pow2 ? 1 : 0, cmap)
    if (bf16_in) {
        if (to_cache) DSA_PREP(true, true); else DSA_PREP(true, false);
    } else {
        if (to_cache) DSA_PREP(false, true); else DSA_PREP(false, false);
    }
#undef DSA_PREP
    return hipGetLastError();
}

// ---------------------------------------------------------------------------
// score (few query rows per batch row): block = 4 waves, covers 64*U
// consecutive keys of one query row. MFMA 16x16x32 bf16, M = 16 heads,
// N = 16 keys, K = 32 features; four K-steps cover the 128 features and four
// head groups cover 64 heads. Operand lane layout: lane (m = l%16, g = l/16)
// supplies row m, feature chunk g; both operands use feature 32g + 8kk + j
// for MFMA kk, element j. Result lane layout: lane (n = l%16, g) holds heads
// 4g..4g+3 of key n.
// ---------------------------------------------------------------------------
template <int U>
__global__ __launch_bounds__(256) void score_rows_kernel(
    int S, int H, int Lmax, int P, const uint8_t* __restrict__ q8,
    const float* __restrict__ qscale, const float* __restrict__ w,
    const int32_t* __restrict__ pos, const uint8_t* __restrict__ kcache,
    const float* __restrict__ kscale, float* __restrict__ scores, int64_t ld, CacheMap cmap) {
    const int row = blockIdx.y;
    const int p = pos[row];
    if (p < 0 || p >= Lmax || p >= P) return;
    const int n_valid = p + 1;
    const int kblock0 = blockIdx.x * (64 * U);
    if (kblock0 >= n_valid) return;

    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int m = lane & 15, g = lane >> 4;
    const int64_t b = row / S;
    const int wkey0 = kblock0 + wave * 16 * U;

    // key loads first; ks = -inf marks a key whose page is not present
    uint4 kraw[U][2];
    float ks[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
        int key = wkey0 + u * 16 + m;
        key = key < n_valid ? key : n_valid - 1;
        const int64_t krow = cmap.row(b, key);
        const uint4* src =
            reinterpret_cast<const uint4*>(kcache + (krow >= 0 ? krow : 0) * 128 + g * 32);
        kraw[u][0] = src[0];
        kraw[u][1] = src[1];
        ks[u] = krow >= 0 ? kscale[krow] : -INFINITY;
    }
    bf16x8 qa[4][4];
    float wq[4][4];
#pragma unroll
    for (int hg = 0; hg < 4; ++hg) {
        const int h = hg * 16 + m;
        if (h < H) {
            const uint4* src = reinterpret_cast<const uint4*>(
                q8 + (static_cast<int64_t>(row) * H + h) * 128 + g * 32);
            const uint4 lo = src[0], hi = src[1];
            qa[hg][0] = e4m3x8_to_bf16x8(lo.x, lo.y);
            qa[hg][1] = e4m3x8_to_bf16x8(lo.z, lo.w);
            qa[hg][2] = e4m3x8_to_bf16x8(hi.x, hi.y);
            qa[hg][3] = e4m3x8_to_bf16x8(hi.z, hi.w);
        } else {
#pragma unroll
            for (int kk = 0; kk < 4; ++kk)
#pragma unroll
                for (int e = 0; e < 8; ++e) qa[hg][kk][e] = static_cast<__bf16>(0.0f);
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int hh = hg * 16 + 4 * g + i;
            wq[hg][i] = hh < H ? w[static_cast<int64_t>(row) * H + hh] *
                                     qscale[static_cast<int64_t>(row) * H + hh]
                               : 0.0f;
        }
    }
    float* out = scores + static_cast<int64_t>(row) * ld;
#pragma unroll
    for (int u = 0; u < U; ++u) {
        const int key0 = wkey0 + u * 16;
        if (key0 >= n_valid) break;
        bf16x8 kbf[4];
        kbf[0] = e4m3x8_to_bf16x8(kraw[u][0].x, kraw[u][0].y);
        kbf[1] = e4m3x8_to_bf16x8(kraw[u][0].z, kraw[u][0].w);
        kbf[2] = e4m3x8_to_bf16x8(kraw[u][1].x, kraw[u][1].y);
        kbf[3] = e4m3x8_to_bf16x8(kraw[u][1].z, kraw[u][1].w);
        float part = 0.0f;
#pragma unroll
        for (int hg = 0; hg < 4; ++hg) {
            v4f acc = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
            for (int kk = 0; kk < 4; ++kk) acc = mfma_bf16_16x16x32(qa[hg][kk], kbf[kk], acc);
#pragma unroll
            for (int i = 0; i < 4; ++i) part += wq[hg][i] * fmaxf(acc[i], 0.0f);
        }
        part += __shfl_xor(part, 16);
        part += __shfl_xor(part, 32);
        const int key = key0 + m;
        if (g == 0 && key < n_valid) out[key] = ks[u] == -INFINITY ? -INFINITY : part * ks[u];
    }
}

// ---------------------------------------------------------------------------
// score (many query rows): block = 4 waves, a tile of 64 queries (of one
// batch row) x 64 kKW keys; wave w covers queries 32 (w & 1) .. +31 and
// keys 32 kKW (w >> 1) .. +32 kKW - 1. Per head h the block's 64 query rows of codes are
// converted to bf16 into LDS (double-buffered: head h+1 is staged while h is
// multiplied) and each wave runs
//   S_h = Q_h K^T    bf16 MFMA 32x32x16, M = 32 queries, N = 32 keys (two
//                    key tiles), K = 16 features, eight K-steps;
// the wave's key codes stay in registers as bf16 B operands for all heads.
// Epilogue per head: I += (w q_scale)[t,h] * ReLU(S_h[t,s]); after the last
// head I is scaled by the key's scale and stored for s < n_valid(t).
// Lane layouts of the 32x32x16 MFMA: A/B lane l supplies row/column l%32,
// features 8 (l/32) + j; result element i of lane l is row
// 8 (i/4) + 4 (l/32) + i%4, column l%32.
// Launch order: block L runs on XCD L % 8 and every XCD works through whole
// query tiles (all their key tiles back to back), so a tile's query codes
// are reused from that XCD's L2.
// ---------------------------------------------------------------------------
typedef float v16f __attribute__((ext_vector_type(16)));
#ifndef DSA_TILE_KW
#define DSA_TILE_KW 2
#endif
#ifndef DSA_TILE_OCC
#define DSA_TILE_OCC 2
#endif
constexpr int kKW = DSA_TILE_KW;            // 32-key tiles per wave
constexpr int kQT = 64, kKT = 64 * kKW;     // queries, keys per block tile
constexpr int kQsStride = 128 + 8;          // bf16 per staged query row (bank stagger)

__device__ __forceinline__ v16f mfma_bf16_32x32x16(bf16x8 a, bf16x8 b, v16f c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

__global__ __launch_bounds__(256, DSA_TILE_OCC) void score_tile_kernel(
    int B, int S, int H, int Lmax, int P, int nqt, int nkt, const uint8_t* __restrict__ q8,
    const float* __restrict__ qscale, const float* __restrict__ w,
    const int32_t* __restrict__ pos, const uint8_t* __restrict__ kcache,
    const float* __restrict__ kscale, float* __restrict__ scores, int64_t ld, CacheMap cmap) {
    __shared__ __align__(16) uint16_t Qs[2][kQT][kQsStride];
    __shared__ __align__(16) float wqs[64][kQT];       // [head][query] w * q_scale
    __shared__ int nv[kQT];                            // n_valid per query of the tile
    __shared__ int s_maxnv;

    const int L = blockIdx.x;
    const int jx = L / 8;
    const int qtile = (jx / nkt) * 8 + (L & 7);
    const int kt = jx % nkt;
    if (qtile >= B * nqt) return;
    const int b = qtile / nqt;
    const int t0 = (qtile - b * nqt) * kQT;
    const int k0 = kt * kKT;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int64_t row0 = static_cast<int64_t>(b) * S + t0;

    if (tid == 0) s_maxnv = 0;
    __syncthreads();
    if (tid < kQT) {
        int n = 0;
        if (t0 + tid < S) {
            const int p = pos[row0 + tid];
            n = (p >= 0 && p < Lmax && p < P) ? p + 1 : 0;
        }
        nv[tid] = n;
        atomicMax(&s_maxnv, n);
    }
    __syncthreads();
    if (k0 >= s_maxnv) return;                         // tile wholly past every causal end

    // per-head query weights
    for (int i = tid; i < 64 * kQT; i += 256) {
        const int h = i / kQT, qi = i - h * kQT;
        float v = 0.0f;
        if (h < H && t0 + qi < S) {
            const int64_t r = row0 + qi;
            v = w[r * H + h] * qscale[r * H + h];
        }
        wqs[h][qi] = v;
    }

    // the wave's key codes as bf16 B operands (two key tiles x eight K-steps)
    const int wq_i = wave & 1, wk = wave >> 1;
    const int hi32 = lane >> 5, l32 = lane & 31;
    bf16x8 kb[kKW][8];
    float ksc[kKW];            // key scale; -inf marks a key whose page is not present
#pragma unroll
    for (int kt2 = 0; kt2 < kKW; ++kt2) {
        int key = k0 + wk * 32 * kKW + kt2 * 32 + l32;
        key = key < Lmax ? key : Lmax - 1;
        const int64_t krow = cmap.row(b, key);
        const uint8_t* kr = kcache + (krow >= 0 ? krow : 0) * 128 + 8 * hi32;
#pragma unroll
        for (int ks = 0; ks < 8; ++ks) {
            const uint2 c = *reinterpret_cast<const uint2*>(kr + 16 * ks);
            kb[kt2][ks] = e4m3x8_to_bf16x8(c.x, c.y);
        }
        ksc[kt2] = krow >= 0 ? kscale[krow] : -INFINITY;
    }

    // staging: thread -> query tid/4, 32 features (tid%4)
    const int sq = tid >> 2, sc = tid & 3;
    const bool sq_ok = t0 + sq < S;
    const uint8_t* qsrc = q8 + (row0 + sq) * H * 128 + 32 * sc;
    uint4 raw0 = make_uint4(0u, 0u, 0u, 0u), raw1 = raw0;
    auto fetch_q = [&](int h) {
        if (sq_ok) {
            const uint4* src = reinterpret_cast<const uint4*>(qsrc + static_cast<int64_t>(h) * 128);
            raw0 = src[0];
            raw1 = src[1];
        }
    };
    auto stage_q = [&](int buf) {
        uint16_t* dst = &Qs[buf][sq][32 * sc];
        *reinterpret_cast<bf16x8*>(dst + 0) = e4m3x8_to_bf16x8(raw0.x, raw0.y);
        *reinterpret_cast<bf16x8*>(dst + 8) = e4m3x8_to_bf16x8(raw0.z, raw0.w);
        *reinterpret_cast<bf16x8*>(dst + 16) = e4m3x8_to_bf16x8(raw1.x, raw1.y);
        *reinterpret_cast<bf16x8*>(dst + 24) = e4m3x8_to_bf16x8(raw1.z, raw1.w);
    };

    v16f I[kKW];
#pragma unroll
    for (int kt2 = 0; kt2 < kKW; ++kt2)
#pragma unroll
        for (int i = 0; i < 16; ++i) I[kt2][i] = 0.0f;
    const uint16_t* arow = &Qs[0][wq_i * 32 + l32][8 * hi32];
    constexpr int kBufStride = kQT * kQsStride;
    fetch_q(0);
    for (int h = 0; h < H; ++h) {
        const int buf = h & 1;
        stage_q(buf);
        if (h + 1 < H) fetch_q(h + 1);
        __syncthreads();
        v16f sacc[kKW];
#pragma unroll
        for (int kt2 = 0; kt2 < kKW; ++kt2)
#pragma unroll
            for (int i = 0; i < 16; ++i) sacc[kt2][i] = 0.0f;
#pragma unroll
        for (int ks = 0; ks < 8; ++ks) {
            const bf16x8 a = *reinterpret_cast<const bf16x8*>(arow + buf * kBufStride + 16 * ks);
#pragma unroll
            for (int kt2 = 0; kt2 < kKW; ++kt2)
                sacc[kt2] = mfma_bf16_32x32x16(a, kb[kt2][ks], sacc[kt2]);
        }
        // result rows of lane: 8 r + 4 hi32 + c (r, c < 4); their weights
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const float4 wv = *reinterpret_cast<const float4*>(&wqs[h][wq_i * 32 + 8 * r + 4 * hi32]);
            const float wr[4] = {wv.x, wv.y, wv.z, wv.w};
#pragma unroll
            for (int c = 0; c < 4; ++c)
#pragma unroll
                for (int kt2 = 0; kt2 < kKW; ++kt2)
                    I[kt2][4 * r + c] += wr[c] * fmaxf(sacc[kt2][4 * r + c], 0.0f);
        }
    }

    // store the valid prefix of every query row
#pragma unroll
    for (int kt2 = 0; kt2 < kKW; ++kt2) {
        const int key = k0 + wk * 32 * kKW + kt2 * 32 + l32;
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            const int qi = wq_i * 32 + 8 * (i >> 2) + 4 * hi32 + (i & 3);
            if (key < nv[qi]) {
                const float v = ksc[kt2] == -INFINITY ? -INFINITY : I[kt2][i] * ksc[kt2];
                scores[(row0 + qi) * ld + key] = v;
            }
        }
    }
}

// ---------------------------------------------------------------------------
// Fused decode path (one query row per batch row): every block quantises its
// row's 64 query heads itself (into LDS) while its key loads are in flight,
// and the block that covers the row's own position also rotates, quantises
// and appends the new key, using it straight from LDS. One launch replaces
// prepare(k) + prepare(q) + score.
// Query quantisation layout: thread t owns head t/4, quarter t%4 of the 128
// features; quarters 0/1 hold rotary pairs (j, j+32) for j in [16q, 16q+16),
// quarters 2/3 hold features 64..95 / 96..127. The head's amax is reduced
// over its four threads.
// ---------------------------------------------------------------------------
template <bool BF16_IN>
__device__ __forceinline__ float load_act(const void* base, int64_t i) {
    if (BF16_IN) return bf16_bits_to_float(static_cast<const uint16_t*>(base)[i]);
    return static_cast<const float*>(base)[i];
}

template <bool BF16_IN>
__device__ __forceinline__ float round_act(float v) {
    return BF16_IN ? bf16_bits_to_float(float_to_bf16_bits(v)) : v;
}

template <int U, bool BF16_IN>
__global__ __launch_bounds__(256) void decode_score_kernel(
    int H, int Lmax, int P, const void* __restrict__ q_raw, const void* __restrict__ k_raw,
    const int32_t* __restrict__ pos, const float* __restrict__ cos_t,
    const float* __restrict__ sin_t, const float* __restrict__ w, uint8_t* __restrict__ kcache,
    float* __restrict__ kscale, uint8_t* __restrict__ q8_out, float* __restrict__ qs_out,
    float* __restrict__ scores, int64_t ld, CacheMap cmap) {
    __shared__ __align__(16) uint8_t qcodes[64 * 128];
    __shared__ float qscale[64];
    __shared__ __align__(16) uint8_t kcodes[128];
    __shared__ float kscale_new;

    const int row = blockIdx.y;
    const int p = pos[row];
    if (p < 0 || p >= Lmax || p >= P) return;
    const int n_valid = p + 1;
    const int kblock0 = blockIdx.x * (64 * U);
    if (kblock0 >= n_valid) return;

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int m = lane & 15, g = lane >> 4;
    const int64_t b = row;
    const int wkey0 = kblock0 + wave * 16 * U;
    const int64_t prow = cmap.row(b, p);                              // the new key's row
    const bool has_new = k_raw != nullptr && prow >= 0 && kblock0 + 64 * U > p;

    // 1. key loads first (the new key, if any, is taken from LDS later);
    // ks = -inf marks a key whose page is not present
    uint4 kraw[U][2];
    float ks[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
        int key = wkey0 + u * 16 + m;
        key = key < n_valid ? key : n_valid - 1;
        const int64_t krow = cmap.row(b, key);
        const uint4* src =
            reinterpret_cast<const uint4*>(kcache + (krow >= 0 ? krow : 0) * 128 + g * 32);
        kraw[u][0] = src[0];
        kraw[u][1] = src[1];
        ks[u] = krow >= 0 ? kscale[krow] : -INFINITY;
    }

    // 2. quantise the row's query heads into LDS
    {
#pragma clang fp contract(off)
        const int hh = tid >> 2, qt = tid & 3;
        float v[32];
        float amax = 0.0f;
        if (hh < H) {
            const int64_t base = (static_cast<int64_t>(row) * H + hh) * 128;
            if (qt < 2) {
                const int j0 = 16 * qt;
                const float* c = cos_t + static_cast<int64_t>(p) * 32 + j0;
                const float* sn = sin_t + static_cast<int64_t>(p) * 32 + j0;
#pragma unroll
                for (int j = 0; j < 16; ++j) {
                    const float a = load_act<BF16_IN>(q_raw, base + j0 + j);
                    const float bb = load_act<BF16_IN>(q_raw, base + j0 + j + 32);
                    const float ac = a * c[j], bs = bb * sn[j];
                    const float as = a * sn[j], bc = bb * c[j];
                    v[j] = round_act<BF16_IN>(ac - bs);
                    v[16 + j] = round_act<BF16_IN>(as + bc);
                }
            } else {
                const int f0 = 64 + 32 * (qt - 2);
#pragma unroll
                for (int j = 0; j < 32; ++j) v[j] = load_act<BF16_IN>(q_raw, base + f0 + j);
            }
#pragma unroll
            for (int j = 0; j < 32; ++j) amax = fmaxf(amax, fabsf(v[j]));
        }
        amax = fmaxf(amax, __shfl_xor(amax, 1));
        amax = fmaxf(amax, __shfl_xor(amax, 2));
        float scale = amax / 448.0f;
        if (!(scale > 0.0f)) scale = 1.0f;
        // 32 codes packed into two 16-byte LDS stores
        uint32_t pk[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            uint32_t word = 0;
#pragma unroll
            for (int e = 0; e < 4; ++e)
                word |= static_cast<uint32_t>(e4m3_encode(v[4 * i + e] / scale)) << (8 * e);
            pk[i] = hh < H ? word : 0u;
        }
        // quarters 0/1: features [16q, 16q+16) and [16q+32, 16q+48); 2/3: [32q, 32q+32)
        const int off0 = qt < 2 ? 16 * qt : 32 * qt;
        const int off1 = qt < 2 ? 16 * qt + 32 : 32 * qt + 16;
        uint4* dst0 = reinterpret_cast<uint4*>(qcodes + hh * 128 + off0);
        uint4* dst1 = reinterpret_cast<uint4*>(qcodes + hh * 128 + off1);
        *dst0 = make_uint4(pk[0], pk[1], pk[2], pk[3]);
        *dst1 = make_uint4(pk[4], pk[5], pk[6], pk[7]);
        if (qt == 0) qscale[hh] = hh < H ? scale : 0.0f;
    }
    // 3. the new key (block covering position p): wave 0, lane l holds l, l+64
    if (has_new && wave == 0) {
#pragma clang fp contract(off)
        const int64_t base = b * 128;
        const float x0 = load_act<BF16_IN>(k_raw, base + lane);
        const float x1 = load_act<BF16_IN>(k_raw, base + lane + 64);
        const float other = __shfl_xor(x0, 32);
        const int j = lane & 31;
        const float c = cos_t[static_cast<int64_t>(p) * 32 + j];
        const float sn = sin_t[static_cast<int64_t>(p) * 32 + j];
        float y0;
        if (lane < 32) {
            const float ac = x0 * c, bs = other * sn;
            y0 = ac - bs;
        } else {
            const float as = other * sn, bc = x0 * c;
            y0 = as + bc;
        }
        y0 = round_act<BF16_IN>(y0);
        const float amax = wave_max(fmaxf(fabsf(y0), fabsf(x1)));
        float scale = amax / 448.0f;
        if (!(scale > 0.0f)) scale = 1.0f;
        const uint8_t c0 = e4m3_encode(y0 / scale), c1 = e4m3_encode(x1 / scale);
        kcodes[lane] = c0;
        kcodes[lane + 64] = c1;
        uint8_t* kdst = kcache + prow * 128;
        kdst[lane] = c0;
        kdst[lane + 64] = c1;
        if (lane == 0) {
            kscale_new = scale;
            kscale[prow] = scale;
        }
    }
    __syncthreads();
    if (blockIdx.x == 0 && q8_out != nullptr) {
        for (int i = tid; i < H * 8; i += 256)
            reinterpret_cast<uint4*>(q8_out + static_cast<int64_t>(row) * H * 128)[i] =
                reinterpret_cast<const uint4*>(qcodes)[i];
        if (tid < H) qs_out[static_cast<int64_t>(row) * H + tid] = qscale[tid];
    }

    // 4. operands from LDS, MFMA stream (as score_kernel)
    bf16x8 qa[4][4];
    float wq[4][4];
#pragma unroll
    for (int hg = 0; hg < 4; ++hg) {
        const uint4* src = reinterpret_cast<const uint4*>(qcodes + (hg * 16 + m) * 128 + g * 32);
        const uint4 lo = src[0], hi = src[1];
        qa[hg][0] = e4m3x8_to_bf16x8(lo.x, lo.y);
        qa[hg][1] = e4m3x8_to_bf16x8(lo.z, lo.w);
        qa[hg][2] = e4m3x8_to_bf16x8(hi.x, hi.y);
        qa[hg][3] = e4m3x8_to_bf16x8(hi.z, hi.w);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int h = hg * 16 + 4 * g + i;
            wq[hg][i] = h < H ? w[static_cast<int64_t>(row) * H + h] * qscale[h] : 0.0f;
        }
    }
    float* out = scores + static_cast<int64_t>(row) * ld;
#pragma unroll
    for (int u = 0; u < U; ++u) {
        const int key0 = wkey0 + u * 16;
        if (key0 >= n_valid) break;
        const int key = key0 + m;
        float ksc = ks[u];
        if (has_new && key == p) {
            kraw[u][0] = reinterpret_cast<const uint4*>(kcodes + g * 32)[0];
            kraw[u][1] = reinterpret_cast<const uint4*>(kcodes + g * 32)[1];
            ksc = kscale_new;
        }
        bf16x8 kbf[4];
        kbf[0] = e4m3x8_to_bf16x8(kraw[u][0].x, kraw[u][0].y);
        kbf[1] = e4m3x8_to_bf16x8(kraw[u][0].z, kraw[u][0].w);
        kbf[2] = e4m3x8_to_bf16x8(kraw[u][1].x, kraw[u][1].y);
        kbf[3] = e4m3x8_to_bf16x8(kraw[u][1].z, kraw[u][1].w);
        float part = 0.0f;
#pragma unroll
        for (int hg = 0; hg < 4; ++hg) {
            v4f acc = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
            for (int kk = 0; kk < 4; ++kk) acc = mfma_bf16_16x16x32(qa[hg][kk], kbf[kk], acc);
#pragma unroll
            for (int i = 0; i < 4; ++i) part += wq[hg][i] * fmaxf(acc[i], 0.0f);
        }
        part += __shfl_xor(part, 16);
        part += __shfl_xor(part, 32);
        if (g == 0 && key < n_valid) out[key] = ksc == -INFINITY ? -INFINITY : part * ksc;
    }
}

hipError_t launch_decode_score(bool bf16_in, int B, int H, int Lmax, int P, const void* q_raw,
                               const void* k_raw, const int32_t* pos, const float* cos_t,
                               const float* sin_t, const float* w, uint8_t* kcache,
                               float* kscale, uint8_t* q8_out, float* qs_out, float* scores,
                               int64_t ld, CacheMap cmap, hipStream_t stream) {
    int U = 4;
    while (U > 1 && static_cast<int64_t>(B) * ((Lmax + 64 * U - 1) / (64 * U)) < 2048) U >>= 1;
    const dim3 grid(static_cast<unsigned>((Lmax + 64 * U - 1) / (64 * U)), static_cast<unsigned>(B));
#define DSA_DEC(UU, BF)                                                                          \
    hipLaunchKernelGGL((decode_score_kernel<UU, BF>), grid, dim3(256), 0, stream, H, Lmax, P,    \
                       q_raw, k_raw, pos, cos_t, sin_t, w, kcache, kscale, q8_out, qs_out,     \
                       scores, ld, cmap)
    if (bf16_in) {
        if (U == 4) DSA_DEC(4, true); else if (U == 2) DSA_DEC(2, true); else DSA_DEC(1, true);
    } else {
        if (U == 4) DSA_DEC(4, false); else if (U == 2) DSA_DEC(2, false); else DSA_DEC(1, false);
    }
#undef DSA_DEC
    return hipGetLastError();
}

// Few queries per batch row (decode-like calls): one block per (row, 64*U
// keys), U the largest that still gives enough blocks to fill the chip.
// More: 64-query x 128-key tiles.
constexpr int kRowsPathMaxS = 8;

hipError_t launch_score(int B, int S, int H, int Lmax, int P, const uint8_t* q8,
                        const float* qscale, const float* w, const int32_t* pos,
                        const uint8_t* kcache, const float* kscale, float* scores, int64_t ld,
                        CacheMap cmap, hipStream_t stream) {
    if (S <= kRowsPathMaxS) {
        const int64_t rows = static_cast<int64_t>(B) * S;
        int U = 4;
        while (U > 1 && rows * ((Lmax + 64 * U - 1) / (64 * U)) < 2048) U >>= 1;
        const dim3 grid(static_cast<unsigned>((Lmax + 64 * U - 1) / (64 * U)),
                        static_cast<unsigned>(rows));
#define DSA_ROWS(UU)                                                                           \
    hipLaunchKernelGGL((score_rows_kernel<UU>), grid, dim3(256), 0, stream, S, H, Lmax, P, q8, \
                       qscale, w, pos, kcache, kscale, scores, ld, cmap)
        if (U == 4) DSA_ROWS(4);
        else if (U == 2) DSA_ROWS(2);
        else DSA_ROWS(1);
#undef DSA_ROWS
        return hipGetLastError();
    }
    const int nqt = (S + kQT - 1) / kQT;
    const int nkt = (Lmax + kKT - 1) / kKT;
    const int64_t qtiles = static_cast<int64_t>(B) * nqt;
    const int64_t nblocks = ((qtiles + 7) / 8) * 8 * nkt;
    hipLaunchKernelGGL(score_tile_kernel, dim3(static_cast<unsigned>(nblocks)), dim3(256), 0,
                       stream, B, S, H, Lmax, P, nqt, nkt, q8, qscale, w, pos, kcache, kscale,
                       scores, ld, cmap);
    return hipGetLastError();
}

}  // namespace dsa
