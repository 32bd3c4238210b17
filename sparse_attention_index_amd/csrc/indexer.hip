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
// Lane l of a wave holds features [8c, 8c + 8), c = l % 16, of row l / 16 of
// a group of four rows (16-byte loads, 8-byte code stores). The rotation
// pairs feature j (chunk c < 4) with j + 32 (chunk c + 4): partner lanes
// differ by 4. The row's amax is reduced over its 16 lanes. Each wave handles
// kPrepGroups groups and issues all their loads (pos, then table entries and
// inputs) together, so the dependent global round trips are paid once per
// 4 kPrepGroups rows.
// Options: `had` replaces the rotated row by H_128 x / sqrt(128) (fast
// Walsh-Hadamard transform in float32, butterfly strides 1, 2, 4 inside the
// lane and 8 .. 64 across lanes, in that order, then a multiplication by
// fl32(128^-0.5), rounded to the activation dtype); `pow2` rounds the block
// scale up to a power of two.
// ---------------------------------------------------------------------------
constexpr int kPrepGroups = 2;
constexpr int kPrepRowsPerWave = 4 * kPrepGroups;
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

// one butterfly stride s (a lane-index bit: features differ by 8 s) of the
// Walsh-Hadamard transform across lanes: (x[i], x[i+s]) -> (x[i] + x[i+s],
// x[i] - x[i+s])
__device__ __forceinline__ void wht_lanes(float (&y)[8], int c, int s) {
    const bool upper = (c & s) != 0;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        const float pa = __shfl_xor(y[e], s);
        y[e] = upper ? pa - y[e] : y[e] + pa;
    }
}

// the same inside the lane for strides 1, 2, 4 of the feature index
__device__ __forceinline__ void wht_lane(float (&y)[8], int s) {
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        if ((e & s) == 0) {
            const float lo = y[e], hi = y[e + s];
            y[e] = lo + hi;
            y[e + s] = lo - hi;
        }
    }
}

template <bool BF16_IN, bool TO_CACHE>
__global__ __launch_bounds__(256) void prepare_rows_kernel(
    int64_t nrows, int rows_per_pos, int S, int Lmax, int P, const void* __restrict__ x,
    const int32_t* __restrict__ pos, const float* __restrict__ cos_t,
    const float* __restrict__ sin_t, uint8_t* __restrict__ codes_out,
    float* __restrict__ scales_out, int had, int pow2, CacheMap cmap) {
    const int lane = threadIdx.x & 63, c = lane & 15, rsub = lane >> 4;
    const int64_t row0 =
        (static_cast<int64_t>(blockIdx.x) * 4 + (threadIdx.x >> 6)) * kPrepRowsPerWave;
    if (row0 >= nrows) return;
    const bool rotary = c < 8;
    const int j0 = 8 * (c & 3);                    // rotary pair index of element 0

    int p[kPrepGroups];
    float xv[kPrepGroups][8];
#pragma unroll
    for (int gi = 0; gi < kPrepGroups; ++gi) {
        const int64_t row = row0 + 4 * gi + rsub;
        const bool ok = row < nrows;
        p[gi] = ok ? pos[row / rows_per_pos] : -1;
        const int64_t rr = ok ? row : 0;
        if (BF16_IN) {
            const uint4 v = *reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(x) +
                                                            rr * 128 + 8 * c);
            const uint32_t w4[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                xv[gi][2 * e] = __uint_as_float(w4[e] << 16);
                xv[gi][2 * e + 1] = __uint_as_float(w4[e] & 0xFFFF0000u);
            }
        } else {
            const float4* src =
                reinterpret_cast<const float4*>(static_cast<const float*>(x) + rr * 128 + 8 * c);
            const float4 a = src[0], bq = src[1];
            xv[gi][0] = a.x; xv[gi][1] = a.y; xv[gi][2] = a.z; xv[gi][3] = a.w;
            xv[gi][4] = bq.x; xv[gi][5] = bq.y; xv[gi][6] = bq.z; xv[gi][7] = bq.w;
        }
    }
    float cs[kPrepGroups][8], sn[kPrepGroups][8];
#pragma unroll
    for (int gi = 0; gi < kPrepGroups; ++gi) {
        const bool ok = p[gi] >= 0 && p[gi] < Lmax && p[gi] < P;
        const int64_t pe = ok ? p[gi] : 0;
        const float4* ct = reinterpret_cast<const float4*>(cos_t + pe * 32 + j0);
        const float4* st = reinterpret_cast<const float4*>(sin_t + pe * 32 + j0);
        float4 c0 = make_float4(0.f, 0.f, 0.f, 0.f), c1 = c0, s0 = c0, s1 = c0;
        if (rotary) {
            c0 = ct[0]; c1 = ct[1];
            s0 = st[0]; s1 = st[1];
        }
        cs[gi][0] = c0.x; cs[gi][1] = c0.y; cs[gi][2] = c0.z; cs[gi][3] = c0.w;
        cs[gi][4] = c1.x; cs[gi][5] = c1.y; cs[gi][6] = c1.z; cs[gi][7] = c1.w;
        sn[gi][0] = s0.x; sn[gi][1] = s0.y; sn[gi][2] = s0.z; sn[gi][3] = s0.w;
        sn[gi][4] = s1.x; sn[gi][5] = s1.y; sn[gi][6] = s1.z; sn[gi][7] = s1.w;
    }
#pragma unroll
    for (int gi = 0; gi < kPrepGroups; ++gi) {
        const int64_t row = row0 + 4 * gi + rsub;
        if (row0 + 4 * gi >= nrows) break;         // wave-uniform
        const bool ok = row < nrows && p[gi] >= 0 && p[gi] < Lmax && p[gi] < P;
        float y[8];
        {
#pragma clang fp contract(off)
            // pair (a, b) = (x[j], x[j+32]):  a' = a c - b s,  b' = a s + b c
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const float other = __shfl_xor(xv[gi][e], 4);
                float r;
                if (c < 4) {
                    const float ac = xv[gi][e] * cs[gi][e], bs = other * sn[gi][e];
                    r = ac - bs;
                } else {
                    const float as = other * sn[gi][e], bc = xv[gi][e] * cs[gi][e];
                    r = as + bc;
                }
                if (BF16_IN) r = bf16_bits_to_float(float_to_bf16_bits(r));   // cast back
                y[e] = rotary ? r : xv[gi][e];
            }
        }
        if (had) {
            wht_lane(y, 1);
            wht_lane(y, 2);
            wht_lane(y, 4);
#pragma unroll
            for (int st = 1; st < 16; st <<= 1) wht_lanes(y, c, st);
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                y[e] = y[e] * kInvSqrt128;
                if (BF16_IN) y[e] = bf16_bits_to_float(float_to_bf16_bits(y[e]));
            }
        }
        float amax = 0.0f;
#pragma unroll
        for (int e = 0; e < 8; ++e) amax = fmaxf(amax, fabsf(y[e]));
#pragma unroll
        for (int o = 1; o < 16; o <<= 1) amax = fmaxf(amax, __shfl_xor(amax, o));
        float scale = amax / 448.0f;
        if (pow2) scale = scale > 0.0f ? pow2_ceil(scale) : 1.0f;
        else if (!(scale > 0.0f)) scale = 1.0f;
        uint32_t w0, w1;
        if (quotient_fast(scale)) {
            const float rs = 1.0f / scale;
            w0 = e4m3_encode4(quotient_rn(y[0], scale, rs), quotient_rn(y[1], scale, rs),
                              quotient_rn(y[2], scale, rs), quotient_rn(y[3], scale, rs));
            w1 = e4m3_encode4(quotient_rn(y[4], scale, rs), quotient_rn(y[5], scale, rs),
                              quotient_rn(y[6], scale, rs), quotient_rn(y[7], scale, rs));
        } else {
            w0 = e4m3_encode4(y[0] / scale, y[1] / scale, y[2] / scale, y[3] / scale);
            w1 = e4m3_encode4(y[4] / scale, y[5] / scale, y[6] / scale, y[7] / scale);
        }
        if (!ok) continue;
        int64_t dst;
        if (TO_CACHE) {
            const int64_t b = (row / rows_per_pos) / S;
            dst = cmap.row(b, p[gi]);
            if (dst < 0) continue;                  // page not present: nothing to write
        } else {
            dst = row;
        }
        *reinterpret_cast<uint2*>(codes_out + dst * 128 + 8 * c) = make_uint2(w0, w1);
        if (c == 0) scales_out[dst] = scale;
    }
}

hipError_t launch_prepare(bool bf16_in, bool to_cache, int64_t nrows, int rows_per_pos, int S,
                          int Lmax, int P, const void* x, const int32_t* pos, const float* cos_t,
                          const float* sin_t, uint8_t* codes, float* scales, bool hadamard,
                          bool pow2, CacheMap cmap, hipStream_t stream) {
    if (nrows <= 0) return hipSuccess;
    const dim3 grid(static_cast<unsigned>((nrows + 4 * kPrepRowsPerWave - 1) / (4 * kPrepRowsPerWave))),
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
constexpr int kKW = 2;                      // 32-key tiles per wave
constexpr int kTileBlocksPerCU = 2;         // occupancy the tile kernel is built for
constexpr int kQT = 64, kKT = 64 * kKW;     // queries, keys per block tile
constexpr int kQsStride = 128 + 8;          // bf16 per staged query row (bank stagger)

__device__ __forceinline__ v16f mfma_bf16_32x32x16(bf16x8 a, bf16x8 b, v16f c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

__global__ __launch_bounds__(256, kTileBlocksPerCU) void score_tile_kernel(
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

    // per-head query weights, halved: the epilogue adds w' (s + |s|), which
    // is w q_scale ReLU(s) exactly
    for (int i = tid; i < 64 * kQT; i += 256) {
        const int h = i / kQT, qi = i - h * kQT;
        float v = 0.0f;
        if (h < H && t0 + qi < S) {
            const int64_t r = row0 + qi;
            v = 0.5f * (w[r * H + h] * qscale[r * H + h]);
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
                for (int kt2 = 0; kt2 < kKW; ++kt2) {
                    const float sv = sacc[kt2][4 * r + c];
                    I[kt2][4 * r + c] = fmaf(wr[c], sv + fabsf(sv), I[kt2][4 * r + c]);
                }
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
// row's 64 query heads itself (into LDS) while its first key loads are in
// flight, and the block that covers the row's own position also rotates,
// quantises and appends the new key, using it straight from LDS. One launch
// replaces prepare(k) + prepare(q) + score.
// A block of NW waves scores chunks of NW * 16 U consecutive keys of its
// row, wave w the keys [16 U w, 16 U w + 16 U) of a chunk; block x takes the
// row's chunks x, x + gridDim.x, ... Calls with few keys in all get one chunk
// per block (many small blocks: latency); calls with many get a few blocks
// per CU that loop over chunks with two chunks in flight (three register
// buffers in rotation), so the query quantisation is paid once per block.
// Query quantisation layout: thread t owns head t / TPH and the part e =
// t % TPH of its features (TPH = NW threads per head): parts e < TPH/2 hold
// rotary pairs (j, j + 32), parts e >= TPH/2 runs of features 64..127. The
// head's amax is reduced over its TPH threads.
// Scoring: per 16 keys (u) and 16 heads (hg), 4 MFMAs over the 128 features;
// lane (m, g) gets heads 4g..4g+3 of key m and accumulates
// w'[h] * (s + |s|) = w[h] q_scale[h] ReLU(s), with w' = w q_scale / 2 (the
// halving and doubling are exact). The four lanes g of a key then add their
// sums with two cross-lane steps that also scatter the U key groups over the
// lanes, so that one store per wave writes up to 64 consecutive scores.
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

// the same for two values at once with the hardware conversion
// (v_cvt_pk_bf16_f32, round to nearest even, as the bit rule above for every
// finite float)
template <bool BF16_IN>
__device__ __forceinline__ void round_act2(float& a, float& b) {
    if constexpr (BF16_IN) {
        const uint32_t pk = pack_bf16x2(a, b);
        a = __uint_as_float(pk << 16);
        b = __uint_as_float(pk & 0xFFFF0000u);
    }
}

// v of the lane whose index differs in bit M: quad permutations (DPP, no
// LDS traffic) for M = 1, 2, a cross-lane shuffle otherwise
template <int M>
__device__ __forceinline__ float lane_xor(float v) {
    if constexpr (M == 1)
        return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0xB1, 0xF, 0xF, true));
    else if constexpr (M == 2)
        return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0x4E, 0xF, 0xF, true));
    else
        return __shfl_xor(v, M);
}

// one butterfly stage across the lanes whose index differs in bit M (M < TPH)
template <int M, int N>
__device__ __forceinline__ void wht_xlanes(float (&v)[N], int e) {
    const bool upper = (e & M) != 0;
#pragma unroll
    for (int j = 0; j < N; ++j) {
        const float pa = lane_xor<M>(v[j]);
        v[j] = upper ? pa - v[j] : v[j] + pa;
    }
}

template <int U>
struct DecChunk {
    uint4 k[U][2];      // key codes: lane (m, g), key 16 u + m, bytes [32 g, 32 g + 32)
    float ks;           // scale of the key this lane stores (-inf: page not present)
};

template <int U, int NW, bool LOOP, bool BF16_IN>
__global__ __launch_bounds__(NW * 64) void decode_score_kernel(
    int H, int Lmax, int P, const void* __restrict__ q_raw, const void* __restrict__ k_raw,
    const int32_t* __restrict__ pos, const float* __restrict__ cos_t,
    const float* __restrict__ sin_t, const float* __restrict__ w, uint8_t* __restrict__ kcache,
    float* __restrict__ kscale, uint8_t* __restrict__ q8_out, float* __restrict__ qs_out,
    float* __restrict__ scores, int64_t ld, CacheMap cmap, int had, int pow2) {
    constexpr int kThreads = NW * 64;
    constexpr int kTPH = kThreads / 64;                 // threads per query head
    constexpr int kFPT = 128 / kTPH;                    // features per thread
    constexpr int kChunkKeys = NW * 16 * U;
    __shared__ __align__(16) uint8_t qcodes[64 * 128];
    __shared__ float qscale[64];
    __shared__ __align__(16) uint8_t kcodes[128];
    __shared__ float kscale_new;

    const int row = blockIdx.y;
    const int chunk = blockIdx.x;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int m = lane & 15, g = lane >> 4;
    const int64_t b = row;
    // the key (within the wave's 16 U) whose score this lane stores
    const int own = U == 4 ? lane : (U == 2 ? 16 * (g >> 1) + m : m);
    const bool stores = U == 4 ? true : (U == 2 ? (g & 1) == 0 : g == 0);
    const bool dense = cmap.table == nullptr;
    const uint8_t* kc_row = kcache + (dense ? b * cmap.batch_rows * 128 : 0);
    const float* ks_row = kscale + (dense ? b * cmap.batch_rows : 0);

    // Loads that need no position, issued before the row's position arrives:
    // the first chunk's key rows (dense cache, chunk inside it; keys at or
    // past n_valid are scored but never stored), the head weights and the
    // raw query.
    auto load_rows = [&](int wkey0, DecChunk<U>& d) {
        const uint4* src =
            reinterpret_cast<const uint4*>(kc_row + static_cast<int64_t>(wkey0 + m) * 128 + g * 32);
#pragma unroll
        for (int u = 0; u < U; ++u) {
            d.k[u][0] = src[u * 128];
            d.k[u][1] = src[u * 128 + 1];
        }
        d.ks = ks_row[wkey0 + own];
    };
    DecChunk<U> A, Bc;
    const int wkeyA = chunk * kChunkKeys + wave * 16 * U;
    const bool specA = dense && wkeyA + 16 * U <= Lmax;
    if (specA) load_rows(wkeyA, A);
    float wraw[4][4];
#pragma unroll
    for (int hg = 0; hg < 4; ++hg)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int h = hg * 16 + 4 * g + i;
            wraw[hg][i] = h < H ? w[static_cast<int64_t>(row) * H + h] : 0.0f;
        }
    constexpr int kHalf = kTPH / 2;
    const int hh = tid / kTPH, e = tid % kTPH;
    float qv[kFPT];
#pragma unroll
    for (int j = 0; j < kFPT; ++j) qv[j] = 0.0f;
    if (hh < H && had) {
        // Hadamard option: thread e holds the contiguous features [FPT e, FPT e + FPT)
        const int64_t base = (static_cast<int64_t>(row) * H + hh) * 128 + kFPT * e;
#pragma unroll
        for (int j = 0; j < kFPT; ++j) qv[j] = load_act<BF16_IN>(q_raw, base + j);
    } else if (hh < H) {
        const int64_t base = (static_cast<int64_t>(row) * H + hh) * 128;
        if (e < kHalf) {
            const int j0 = (kFPT / 2) * e;
#pragma unroll
            for (int j = 0; j < kFPT / 2; ++j) {
                qv[j] = load_act<BF16_IN>(q_raw, base + j0 + j);
                qv[kFPT / 2 + j] = load_act<BF16_IN>(q_raw, base + j0 + j + 32);
            }
        } else {
            const int f0 = 64 + kFPT * (e - kHalf);
#pragma unroll
            for (int j = 0; j < kFPT; ++j) qv[j] = load_act<BF16_IN>(q_raw, base + f0 + j);
        }
    }

    const int p = pos[row];
    if (p < 0 || p >= Lmax || p >= P) return;
    const int n_valid = p + 1;
    const int nchunks = (n_valid + kChunkKeys - 1) / kChunkKeys;
    const int stride = static_cast<int>(gridDim.x);
    if (chunk >= nchunks) return;
    const int64_t prow = cmap.row(b, p);                              // the new key's row
    const int chunk_p = p / kChunkKeys;                               // chunk holding p
    const bool has_new = k_raw != nullptr && prow >= 0 && chunk_p % stride == chunk;

    // 1. key loads of chunk c (the new key, if any, is taken from LDS later)
    auto load_chunk = [&](int c, DecChunk<U>& d) {
        const int wkey0 = c * kChunkKeys + wave * 16 * U;
        if (dense && wkey0 + 16 * U <= n_valid) {
            load_rows(wkey0, d);
        } else {
#pragma unroll
            for (int u = 0; u < U; ++u) {
                int key = wkey0 + u * 16 + m;
                key = key < n_valid ? key : n_valid - 1;
                const int64_t krow = cmap.row(b, key);
                const uint4* src =
                    reinterpret_cast<const uint4*>(kcache + (krow >= 0 ? krow : 0) * 128 + g * 32);
                d.k[u][0] = src[0];
                d.k[u][1] = src[1];
            }
            int okey = wkey0 + own;
            okey = okey < n_valid ? okey : n_valid - 1;
            const int64_t orow = cmap.row(b, okey);
            d.ks = orow >= 0 ? kscale[orow] : -INFINITY;
        }
    };
    if (!specA) load_chunk(chunk, A);
    if constexpr (LOOP) {                    // two chunks in flight during the quantisation
        if (chunk + stride < nchunks) load_chunk(chunk + stride, Bc);
    }

    // 2. quantise the row's query heads into LDS
    {
#pragma clang fp contract(off)
        float v[kFPT];
        float amax = 0.0f;
        if (had) {
            // contiguous layout: the rotary partner of feature f < 64 (f +- 32)
            // sits in thread e ^ (32 / FPT) at the same j; every lane takes
            // part in the exchanges (a head's threads are adjacent lanes)
            constexpr int kPairX = 32 / kFPT;
            const bool rot = kFPT * e < 64, lower = kFPT * e < 32;
            const int64_t tb = static_cast<int64_t>(p) * 32 + ((kFPT * e) & 31);
#pragma unroll
            for (int j = 0; j < kFPT; ++j) {
                const float other = lane_xor<kPairX>(qv[j]);
                float r = qv[j];
                if (rot) {
                    const float c = cos_t[tb + j], sn = sin_t[tb + j];
                    if (lower) {
                        const float ac = qv[j] * c, bs = other * sn;
                        r = ac - bs;
                    } else {
                        const float as = other * sn, bc = qv[j] * c;
                        r = as + bc;
                    }
                }
                v[j] = r;
            }
            // cast back to the activation dtype (the non-rotary values are
            // already representable, so rounding them changes nothing)
#pragma unroll
            for (int j = 0; j < kFPT; j += 2) round_act2<BF16_IN>(v[j], v[j + 1]);
            // H_128 x / sqrt(128): butterflies (x[f], x[f + s]) -> (sum,
            // difference) over every bit of the feature index; strides below
            // FPT inside the thread, the others across the head's lanes
#pragma unroll
            for (int st = 1; st < kFPT; st <<= 1)
#pragma unroll
                for (int j = 0; j < kFPT; ++j)
                    if ((j & st) == 0) {
                        const float lo = v[j], hi = v[j + st];
                        v[j] = lo + hi;
                        v[j + st] = lo - hi;
                    }
            wht_xlanes<1>(v, e);
            if constexpr (kTPH > 2) wht_xlanes<2>(v, e);
            if constexpr (kTPH > 4) wht_xlanes<4>(v, e);
            static_assert(kTPH <= 8, "a head spans at most 8 lanes");
#pragma unroll
            for (int j = 0; j < kFPT; j += 2) {
                v[j] *= kInvSqrt128;
                v[j + 1] *= kInvSqrt128;
                round_act2<BF16_IN>(v[j], v[j + 1]);
            }
            if (hh < H) {
#pragma unroll
                for (int j = 0; j < kFPT; ++j) amax = fmaxf(amax, fabsf(v[j]));
            }
        } else if (hh < H) {
            if (e < kHalf) {
                const int j0 = (kFPT / 2) * e;
                const float* c = cos_t + static_cast<int64_t>(p) * 32 + j0;
                const float* sn = sin_t + static_cast<int64_t>(p) * 32 + j0;
#pragma unroll
                for (int j = 0; j < kFPT / 2; ++j) {
                    const float a = qv[j];
                    const float bb = qv[kFPT / 2 + j];
                    const float ac = a * c[j], bs = bb * sn[j];
                    const float as = a * sn[j], bc = bb * c[j];
                    v[j] = ac - bs;
                    v[kFPT / 2 + j] = as + bc;
                    round_act2<BF16_IN>(v[j], v[kFPT / 2 + j]);
                }
            } else {
#pragma unroll
                for (int j = 0; j < kFPT; ++j) v[j] = qv[j];
            }
#pragma unroll
            for (int j = 0; j < kFPT; ++j) amax = fmaxf(amax, fabsf(v[j]));
        }
#pragma unroll
        for (int o = 1; o < kTPH; o <<= 1) amax = fmaxf(amax, __shfl_xor(amax, o));
        float scale = amax / 448.0f;
        if (pow2) scale = scale > 0.0f ? pow2_ceil(scale) : 1.0f;
        else if (!(scale > 0.0f)) scale = 1.0f;
        uint32_t pk[kFPT / 4];
        if (quotient_fast(scale)) {
            const float rs = 1.0f / scale;
#pragma unroll
            for (int i = 0; i < kFPT / 4; ++i)
                pk[i] = e4m3_encode4(quotient_rn(v[4 * i], scale, rs),
                                     quotient_rn(v[4 * i + 1], scale, rs),
                                     quotient_rn(v[4 * i + 2], scale, rs),
                                     quotient_rn(v[4 * i + 3], scale, rs));
        } else {
#pragma unroll
            for (int i = 0; i < kFPT / 4; ++i)
                pk[i] = e4m3_encode4(v[4 * i] / scale, v[4 * i + 1] / scale, v[4 * i + 2] / scale,
                                     v[4 * i + 3] / scale);
        }
#pragma unroll
        for (int i = 0; i < kFPT / 4; ++i) pk[i] = hh < H ? pk[i] : 0u;
        // parts e < TPH/2: bytes [j0, j0 + FPT/2) and [32 + j0, ...); others [f0, f0 + FPT)
        // (Hadamard option: every part [FPT e, FPT e + FPT))
        uint8_t* dst = qcodes + hh * 128;
        const int off0 = had ? kFPT * e : (e < kHalf ? (kFPT / 2) * e : 64 + kFPT * (e - kHalf));
        const int off1 = had ? kFPT * e + kFPT / 2
                             : (e < kHalf ? 32 + (kFPT / 2) * e : off0 + kFPT / 2);
#pragma unroll
        for (int i = 0; i < kFPT / 16; ++i) {          // FPT/2 bytes per half, 8 per store
            reinterpret_cast<uint2*>(dst + off0)[i] = make_uint2(pk[2 * i], pk[2 * i + 1]);
            reinterpret_cast<uint2*>(dst + off1)[i] =
                make_uint2(pk[kFPT / 8 + 2 * i], pk[kFPT / 8 + 2 * i + 1]);
        }
        if (e == 0) qscale[hh] = hh < H ? scale : 0.0f;
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
        float y1 = x1;
        if (had) {
            // H_128 x / sqrt(128): stride 64 inside the lane, 1 .. 32 across lanes
            const float lo = y0 + y1, hi = y0 - y1;
            y0 = lo;
            y1 = hi;
#pragma unroll
            for (int st = 1; st < 64; st <<= 1) {
                const bool upper = (lane & st) != 0;
                const float p0 = __shfl_xor(y0, st), p1 = __shfl_xor(y1, st);
                y0 = upper ? p0 - y0 : y0 + p0;
                y1 = upper ? p1 - y1 : y1 + p1;
            }
            y0 = round_act<BF16_IN>(y0 * kInvSqrt128);
            y1 = round_act<BF16_IN>(y1 * kInvSqrt128);
        }
        const float amax = wave_max(fmaxf(fabsf(y0), fabsf(y1)));
        float scale = amax / 448.0f;
        if (pow2) scale = scale > 0.0f ? pow2_ceil(scale) : 1.0f;
        else if (!(scale > 0.0f)) scale = 1.0f;
        const uint8_t c0 = e4m3_encode(y0 / scale), c1 = e4m3_encode(y1 / scale);
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
        for (int i = tid; i < H * 8; i += kThreads)
            reinterpret_cast<uint4*>(q8_out + static_cast<int64_t>(row) * H * 128)[i] =
                reinterpret_cast<const uint4*>(qcodes)[i];
        if (tid < H) qs_out[static_cast<int64_t>(row) * H + tid] = qscale[tid];
    }

    // 4. query operands from LDS (lane (m, g): head 16 hg + m, features
    // 32 g + 8 kk + j), halved head weights
    bf16x8 qa[4][4];
    float wq2[4][4];
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
            wq2[hg][i] = h < H ? 0.5f * (wraw[hg][i] * qscale[h]) : 0.0f;
        }
    }
    float* out = scores + static_cast<int64_t>(row) * ld;

    // 5. score chunk c (the chunk holding p first takes the new key's codes
    // from LDS)
    auto score_chunk = [&](int c, DecChunk<U>& d) {
        const int wkey0 = c * kChunkKeys + wave * 16 * U;
        if (has_new && c == chunk_p) {
#pragma unroll
            for (int u = 0; u < U; ++u) {
                if (wkey0 + 16 * u + m == p) {
                    d.k[u][0] = reinterpret_cast<const uint4*>(kcodes + g * 32)[0];
                    d.k[u][1] = reinterpret_cast<const uint4*>(kcodes + g * 32)[1];
                }
            }
        }
        float part[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const uint4 k0 = d.k[u][0], k1 = d.k[u][1];
            bf16x8 kbf[4];
            kbf[0] = e4m3x8_to_bf16x8(k0.x, k0.y);
            kbf[1] = e4m3x8_to_bf16x8(k0.z, k0.w);
            kbf[2] = e4m3x8_to_bf16x8(k1.x, k1.y);
            kbf[3] = e4m3x8_to_bf16x8(k1.z, k1.w);
            float sum = 0.0f;
#pragma unroll
            for (int hg = 0; hg < 4; ++hg) {
                v4f acc = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
                for (int kk = 0; kk < 4; ++kk) acc = mfma_bf16_16x16x32(qa[hg][kk], kbf[kk], acc);
#pragma unroll
                for (int i = 0; i < 4; ++i) sum = fmaf(wq2[hg][i], acc[i] + fabsf(acc[i]), sum);
            }
            part[u] = sum;
        }
        // head sum over g, scattering the key groups: afterwards lane (m, g)
        // holds the total of key `own`
        float tot;
        if constexpr (U == 4) {
            const bool hi = g >= 2;                  // keeps groups 2, 3 (else 0, 1)
            const float r0 = (hi ? part[2] : part[0]) + __shfl_xor(hi ? part[0] : part[2], 32);
            const float r1 = (hi ? part[3] : part[1]) + __shfl_xor(hi ? part[1] : part[3], 32);
            const bool odd = (g & 1) != 0;           // keeps the second of the two
            tot = (odd ? r1 : r0) + __shfl_xor(odd ? r0 : r1, 16);
        } else if constexpr (U == 2) {
            const bool hi = g >= 2;                  // keeps group 1 (else 0)
            const float r = (hi ? part[1] : part[0]) + __shfl_xor(hi ? part[0] : part[1], 32);
            tot = r + __shfl_xor(r, 16);
        } else {
            const float r = part[0] + __shfl_xor(part[0], 32);
            tot = r + __shfl_xor(r, 16);
        }
        const int key = wkey0 + own;
        const float ksc = (has_new && key == p) ? kscale_new : d.ks;
        if (stores && key < n_valid) out[key] = ksc == -INFINITY ? -INFINITY : tot * ksc;
    };

    if constexpr (!LOOP) {
        score_chunk(chunk, A);
    } else {
        // three buffers in rotation, two chunks in flight: A holds chunk x,
        // Bc chunk x + stride, C is free
        DecChunk<U> C;
        for (int x = chunk;; x += 3 * stride) {
            if (x + 2 * stride < nchunks) load_chunk(x + 2 * stride, C);
            score_chunk(x, A);
            if (x + stride >= nchunks) break;
            if (x + 3 * stride < nchunks) load_chunk(x + 3 * stride, A);
            score_chunk(x + stride, Bc);
            if (x + 2 * stride >= nchunks) break;
            if (x + 4 * stride < nchunks) load_chunk(x + 4 * stride, Bc);
            score_chunk(x + 2 * stride, C);
            if (x + 3 * stride >= nchunks) break;
        }
    }
}

// Looping decode grid: blocks of kDecLoopWaves waves scoring chunks of
// kDecLoopWaves * 64 keys, about kDecLoopBlocks blocks in all; used
// when a call has more than that many chunks.
constexpr int kDecLoopBlocks = 256;         // blocks of the looping decode grid, about
constexpr int kDecLoopWaves = 8;            // waves per block of the looping grid

hipError_t launch_decode_score(bool bf16_in, int B, int H, int Lmax, int P, const void* q_raw,
                               const void* k_raw, const int32_t* pos, const float* cos_t,
                               const float* sin_t, const float* w, uint8_t* kcache,
                               float* kscale, uint8_t* q8_out, float* qs_out, float* scores,
                               int64_t ld, CacheMap cmap, bool hadamard, bool pow2,
                               hipStream_t stream) {
    constexpr int kLoopChunk = kDecLoopWaves * 64;
    const int chunksl = (Lmax + kLoopChunk - 1) / kLoopChunk;
    const bool loop = static_cast<int64_t>(B) * chunksl > kDecLoopBlocks;
    int U = 4;
    unsigned gx, threads;
    if (loop) {
        const int bpr = (kDecLoopBlocks + B - 1) / B;
        gx = static_cast<unsigned>(bpr < chunksl ? bpr : chunksl);
        threads = kDecLoopWaves * 64;
    } else {
        // one chunk of 64 U keys per block, U shrunk (down to 1) to give more blocks
        while (U > 1 && static_cast<int64_t>(B) * ((Lmax + 64 * U - 1) / (64 * U)) < 2048) U >>= 1;
        gx = static_cast<unsigned>((Lmax + 64 * U - 1) / (64 * U));
        threads = 256;
    }
    const dim3 grid(gx, static_cast<unsigned>(B));
#define DSA_DEC(UU, NWW, LP, BF)                                                                 \
    hipLaunchKernelGGL((decode_score_kernel<UU, NWW, LP, BF>), grid, dim3(threads), 0, stream, H, \
                       Lmax, P, q_raw, k_raw, pos, cos_t, sin_t, w, kcache, kscale, q8_out,    \
                       qs_out, scores, ld, cmap, hadamard ? 1 : 0, pow2 ? 1 : 0)
    if (bf16_in) {
        if (loop) DSA_DEC(4, kDecLoopWaves, true, true);
        else if (U == 4) DSA_DEC(4, 4, false, true);
        else if (U == 2) DSA_DEC(2, 4, false, true);
        else DSA_DEC(1, 4, false, true);
    } else {
        if (loop) DSA_DEC(4, kDecLoopWaves, true, false);
        else if (U == 4) DSA_DEC(4, 4, false, false);
        else if (U == 2) DSA_DEC(2, 4, false, false);
        else DSA_DEC(1, 4, false, false);
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
