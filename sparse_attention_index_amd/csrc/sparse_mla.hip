// sparse_mla.hip -- sparse latent attention, absorbed (MQA) form, gfx950.
//
// Method (page "Similarities", MLA decode excerpt; page "Sparse latent
// attention", S' = S m^2/sqrt(192), softmax, O = AV, attention over the
// selected positions alone): for query row r and head h, over the selected
// positions p_j,
//   z_j = scale * (q[h][0:512] . latent[p_j] + q[h][512:576] . rope[p_j])
//   out[h] = sum_j softmax(z)_j latent[p_j],  lse[h] = log sum_j exp(z_j).
//
// Design: one block of 4 waves serves 64 heads (16 per wave) of one query
// row over a contiguous range ("split") of its selected positions (2 waves
// and 32 heads in the build for the fewest blocks, below). The two
// head-group blocks of a (row, split) get launch indices 8 apart in one 1-D
// grid: the same XCD and back to back in dispatch order, so the second
// block's gather is served by that XCD's L2. The split's index list is
// staged in LDS once. Selected rows are gathered 32 at a time (8 threads
// per row, each thread one or two rows) into an LDS tile K [32][576]
// (row-major, padded).
// Per wave:
//   S^T = K Q^T       bf16 MFMA 16x16x32, M = keys (2 tiles of 16), N = the
//                     wave's 16 heads, K = features, four independent
//                     accumulation chains; Q^T stays in VGPRs.
//   online softmax    per head (one head per lane column, four lanes per
//                     head), in log2 units, against a reference maximum that
//                     moves only when the running maximum passes it by 8:
//                     the accumulator is rescaled only then.
//   O^T += V^T P^T    bf16 MFMA 16x16x32, M = 16 latent features (32 tiles),
//                     N = heads, K = the 32 keys. P^T comes straight from the
//                     S^T result registers (the key order inside the MFMA K
//                     dimension only has to match between the operands); V^T
//                     is read from the row-major K tile with the transposing
//                     LDS read ds_read_b64_tr_b16: within each 16-lane group,
//                     lane 4e+q addresses features 4q..4q+3 of key e and lane
//                     i receives feature i of keys 0..3.
// Three builds of the kernel: when the grid has at most one block per CU
// (few query rows), one wave per SIMD has the CU to itself, so the gather of
// the next tile is held in registers while the current one is computed and
// the LDS operand reads run several MFMAs ahead; with the fewest rows the
// blocks serve 32 heads, which halves the LDS reads per CU and tile (the
// CU's LDS bandwidth and the MFMA chain take about equal time per tile with
// 4 waves reading every operand); with more blocks, two 64-head blocks
// share a CU and hide each other's latencies instead.
// With several splits per row the unnormalised partials (O, m, l) go to the
// workspace, each wave's 16 x 512 block of O stored exactly as its registers
// hold it, rounded to bf16 (every store instruction writes 512 consecutive
// bytes; halving the partials' bytes shortens the call more than the extra
// rounding, at most 2^-9 of the split's weighted |latent|, costs), and
// combine_kernel (merge_few_kernel for the fewest rows) merges them in
// float32 with the log-sum-exp rule.
#include "dsa_common.h"

namespace dsa {

typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
constexpr int kDl = 512, kDq = 576;
constexpr int kTile = 32;
constexpr int kKtStride = kDq + 8;      // bf16 per K-tile row (1168 B, staggers banks)
constexpr int kHeadsPerBlock = 64;      // 4 waves x 16 heads
constexpr int kHeadsPerBlockFew = 32;   // 2 waves: the build for the fewest blocks
constexpr int kMaxSlots = 2048;         // selected positions per split, at most
constexpr int kMaxSplits = 64;
constexpr int kT2 = kDl / 16;           // 16-feature output tiles per head
constexpr size_t kMlaLdsBytes = sizeof(uint16_t) * kTile * kKtStride + sizeof(int) * kMaxSlots;

// Scheduling-group hints (no instructions): the next `n` instructions of a
// kind (LDS reads / MFMAs) are placed in the order of these calls, which
// keeps the LDS operand reads of a tile a fixed number of MFMAs ahead.
constexpr int kSchedMfma = 0x008, kSchedDsRead = 0x100;
#define DSA_SCHED_GROUP(mask, n) __builtin_amdgcn_sched_group_barrier((mask), (n), 0)

// HPB = heads per block (4 HPB threads, one wave per 16 heads)
template <bool PIPE, int HPB>
__global__ __launch_bounds__(4 * HPB, PIPE ? 1 : 2) void sparse_mla_kernel(
    int S, int Hq, int Lmax, int K, int slots_per_split, int nsplit, int nitems, int hgroups,
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ latent, int64_t lat_rs,
    int64_t lat_bs, const uint16_t* __restrict__ rope, int64_t rope_rs, int64_t rope_bs,
    const int32_t* __restrict__ idx, float scale_log2, uint16_t* __restrict__ out,
    float* __restrict__ lse, uint16_t* __restrict__ ws_o, float* __restrict__ ws_ml, CacheMap cmap) {
    extern __shared__ __align__(16) unsigned char smem[];
    uint16_t* Kt = reinterpret_cast<uint16_t*>(smem);
    int* sidx = reinterpret_cast<int*>(Kt + kTile * kKtStride);

    // launch index -> (work item = row * nsplit + split, head group): the
    // head groups of one item sit 8 apart (same XCD, adjacent dispatch)
    const int L = blockIdx.x;
    const int item = (L / (8 * hgroups)) * 8 + (L & 7);
    const int hg = (L / 8) % hgroups;
    if (item >= nitems) return;
    const int row = item / nsplit, split = item - row * nsplit;
    const int64_t b = row / S;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int m = lane & 15, g = lane >> 4;
    constexpr int kThr = 4 * HPB;                                 // threads per block
    constexpr int kRP = kThr / 8;                                 // gathered rows per pass
    constexpr int kNP = kTile / kRP;                              // gather passes per tile
    const int wg = hg * (HPB / 16) + wave;                        // 16-head group
    const int h = wg * 16 + m;
    const bool active = wg * 16 < Hq;                             // wave has a real head

    const int j_begin = split * slots_per_split;
    const int j_end = min(K, j_begin + slots_per_split);
    const int count = j_end - j_begin;
    const int ntiles = count > 0 ? (count + kTile - 1) / kTile : 0;
    // selected slots -> cache rows: the position itself (dense caches, batch
    // offset added below) or the pool row of its page (paged caches); -1 for
    // unselected slots and positions whose page is not present
    const bool paged = cmap.table != nullptr;
    {
        const int32_t* irow = idx + static_cast<int64_t>(row) * K + j_begin;
        for (int i = tid; i < ntiles * kTile; i += kThr) {
            const int p = i < count ? irow[i] : -1;
            int v = -1;
            if (p >= 0 && p < Lmax) v = paged ? static_cast<int>(cmap.row(b, p)) : p;
            sidx[i] = v;
        }
    }

    // Q^T operand: lane (head h, chunk g) holds q[h][32 ks + 8 g .. +7].
    bf16x8 qreg[kDq / 32];
    {
        const uint16_t* qh =
            q + (static_cast<int64_t>(row) * Hq + (h < Hq ? h : 0)) * kDq + 8 * g;
#pragma unroll
        for (int ks = 0; ks < kDq / 32; ++ks) {
            uint4 v = *reinterpret_cast<const uint4*>(qh + ks * 32);
            if (h >= Hq) v = make_uint4(0u, 0u, 0u, 0u);
            qreg[ks] = __builtin_bit_cast(bf16x8, v);
        }
    }
    v4f acc[kT2];
#pragma unroll
    for (int t2 = 0; t2 < kT2; ++t2) acc[t2] = v4f{0.0f, 0.0f, 0.0f, 0.0f};
    // l_run sums the float32 probabilities (for lse); lr_run sums the bf16
    // values that actually weight the latent rows (for the normalisation).
    float m_run = -INFINITY, l_run = 0.0f, lr_run = 0.0f;

    const uint16_t* lat_b = latent + (paged ? 0 : b * lat_bs);
    const uint16_t* rope_b = rope + (paged ? 0 : b * rope_bs);
    __syncthreads();                               // sidx ready

    // Gather mapping: 8 threads per key row (in each pass over kRP rows,
    // wave w loads keys 8w..8w+7);
    // thread sub = tid % 8 loads latent chunks sub + 8i (i < 8, 8 features
    // each) and rope chunk sub: one row pointer per thread, immediate offsets,
    // 128 contiguous bytes per 8 lanes. Unselected slots read row 0 and are
    // zeroed (no divergent branches).
    const int gkey = tid >> 3, gsub = tid & 7;
    uint4 GA[kNP][9];
    auto fetch_tile = [&](int t, uint4 (&G)[kNP][9]) {
#pragma unroll
        for (int pp = 0; pp < kNP; ++pp) {
            const int p = sidx[t * kTile + gkey + kRP * pp];
            const int pc = p >= 0 ? p : 0;
            const uint16_t* lrow = lat_b + static_cast<int64_t>(pc) * lat_rs + gsub * 8;
            const uint16_t* rrow = rope_b + static_cast<int64_t>(pc) * rope_rs + gsub * 8;
#pragma unroll
            for (int i = 0; i < 8; ++i) G[pp][i] = *reinterpret_cast<const uint4*>(lrow + 64 * i);
            G[pp][8] = *reinterpret_cast<const uint4*>(rrow);
        }
    };
    auto store_tile = [&](int t, uint4 (&G)[kNP][9]) {
#pragma unroll
        for (int pp = 0; pp < kNP; ++pp) {
            const int key = gkey + kRP * pp;
            if (sidx[t * kTile + key] < 0) {
#pragma unroll
                for (int i = 0; i < 9; ++i) G[pp][i] = make_uint4(0u, 0u, 0u, 0u);
            }
            uint16_t* dst = Kt + key * kKtStride + gsub * 8;
#pragma unroll
            for (int i = 0; i < 8; ++i) *reinterpret_cast<uint4*>(dst + 64 * i) = G[pp][i];
            *reinterpret_cast<uint4*>(dst + 512) = G[pp][8];
        }
    };

    // transposing-read addresses (bf16 units within the tile): lane 4e+q of
    // group g reads features 4q.. of key 4g+e (k-step keys 0..15) and of key
    // 16+4g+e (keys 16..31)
    const int tr_off = (4 * g + ((lane >> 2) & 3)) * kKtStride + 4 * (lane & 3);
    auto read_v = [&](int t2) -> bf16x8 {
        // whole-register bit casts: element-wise 16-bit extraction here was
        // mis-scheduled into a lane-mixing permute
        const uint2 lo = __builtin_bit_cast(uint2, lds_read_tr16(Kt + tr_off + 16 * t2));
        const uint2 hi =
            __builtin_bit_cast(uint2, lds_read_tr16(Kt + tr_off + 16 * kKtStride + 16 * t2));
        return __builtin_bit_cast(bf16x8, make_uint4(lo.x, lo.y, hi.x, hi.y));
    };
    const uint16_t* ka_row = Kt + m * kKtStride + 8 * g;
    const uint16_t* kb_row = Kt + (16 + m) * kKtStride + 8 * g;

    // LDS operand reads in flight ahead of their MFMAs
    constexpr int kPipe = PIPE ? 4 : 2;       // S: K-operand pairs
    constexpr int kPipeV = PIPE ? 6 : 3;      // O: V^T operands
    // PIPE: the gather of the next tile is in flight in registers while the
    // current one is computed
    if (PIPE && ntiles > 0) fetch_tile(0, GA);
    auto tile_step = [&](int t, uint4 (&G)[kNP][9]) {
        __syncthreads();                           // previous tile fully consumed
        if (!PIPE) fetch_tile(t, G);
        store_tile(t, G);
        __syncthreads();
        if (PIPE && t + 1 < ntiles) fetch_tile(t + 1, G);
        if (!active) return;

        // S^T for keys 0..15 (s0) and 16..31 (s1); lane holds keys 4g+i.
        // Even and odd k-steps accumulate separately (four MFMA chains).
        v4f s0, s1;
        {
            v4f c0[2] = {{0.0f, 0.0f, 0.0f, 0.0f}, {0.0f, 0.0f, 0.0f, 0.0f}};
            v4f c1[2] = {{0.0f, 0.0f, 0.0f, 0.0f}, {0.0f, 0.0f, 0.0f, 0.0f}};
            bf16x8 a0[kPipe], a1[kPipe];
#pragma unroll
            for (int d = 0; d < kPipe; ++d) {
                a0[d] = *reinterpret_cast<const bf16x8*>(ka_row + d * 32);
                a1[d] = *reinterpret_cast<const bf16x8*>(kb_row + d * 32);
            }
            DSA_SCHED_GROUP(kSchedDsRead, 2 * kPipe);
#pragma unroll
            for (int ks = 0; ks < kDq / 32; ++ks) {
                const int sl = ks % kPipe;
                c0[ks & 1] = mfma_bf16_16x16x32(a0[sl], qreg[ks], c0[ks & 1]);
                c1[ks & 1] = mfma_bf16_16x16x32(a1[sl], qreg[ks], c1[ks & 1]);
                DSA_SCHED_GROUP(kSchedMfma, 2);
                if (ks + kPipe < kDq / 32) {
                    a0[sl] = *reinterpret_cast<const bf16x8*>(ka_row + (ks + kPipe) * 32);
                    a1[sl] = *reinterpret_cast<const bf16x8*>(kb_row + (ks + kPipe) * 32);
                    DSA_SCHED_GROUP(kSchedDsRead, 2);
                }
            }
            s0 = c0[0] + c0[1];
            s1 = c1[0] + c1[1];
        }
        // the first V^T operands are read while the softmax runs
        bf16x8 va[kPipeV];
#pragma unroll
        for (int d = 0; d < kPipeV; ++d) va[d] = read_v(d);
        DSA_SCHED_GROUP(kSchedDsRead, 2 * kPipeV);

        float z[8];
        float tmax = -INFINITY;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            z[i] = sidx[t * kTile + 4 * g + i] >= 0 ? s0[i] * scale_log2 : -INFINITY;
            z[4 + i] = sidx[t * kTile + 16 + 4 * g + i] >= 0 ? s1[i] * scale_log2 : -INFINITY;
        }
#pragma unroll
        for (int i = 0; i < 8; ++i) tmax = fmaxf(tmax, z[i]);
        tmax = fmaxf(tmax, __shfl_xor(tmax, 16));
        tmax = fmaxf(tmax, __shfl_xor(tmax, 32));
        // Lazy rescaling: probabilities are taken relative to a reference
        // maximum m_run that only moves when the running maximum exceeds it
        // by more than 8 (so p <= 2^8, exact enough in float and bf16).
        if (tmax > m_run + 8.0f) {
            const float corr = (m_run == -INFINITY) ? 0.0f : exp2f(m_run - tmax);
            l_run *= corr;
            lr_run *= corr;
            m_run = tmax;
            if (__ballot(corr != 1.0f)) {
#pragma unroll
                for (int t2 = 0; t2 < kT2; ++t2) acc[t2] *= corr;
            }
        }
        bf16x8 pv;
        {
            const bool live = m_run != -INFINITY;
            float psum = 0.0f, prsum = 0.0f;
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                const float pe = live ? __builtin_amdgcn_exp2f(z[i] - m_run) : 0.0f;
                const __bf16 pb = static_cast<__bf16>(pe);
                pv[i] = pb;
                psum += pe;
                prsum += static_cast<float>(pb);
            }
            l_run += psum;
            lr_run += prsum;
        }
        // O^T += V^T P^T, V^T operands by transposing reads of the K tile
#pragma unroll
        for (int t2 = 0; t2 < kT2; ++t2) {
            const int sl = t2 % kPipeV;
            acc[t2] = mfma_bf16_16x16x32(va[sl], pv, acc[t2]);
            DSA_SCHED_GROUP(kSchedMfma, 1);
            if (t2 + kPipeV < kT2) {
                va[sl] = read_v(t2 + kPipeV);
                DSA_SCHED_GROUP(kSchedDsRead, 2);
            }
        }
    };
    for (int t = 0; t < ntiles; ++t) tile_step(t, GA);

    float l_tot = l_run + __shfl_xor(l_run, 16);
    l_tot += __shfl_xor(l_tot, 32);
    float lr_tot = lr_run + __shfl_xor(lr_run, 16);
    lr_tot += __shfl_xor(lr_tot, 32);
    if (!active) return;
    // lane holds O^T[16 t2 + 4 g + i][h], i = 0..3
    if (nsplit == 1) {
        if (h >= Hq) return;
        const float inv = lr_tot > 0.0f ? 1.0f / lr_tot : 0.0f;
        uint16_t* oh = out + (static_cast<int64_t>(row) * Hq + h) * kDl + 4 * g;
#pragma unroll
        for (int t2 = 0; t2 < kT2; ++t2) {
            const uint32_t lo = pack_bf16x2(acc[t2][0] * inv, acc[t2][1] * inv);
            const uint32_t hi = pack_bf16x2(acc[t2][2] * inv, acc[t2][3] * inv);
            *reinterpret_cast<uint2*>(oh + 16 * t2) = make_uint2(lo, hi);
        }
        if (lse != nullptr && g == 0)
            lse[static_cast<int64_t>(row) * Hq + h] =
                l_tot > 0.0f ? m_run * 0.69314718055994531f + logf(l_tot) : -INFINITY;
    } else {
        // partial block of (row, split, 16-head group): [t2][lane] 4 x bf16
        const int nwg = (Hq + 15) / 16;
        const int64_t blk = (static_cast<int64_t>(row) * nsplit + split) * nwg + wg;
        uint16_t* wo = ws_o + blk * (kT2 * 64 * 4) + lane * 4;
#pragma unroll
        for (int t2 = 0; t2 < kT2; ++t2) {
            const uint32_t lo = pack_bf16x2(acc[t2][0], acc[t2][1]);
            const uint32_t hi = pack_bf16x2(acc[t2][2], acc[t2][3]);
            // fewest rows: streamed past L2 (measured 0.2 us shorter for one
            // row, slower for 32 rows)
            if constexpr (PIPE && HPB == kHeadsPerBlockFew)
                __builtin_nontemporal_store(u32x2{lo, hi}, reinterpret_cast<u32x2*>(wo + t2 * 256));
            else
                *reinterpret_cast<uint2*>(wo + t2 * 256) = make_uint2(lo, hi);
        }
        if (g == 0 && h < Hq)
            *reinterpret_cast<float4*>(ws_ml + ((static_cast<int64_t>(row) * nsplit + split) * Hq + h) * 4) =
                make_float4(m_run, l_tot, lr_tot, 0.0f);
    }
}

// DPP prefix sum of a float over the wave (same lane moves as the integer
// scan); lane 63 ends up with the total.
__device__ __forceinline__ float wave_incl_sum_f(float v) {
    int x = __float_as_int(v);
    x = __float_as_int(__int_as_float(x) + __int_as_float(dpp_move<kDppRowShr1, 0xF>(0, x)));
    x = __float_as_int(__int_as_float(x) + __int_as_float(dpp_move<kDppRowShr2, 0xF>(0, x)));
    x = __float_as_int(__int_as_float(x) + __int_as_float(dpp_move<kDppRowShr4, 0xF>(0, x)));
    x = __float_as_int(__int_as_float(x) + __int_as_float(dpp_move<kDppRowShr8, 0xF>(0, x)));
    x = __float_as_int(__int_as_float(x) + __int_as_float(dpp_move<kDppRowBcast15, 0xA>(0, x)));
    x = __float_as_int(__int_as_float(x) + __int_as_float(dpp_move<kDppRowBcast31, 0xC>(0, x)));
    return __int_as_float(x);
}

// Merge of key-split partials. Block = (row, 16-head group, quarter of the
// 512 features), 256 threads: wave w covers feature tiles t2 = 8 quarter +
// 2 w + {0, 1}; lane l = 16 g + m reads exactly what lane l of the producing
// wave stored (head m, features 16 t2 + 4 g .. +3), so each partial load of
// a wave is 512 consecutive bytes. Per head, wave w first turns the
// (m, l, lr) triples of all splits (one split per lane) into weights
// 2^(m_s - M) in LDS and the totals L, Lr.
#ifndef DSA_COMBINE_CFG
#define DSA_COMBINE_CFG 408                  // feature parts per 16-head group * 100 + unroll
#endif
constexpr int kCombineQuarters = DSA_COMBINE_CFG / 100;
constexpr int kCombineUnroll = DSA_COMBINE_CFG % 100;
constexpr int kCombineT2 = kT2 / kCombineQuarters / 4;     // 16-feature tiles per wave

__global__ __launch_bounds__(256) void combine_kernel(int Hq, int nsplit,
                                                      const uint16_t* __restrict__ ws_o,
                                                      const float* __restrict__ ws_ml,
                                                      uint16_t* __restrict__ out,
                                                      float* __restrict__ lse) {
    __shared__ float wgt[kMaxSplits][16];
    __shared__ float s_L[16], s_Lr[16], s_M[16];
    const int nwg = (Hq + 15) / 16;
    const int quarter = blockIdx.x % kCombineQuarters;
    const int wg = (blockIdx.x / kCombineQuarters) % nwg;
    const int64_t row = blockIdx.x / (kCombineQuarters * nwg);
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;

    // weights: wave w handles heads 4w .. 4w+3 of the group
    for (int mm = 4 * wave; mm < 4 * wave + 4; ++mm) {
        const int h = wg * 16 + mm;
        if (h >= Hq) break;                        // wave-uniform
        float4 ml = make_float4(-INFINITY, 0.0f, 0.0f, 0.0f);
        if (lane < nsplit)
            ml = *reinterpret_cast<const float4*>(ws_ml + ((row * nsplit + lane) * Hq + h) * 4);
        const float M = wave_max_dpp(ml.x);
        const float e = (ml.x == -INFINITY) ? 0.0f : exp2f(ml.x - M);
        if (lane < nsplit) wgt[lane][mm] = e;
        const float Ls = wave_incl_sum_f(ml.y * e);
        const float Lrs = wave_incl_sum_f(ml.z * e);
        if (lane == 63) {
            s_M[mm] = M;
            s_L[mm] = Ls;
            s_Lr[mm] = Lrs;
        }
    }
    __syncthreads();

    const int m = lane & 15, g = lane >> 4;
    const int h = wg * 16 + m;
    const int t2a = quarter * (kT2 / kCombineQuarters) + kCombineT2 * wave;
    const uint16_t* base = ws_o + (row * nsplit * nwg + wg) * (kT2 * 64 * 4) + lane * 4;
    const int64_t sstride = static_cast<int64_t>(nwg) * kT2 * 64 * 4;
    float4 a[kCombineT2];
#pragma unroll
    for (int u = 0; u < kCombineT2; ++u) a[u] = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
#pragma unroll kCombineUnroll
    for (int s = 0; s < nsplit; ++s) {
        const float e = wgt[s][m];
#pragma unroll
        for (int u = 0; u < kCombineT2; ++u) {
            const uint2 w = *reinterpret_cast<const uint2*>(base + s * sstride + (t2a + u) * 256);
            a[u].x += e * __uint_as_float(w.x << 16);
            a[u].y += e * __uint_as_float(w.x & 0xFFFF0000u);
            a[u].z += e * __uint_as_float(w.y << 16);
            a[u].w += e * __uint_as_float(w.y & 0xFFFF0000u);
        }
    }
    if (h >= Hq) return;
    const float Lr = s_Lr[m];
    const float inv = Lr > 0.0f ? 1.0f / Lr : 0.0f;
    uint16_t* oh = out + (row * Hq + h) * kDl + 4 * g;
#pragma unroll
    for (int u = 0; u < kCombineT2; ++u) {
        const uint32_t lo = pack_bf16x2(a[u].x * inv, a[u].y * inv);
        const uint32_t hi = pack_bf16x2(a[u].z * inv, a[u].w * inv);
        *reinterpret_cast<uint2*>(oh + 16 * (t2a + u)) = make_uint2(lo, hi);
    }
    if (lse != nullptr && quarter == 0 && wave == 0 && g == 0) {
        const float Ls = s_L[m];
        lse[row * Hq + h] = Ls > 0.0f ? s_M[m] * 0.69314718055994531f + logf(Ls) : -INFINITY;
    }
}

// Merge for the fewest rows (the grid of the 32-head build): one 64-thread
// block per (row, 16-head group, 16-feature tile t2), so that even one row's
// merge spreads over the whole chip, with no LDS and no barrier. Lane
// l = 16 g + m reads what lane l of each producing wave stored (head m,
// features 16 t2 + 4 g .. +3) and its head's (m, l, lr) triple; every load of
// a chunk of CH splits is issued before the first is used, so a row's merge
// costs one memory round trip per chunk instead of one for the weights and
// more for the partials. The accumulators follow the running maximum of m
// (log-sum-exp rule); with a single chunk each split is weighted by
// 2^(m_s - max m) directly, as in combine_kernel.
template <int CH>
__global__ __launch_bounds__(64) void merge_few_kernel(int Hq, int nsplit,
                                                       const uint16_t* __restrict__ ws_o,
                                                       const float* __restrict__ ws_ml,
                                                       uint16_t* __restrict__ out,
                                                       float* __restrict__ lse) {
    const int nwg = (Hq + 15) / 16;
    const int lane = threadIdx.x;
    const int t2 = static_cast<int>(blockIdx.x % kT2);
    const int wg = static_cast<int>((blockIdx.x / kT2) % nwg);
    const int64_t row = blockIdx.x / (kT2 * nwg);
    const int m = lane & 15, g = lane >> 4;
    const int h = wg * 16 + m;
    const int hc = h < Hq ? h : Hq - 1;
    const uint16_t* pb = ws_o + (row * nsplit * nwg + wg) * (kT2 * 64 * 4) + t2 * 256 + lane * 4;
    const int64_t ps = static_cast<int64_t>(nwg) * kT2 * 64 * 4;   // split stride of the partials
    const float* mb = ws_ml + (row * nsplit * Hq + hc) * 4;
    const int64_t ms = static_cast<int64_t>(Hq) * 4;               // split stride of the triples

    float4 a = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
    float M = -INFINITY, Ls = 0.0f, Lr = 0.0f;
    for (int s0 = 0; s0 < nsplit; s0 += CH) {
        float4 ml[CH];
        uint2 w[CH];
#pragma unroll
        for (int c = 0; c < CH; ++c) {
            ml[c] = make_float4(-INFINITY, 0.0f, 0.0f, 0.0f);
            w[c] = make_uint2(0u, 0u);
            if (s0 + c < nsplit) {
                ml[c] = *reinterpret_cast<const float4*>(mb + (s0 + c) * ms);
                w[c] = *reinterpret_cast<const uint2*>(pb + (s0 + c) * ps);
            }
        }
        float Mn = M;
#pragma unroll
        for (int c = 0; c < CH; ++c) Mn = fmaxf(Mn, ml[c].x);
        const float r = M == -INFINITY ? 0.0f : exp2f(M - Mn);
        M = Mn;
        Ls *= r;
        Lr *= r;
        a.x *= r;
        a.y *= r;
        a.z *= r;
        a.w *= r;
#pragma unroll
        for (int c = 0; c < CH; ++c) {
            const float e = ml[c].x == -INFINITY ? 0.0f : exp2f(ml[c].x - Mn);
            Ls += ml[c].y * e;
            Lr += ml[c].z * e;
            a.x += e * __uint_as_float(w[c].x << 16);
            a.y += e * __uint_as_float(w[c].x & 0xFFFF0000u);
            a.z += e * __uint_as_float(w[c].y << 16);
            a.w += e * __uint_as_float(w[c].y & 0xFFFF0000u);
        }
    }
    if (h >= Hq) return;
    const float inv = Lr > 0.0f ? 1.0f / Lr : 0.0f;
    *reinterpret_cast<uint2*>(out + (row * Hq + h) * kDl + 16 * t2 + 4 * g) =
        make_uint2(pack_bf16x2(a.x * inv, a.y * inv), pack_bf16x2(a.z * inv, a.w * inv));
    if (lse != nullptr && t2 == 0 && g == 0)
        lse[row * Hq + h] = Ls > 0.0f ? M * 0.69314718055994531f + logf(Ls) : -INFINITY;
}

template <int CH>
static hipError_t launch_merge_few(hipStream_t stream, int rows, int Hq, int ns,
                                   const uint16_t* ws_o, const float* ws_ml, uint16_t* out,
                                   float* lse) {
    const unsigned blocks = static_cast<unsigned>(rows) * ((Hq + 15) / 16) * kT2;
    hipLaunchKernelGGL(merge_few_kernel<CH>, dim3(blocks), dim3(64), 0, stream, Hq, ns, ws_o, ws_ml,
                       out, lse);
    return hipGetLastError();
}

// Split plan: enough (row, split) blocks to occupy the chip, each split a
// whole number of 32-key tiles and at least two of them (fewer, longer splits
// cost more per block than the extra partials cost the merge; measured at
// 16K and 128K context), at most kMaxSplits.
void mla_plan(int rows, int K, int* nsplit, int* slots_per_split) {
    const int tiles = (K + kTile - 1) / kTile;
    int ns = (256 + rows - 1) / rows;
    int cap = tiles / 2;
    if (cap > kMaxSplits) cap = kMaxSplits;
    if (ns > cap) ns = cap;
    if (ns < 1) ns = 1;
    const int tiles_per = (tiles + ns - 1) / ns;
    ns = (tiles + tiles_per - 1) / tiles_per;
    *nsplit = ns;
    *slots_per_split = tiles_per * kTile;
}

size_t mla_workspace_bytes(int rows, int Hq, int K) {
    int ns, sps;
    mla_plan(rows, K, &ns, &sps);
    if (ns == 1) return 0;
    const size_t nwg = static_cast<size_t>((Hq + 15) / 16);
    const size_t blocks = static_cast<size_t>(rows) * ns * nwg;
    const size_t slots = static_cast<size_t>(rows) * ns * Hq;
    return blocks * kT2 * 64 * 4 * sizeof(uint16_t) + slots * 4 * sizeof(float) + 256;
}

template <bool PIPE, int HPB>
static hipError_t launch_mla_kernel(dim3 grid, hipStream_t stream, int S, int Hq, int Lmax,
                                    int K, int sps, int ns, int nitems, int hgroups,
                                    const uint16_t* q, const uint16_t* latent, int64_t lat_rs,
                                    int64_t lat_bs, const uint16_t* rope, int64_t rope_rs,
                                    int64_t rope_bs, const int32_t* idx, float scale_log2,
                                    uint16_t* out, float* lse, uint16_t* ws_o, float* ws_ml,
                                    CacheMap cmap) {
    // thread-safe one-time opt-in to more than 64 KiB of dynamic LDS
    static const hipError_t attr = hipFuncSetAttribute(
        reinterpret_cast<const void*>(&sparse_mla_kernel<PIPE, HPB>),
        hipFuncAttributeMaxDynamicSharedMemorySize, static_cast<int>(kMlaLdsBytes));
    if (attr != hipSuccess) return attr;
    hipLaunchKernelGGL((sparse_mla_kernel<PIPE, HPB>), grid, dim3(4 * HPB), kMlaLdsBytes, stream, S,
                       Hq, Lmax, K, sps, ns, nitems, hgroups, q, latent, lat_rs, lat_bs, rope,
                       rope_rs, rope_bs, idx, scale_log2, out, lse, ws_o, ws_ml, cmap);
    return hipGetLastError();
}

hipError_t launch_sparse_mla(int B, int S, int Hq, int Lmax, int K, const uint16_t* q,
                             const uint16_t* latent, int64_t lat_rs, int64_t lat_bs,
                             const uint16_t* rope, int64_t rope_rs, int64_t rope_bs,
                             const int32_t* idx, float scale, uint16_t* out, float* lse,
                             void* workspace, CacheMap cmap, hipStream_t stream) {
    const int rows = B * S;
    int ns, sps;
    mla_plan(rows, K, &ns, &sps);
    uint16_t* ws_o = nullptr;
    float* ws_ml = nullptr;
    const int nwg = (Hq + 15) / 16;
    if (ns > 1) {
        ws_o = static_cast<uint16_t*>(workspace);
        ws_ml = reinterpret_cast<float*>(ws_o + static_cast<size_t>(rows) * ns * nwg * kT2 * 64 * 4);
    }
    const float scale_log2 = scale * 1.4426950408889634f;
    const int nitems = rows * ns;
    const int hgroups = (Hq + kHeadsPerBlock - 1) / kHeadsPerBlock;
    const int nblocks = ((nitems + 7) / 8) * 8 * hgroups;
    const int hg_few = (Hq + kHeadsPerBlockFew - 1) / kHeadsPerBlockFew;
    const int nb_few = ((nitems + 7) / 8) * 8 * hg_few;
    const bool few = nb_few <= 256;
    hipError_t e;
    if (few) {
        // fewest blocks: 32 heads (2 waves) per block, one block per CU; twice
        // the blocks of the 64-head build and half its LDS operand reads per
        // CU and tile (the two head groups of a (row, split) gather the same
        // rows, the second from L2)
        e = launch_mla_kernel<true, kHeadsPerBlockFew>(
            dim3(nb_few), stream, S, Hq, Lmax, K, sps, ns, nitems, hg_few, q, latent, lat_rs,
            lat_bs, rope, rope_rs, rope_bs, idx, scale_log2, out, lse, ws_o, ws_ml, cmap);
    } else if (nblocks <= 256) {
        // at most one block per CU: the pipelined one-block-per-CU build
        e = launch_mla_kernel<true, kHeadsPerBlock>(
            dim3(nblocks), stream, S, Hq, Lmax, K, sps, ns, nitems, hgroups, q, latent, lat_rs,
            lat_bs, rope, rope_rs, rope_bs, idx, scale_log2, out, lse, ws_o, ws_ml, cmap);
    } else {
        e = launch_mla_kernel<false, kHeadsPerBlock>(
            dim3(nblocks), stream, S, Hq, Lmax, K, sps, ns, nitems, hgroups, q, latent, lat_rs,
            lat_bs, rope, rope_rs, rope_bs, idx, scale_log2, out, lse, ws_o, ws_ml, cmap);
    }
    if (e != hipSuccess) return e;
    if (ns > 1) {
        if (few) {
            e = ns <= 8    ? launch_merge_few<8>(stream, rows, Hq, ns, ws_o, ws_ml, out, lse)
                : ns <= 16 ? launch_merge_few<16>(stream, rows, Hq, ns, ws_o, ws_ml, out, lse)
                           : launch_merge_few<32>(stream, rows, Hq, ns, ws_o, ws_ml, out, lse);
        } else {
            hipLaunchKernelGGL(combine_kernel, dim3(rows * nwg * kCombineQuarters), dim3(256), 0,
                               stream, Hq, ns, ws_o, ws_ml, out, lse);
            e = hipGetLastError();
        }
    }
    return e;
}

}  // namespace dsa
