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
#include <type_traits>

#include "dsa_common.h"

namespace dsa {

typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
constexpr int kDl = 512, kDq = 576;
constexpr int kTile = 32;
// bf16 per K-tile row: 1184 B, 32 B past a multiple of 128 B. Measured with
// the LDS bank-conflict counter on gfx950, this pitch leaves the score operand
// reads (16 rows x one 16-B chunk), the transposing value reads (4 rows x
// 32 B per 16 lanes) and the gather stores free of conflicts; 1168 B and
// 1152 B cost one and three extra cycles per read.
constexpr int kKtStride = kDq + 16;
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

// One 32-key tile for one wave's 16 heads: S^T = K Q^T, the online-softmax
// update and O^T += V^T P^T. Kt: the tile, latent features of key row r at
// Kt + r kPitch; the rotary part of the score operand (k-steps 16 and 17) at
// Kt + rope16 / rope17 for row m = lane % 16, kRopeHalf further for row 16 + m
// (bf16 units). sk: the tile's cache rows (negative: unselected, scored
// -inf). kPipe / kPipeV: LDS operand reads kept in flight ahead of the score
// / value MFMAs.
struct NoWork {
    __device__ void operator()() const {}
};

// max over the four lanes l ^ 16 k (k = 0..3): lane-swap VALU moves, no LDS
__device__ __forceinline__ float max_over_row_groups(float v) {
    const uint32_t u = __float_as_uint(v);
    const auto a = __builtin_amdgcn_permlane16_swap(u, u, false, false);
    v = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
    const uint32_t w = __float_as_uint(v);
    const auto c = __builtin_amdgcn_permlane32_swap(w, w, false, false);
    return fmaxf(__uint_as_float(c[0]), __uint_as_float(c[1]));
}

// sum over the four lanes l ^ 16 k (k = 0..3)
__device__ __forceinline__ float sum_over_row_groups(float v) {
    const uint32_t u = __float_as_uint(v);
    const auto a = __builtin_amdgcn_permlane16_swap(u, u, false, false);
    v = __uint_as_float(a[0]) + __uint_as_float(a[1]);
    const uint32_t w = __float_as_uint(v);
    const auto c = __builtin_amdgcn_permlane32_swap(w, w, false, false);
    return __uint_as_float(c[0]) + __uint_as_float(c[1]);
}

// Q^T operand of one 16-head group: lane (head h, chunk g) holds
// q[row][h][32 ks + 8 g .. +7]; heads past Hq read as zeros.
__device__ __forceinline__ void mla_load_q(const uint16_t* __restrict__ q, int row, int Hq, int h,
                                           int g, bf16x8 (&qreg)[kDq / 32]) {
    const uint16_t* qh = q + (static_cast<int64_t>(row) * Hq + (h < Hq ? h : 0)) * kDq + 8 * g;
#pragma unroll
    for (int ks = 0; ks < kDq / 32; ++ks) {
        uint4 v = *reinterpret_cast<const uint4*>(qh + ks * 32);
        if (h >= Hq) v = make_uint4(0u, 0u, 0u, 0u);
        qreg[ks] = __builtin_bit_cast(bf16x8, v);
    }
}

// V^T operand of output tile t2 (16 latent features) for the 32 keys of the
// tile at Kt (rows kPitch apart), by transposing reads: lane 4e+q of group g
// reads features 4q.. of key 4g+e (k-step keys 0..15) and of key 16+4g+e
// (keys 16..31)
template <int kPitch>
__device__ __forceinline__ bf16x8 mla_read_v(const uint16_t* Kt, int lane, int t2) {
    const int tr_off = (4 * (lane >> 4) + ((lane >> 2) & 3)) * kPitch + 4 * (lane & 3);
    // whole-register bit casts: element-wise 16-bit extraction here was
    // mis-scheduled into a lane-mixing permute
    const uint2 lo = __builtin_bit_cast(uint2, lds_read_tr16(Kt + tr_off + 16 * t2));
    const uint2 hi = __builtin_bit_cast(uint2, lds_read_tr16(Kt + tr_off + 16 * kPitch + 16 * t2));
    return __builtin_bit_cast(bf16x8, make_uint4(lo.x, lo.y, hi.x, hi.y));
}

// The scores and online-softmax half of one 32-key tile for NG groups of 16
// heads held by one wave: S^T = K Q^T (each score operand read from LDS
// serves all NG groups), the running maximum, sums and (when the maximum
// moves) the accumulator rescale; P^T of group j, as the bf16 MFMA operand,
// goes to pv[j]. Kt: the tile, latent features of key row r at
// Kt + r kPitch; the rotary part of the score operand (k-steps 16 and 17) at
// Kt + rope16 / rope17 for row m = lane % 16, kRopeHalf further for row
// 16 + m (bf16 units). sk: the tile's cache rows (negative: unselected,
// scored -inf); with kCounted the rows are compacted and the first nk keys
// of the tile are the selected ones (no LDS reads for the mask). kPipe:
// score operand reads kept in flight ahead of the MFMAs; kChains: separate
// accumulation chains per score output; the first kEarlyV value operands of
// the tile are read into va while the softmax runs. mid(): work run once the
// score MFMAs are issued, before the softmax waits for them.
template <int NG, int kPipe, int kPipeV, int kEarlyV, int kPitch, int kRopeHalf, int kChains,
          bool kCounted, typename Mid = NoWork>
__device__ __forceinline__ void mla_scores(const uint16_t* Kt, int rope16, int rope17,
                                           const int* sk, int nk, int lane,
                                           const bf16x8 (&qreg)[NG][kDq / 32],
                                           v4f (&acc)[NG][kT2], float scale_log2,
                                           float (&m_run)[NG], float (&l_run)[NG],
                                           float (&lr_run)[NG], bf16x8 (&va)[kPipeV],
                                           bf16x8 (&pv)[NG], Mid mid = Mid()) {
    const int m = lane & 15, g = lane >> 4;
    // score operand of k-step ks (compile-time) for keys m (h = 0) and 16 + m
    const int lat_off = m * kPitch + 8 * g;
    auto kop = [&](int ks, int hh) -> bf16x8 {
        const int off = ks < kDl / 32 ? lat_off + 32 * ks + hh * 16 * kPitch
                                      : (ks == kDl / 32 ? rope16 : rope17) + hh * kRopeHalf;
        return *reinterpret_cast<const bf16x8*>(Kt + off);
    };
    // S^T for keys 0..15 (s0) and 16..31 (s1) of each group; lane holds keys
    // 4g+i. Consecutive k-steps rotate over kChains accumulators.
    v4f s0[NG], s1[NG];
    {
        v4f c0[NG][kChains], c1[NG][kChains];
#pragma unroll
        for (int j = 0; j < NG; ++j)
#pragma unroll
            for (int c = 0; c < kChains; ++c) {
                c0[j][c] = v4f{0.0f, 0.0f, 0.0f, 0.0f};
                c1[j][c] = v4f{0.0f, 0.0f, 0.0f, 0.0f};
            }
        bf16x8 a0[kPipe], a1[kPipe];
#pragma unroll
        for (int d = 0; d < kPipe; ++d) {
            a0[d] = kop(d, 0);
            a1[d] = kop(d, 1);
        }
        DSA_SCHED_GROUP(kSchedDsRead, 2 * kPipe);
#pragma unroll
        for (int ks = 0; ks < kDq / 32; ++ks) {
            const int sl = ks % kPipe, ch = ks % kChains;
#pragma unroll
            for (int j = 0; j < NG; ++j) {
                c0[j][ch] = mfma_bf16_16x16x32(a0[sl], qreg[j][ks], c0[j][ch]);
                c1[j][ch] = mfma_bf16_16x16x32(a1[sl], qreg[j][ks], c1[j][ch]);
            }
            DSA_SCHED_GROUP(kSchedMfma, 2 * NG);
            if (ks + kPipe < kDq / 32) {
                a0[sl] = kop(ks + kPipe, 0);
                a1[sl] = kop(ks + kPipe, 1);
                DSA_SCHED_GROUP(kSchedDsRead, 2);
            }
        }
        mid();
#pragma unroll
        for (int j = 0; j < NG; ++j) {
            s0[j] = c0[j][0];
            s1[j] = c1[j][0];
#pragma unroll
            for (int c = 1; c < kChains; ++c) {
                s0[j] += c0[j][c];
                s1[j] += c1[j][c];
            }
        }
    }
    // the first V^T operands are read while the softmax runs
#pragma unroll
    for (int d = 0; d < kEarlyV; ++d) va[d] = mla_read_v<kPitch>(Kt, lane, d);
    if constexpr (kEarlyV > 0) DSA_SCHED_GROUP(kSchedDsRead, 2 * kEarlyV);

    // kFull: a counted tile whose 32 keys are all selected (every tile of a
    // split but its last) needs no mask
    auto softmax = [&](auto full_c) {
        constexpr bool kFull = decltype(full_c)::value;
        bool valid[8];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            valid[i] = kFull || (kCounted ? 4 * g + i < nk : sk[4 * g + i] >= 0);
            valid[4 + i] = kFull || (kCounted ? 16 + 4 * g + i < nk : sk[16 + 4 * g + i] >= 0);
        }
#pragma unroll
        for (int j = 0; j < NG; ++j) {
            float z[8];
            float tmax = -INFINITY;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                z[i] = valid[i] ? s0[j][i] * scale_log2 : -INFINITY;
                z[4 + i] = valid[4 + i] ? s1[j][i] * scale_log2 : -INFINITY;
            }
#pragma unroll
            for (int i = 0; i < 8; ++i) tmax = fmaxf(tmax, z[i]);
            tmax = max_over_row_groups(tmax);
            // Lazy rescaling: probabilities are taken relative to a reference
            // maximum m_run that only moves when the running maximum exceeds
            // it by more than 8 (so p <= 2^8, exact enough in float and bf16).
            if (tmax > m_run[j] + 8.0f) {
                const float corr = (m_run[j] == -INFINITY) ? 0.0f : exp2f(m_run[j] - tmax);
                l_run[j] *= corr;
                lr_run[j] *= corr;
                m_run[j] = tmax;
                if (__ballot(corr != 1.0f)) {
#pragma unroll
                    for (int t2 = 0; t2 < kT2; ++t2) acc[j][t2] *= corr;
                }
            }
            // while m_run is -inf every z is -inf too, and 2^(-inf - 0) = 0
            const float mref = m_run[j] == -INFINITY ? 0.0f : m_run[j];
            float psum = 0.0f, prsum = 0.0f;
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                const float pe = __builtin_amdgcn_exp2f(z[i] - mref);
                const __bf16 pb = static_cast<__bf16>(pe);
                pv[j][i] = pb;
                psum += pe;
                prsum += static_cast<float>(pb);
            }
            l_run[j] += psum;
            lr_run[j] += prsum;
        }
    };
    if constexpr (kCounted) {
        if (nk >= kTile) softmax(std::true_type{});
        else softmax(std::false_type{});
    } else {
        softmax(std::false_type{});
    }
}

// The value half: O^T += V^T P^T over the tile at Kt for the NG groups (each
// V^T operand read from LDS serves all of them), the first kPipeV V^T
// operands already in va, the rest read kPipeV steps ahead.
template <int NG, int kPipeV, int kPitch>
__device__ __forceinline__ void mla_values(const uint16_t* Kt, int lane, const bf16x8 (&pv)[NG],
                                           bf16x8 (&va)[kPipeV], v4f (&acc)[NG][kT2]) {
#pragma unroll
    for (int t2 = 0; t2 < kT2; ++t2) {
        const int sl = t2 % kPipeV;
#pragma unroll
        for (int j = 0; j < NG; ++j) acc[j][t2] = mfma_bf16_16x16x32(va[sl], pv[j], acc[j][t2]);
        DSA_SCHED_GROUP(kSchedMfma, NG);
        if (t2 + kPipeV < kT2) {
            va[sl] = mla_read_v<kPitch>(Kt, lane, t2 + kPipeV);
            DSA_SCHED_GROUP(kSchedDsRead, 2);
        }
    }
}

// One whole tile: the scores half, then the value half.
template <int NG, int kPipe, int kPipeV, int kPitch, int kRopeHalf, int kChains,
          bool kCounted, typename Mid = NoWork>
__device__ __forceinline__ void mla_tile_math(const uint16_t* Kt, int rope16, int rope17,
                                              const int* sk, int nk, int lane,
                                              const bf16x8 (&qreg)[NG][kDq / 32],
                                              v4f (&acc)[NG][kT2], float scale_log2,
                                              float (&m_run)[NG], float (&l_run)[NG],
                                              float (&lr_run)[NG], Mid mid = Mid()) {
    bf16x8 va[kPipeV], pv[NG];
    mla_scores<NG, kPipe, kPipeV, kPipeV, kPitch, kRopeHalf, kChains, kCounted>(
        Kt, rope16, rope17, sk, nk, lane, qreg, acc, scale_log2, m_run, l_run, lr_run, va, pv,
        mid);
    mla_values<NG, kPipeV, kPitch>(Kt, lane, pv, va, acc);
}

// A wave's result for its 16 heads (lane holds O^T[16 t2 + 4 g + i][h],
// i = 0..3): with one split the normalised bf16 output and the lse; else the
// unnormalised bf16 partial block and its (m, lr, l) for the merge. kStream:
// partials stored past L2.
template <bool kStream>
__device__ __forceinline__ void mla_store_result(const v4f (&acc)[kT2], float m_run, float l_tot,
                                                 float lr_tot, int lane, int wg, int Hq, int row,
                                                 int split, int nsplit, uint16_t* __restrict__ out,
                                                 float* __restrict__ lse,
                                                 uint16_t* __restrict__ ws_o,
                                                 float* __restrict__ ws_ml) {
    const int g = lane >> 4, h = wg * 16 + (lane & 15);
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
            if constexpr (kStream)
                __builtin_nontemporal_store(u32x2{lo, hi}, reinterpret_cast<u32x2*>(wo + t2 * 256));
            else
                *reinterpret_cast<uint2*>(wo + t2 * 256) = make_uint2(lo, hi);
        }
        if (g == 0 && h < Hq)
            *reinterpret_cast<float4*>(ws_ml + ((static_cast<int64_t>(row) * nsplit + split) * Hq + h) * 4) =
                make_float4(m_run, lr_tot, l_tot, 0.0f);
    }
}

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

    bf16x8 qreg[1][kDq / 32];
    mla_load_q(q, row, Hq, h, g, qreg[0]);
    v4f acc[1][kT2];
#pragma unroll
    for (int t2 = 0; t2 < kT2; ++t2) acc[0][t2] = v4f{0.0f, 0.0f, 0.0f, 0.0f};
    // l_run sums the float32 probabilities (for lse); lr_run sums the bf16
    // values that actually weight the latent rows (for the normalisation).
    float m_run[1] = {-INFINITY}, l_run[1] = {0.0f}, lr_run[1] = {0.0f};

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
        mla_tile_math<1, kPipe, kPipeV, kKtStride, 16 * kKtStride, 2, false>(
            Kt, m * kKtStride + 8 * g + kDl, m * kKtStride + 8 * g + kDl + 32, sidx + t * kTile,
            0, lane, qreg, acc, scale_log2, m_run, l_run, lr_run);
    };
    for (int t = 0; t < ntiles; ++t) tile_step(t, GA);

    const float l_tot = sum_over_row_groups(l_run[0]);
    const float lr_tot = sum_over_row_groups(lr_run[0]);
    if (!active) return;
    mla_store_result<PIPE && HPB == kHeadsPerBlockFew>(acc[0], m_run[0], l_tot, lr_tot, lane, wg,
                                                       Hq, row, split, nsplit, out, lse, ws_o,
                                                       ws_ml);
}

// The build for grids of more than one block per CU with more than 64 heads
// (batched decode, prefill): 8 waves serve 128 heads of one (row, split), so
// every selected row is gathered once for all its heads, and the gather runs
// two tiles ahead of the math through a ring of three LDS tiles filled
// straight from global memory (global_load_lds, 16 bytes per lane, no
// registers held). A ring tile keeps the latent and rotary parts apart:
//   latent: 32 rows of 1024 B at a 1056-B pitch (32 B past a multiple of
//           256 B: the score operand and transposing value reads are free of
//           bank conflicts, measured), one load instruction per row, whose
//           64 lanes read the row's 64 chunks from one scalar base address;
//   rotary: wave w's 1 KiB block holds rows 4w..4w+3, 128 B each, 16-byte
//           chunk c of row r stored at c ^ (r & 6) (conflict free as well),
//           filled by the first 32 lanes of one instruction (the other 32
//           repeat them into the unused half).
// Wave w loads rows 4w..4w+3: four latent instructions and one rotary, the
// same five per wave and tile. Unselected rows read a block of zeros. The
// split's selected rows are compacted first, so tiles of unselected slots
// (a causal row shorter than the top-k count, say) cost nothing.
constexpr int kRingWaves = 8;
constexpr int kRingGroups = 1;                                 // 16-head groups per wave
constexpr int kRingHeads = 16 * kRingGroups * kRingWaves;
constexpr int kRingStages = 3;
constexpr int kRingRows = kTile / kRingWaves;                  // rows loaded per wave
constexpr int kRingLoads = kRingRows + 1;                      // per wave and tile
constexpr int kLatPitch = kDl + 16;                            // bf16 (1056 B)
constexpr int kRingLatBytes = kTile * kLatPitch * 2;           // 33,792
constexpr int kRingStageBytes = kRingLatBytes + kRingWaves * 1024;
constexpr int kRopeHalfRows = 16 / kRingRows * 512;            // bf16 from row m to 16 + m
static_assert(kRingRows == 4, "one rotary instruction (4 rows of 128 B, twice) per wave");
constexpr size_t kRingLdsBytes =
    static_cast<size_t>(kRingStages) * kRingStageBytes + sizeof(int) * (kMaxSlots + kRingWaves);

__device__ uint4 mla_zero_kb[64];    // 1 KiB of zeros (zero-initialised, never written)

// The ring's loads, waits and barrier are inline asm that the compiler sees
// only as opaque memory operations. Written with the global_load_lds builtin
// the compiler cannot tell the ring stages apart, and makes the first
// transposing LDS read of every tile wait for all loads in flight, the next
// tiles' included (vmcnt(0)), which leaves nothing in flight during the math.
// Here the waits are exactly the ring's: before a tile is read, every load
// but those of the next tile has landed (vector-memory loads complete in
// issue order), then the barrier makes all waves' loads visible.
// 16 bytes per lane to LDS address m0 + 16 lane: from base + voff (scalar
// base, per-lane 32-bit offset) or from a per-lane 64-bit address.
__device__ __forceinline__ void ring_load_s(uint64_t base, uint32_t voff, uint32_t lds_dst) {
    asm volatile("s_mov_b32 m0, %2\n\tglobal_load_lds_dwordx4 %0, %1"
                 :
                 : "v"(voff), "s"(base), "s"(lds_dst)
                 : "memory");
}
__device__ __forceinline__ void ring_load_v(uint64_t addr, uint32_t lds_dst) {
    asm volatile("s_mov_b32 m0, %1\n\tglobal_load_lds_dwordx4 %0, off"
                 :
                 : "v"(addr), "s"(lds_dst)
                 : "memory");
}
template <int n>
__device__ __forceinline__ void ring_wait_barrier() {
    asm volatile("s_waitcnt vmcnt(%0)\n\ts_barrier" : : "n"(n) : "memory");
}

__global__ __launch_bounds__(64 * kRingWaves, 1) void sparse_mla_ring_kernel(
    int S, int Hq, int Lmax, int K, int slots_per_split, int nsplit, int nitems, int hgroups,
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ latent, int64_t lat_rs,
    int64_t lat_bs, const uint16_t* __restrict__ rope, int64_t rope_rs, int64_t rope_bs,
    const int32_t* __restrict__ idx, float scale_log2, uint16_t* __restrict__ out,
    float* __restrict__ lse, uint16_t* __restrict__ ws_o, float* __restrict__ ws_ml, CacheMap cmap) {
    extern __shared__ __align__(16) unsigned char smem[];
    int* sidx = reinterpret_cast<int*>(smem + kRingStages * kRingStageBytes);

    // launch index -> (work item = row * nsplit + split, head group): launch
    // L runs on XCD L % 8; the nsplit splits of a row (and its head groups)
    // go to one XCD, consecutive rows round the XCDs
    const int L = blockIdx.x;
    const int jj = (L >> 3) / hgroups;
    const int hg = (L >> 3) % hgroups;
    const int item_l = ((jj / nsplit) * 8 + (L & 7)) * nsplit + jj % nsplit;
    if (item_l >= nitems) return;
    // items in reverse: in a causal prefill the last rows select the most
    // keys, so the longest blocks start first and the short ones fill the
    // tail (a row's splits stay together)
    const int item = nitems - 1 - item_l;
    const int row = item / nsplit, split = item - row * nsplit;
    const int64_t b = row / S;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int m = lane & 15, g = lane >> 4;
    constexpr int kThr = 64 * kRingWaves;
    const int wg0 = (hg * kRingWaves + wave) * kRingGroups;        // first 16-head group
    const bool active = wg0 * 16 < Hq;

    const int j_begin = split * slots_per_split;
    const int j_end = min(K, j_begin + slots_per_split);
    const int count = j_end - j_begin;
    const bool paged = cmap.table != nullptr;
    // the split's cache rows, compacted: the selected, present rows first (in
    // slot order); the tail of the last tile is -1
    int nvalid = 0;
    {
        // every index (and page-table) load of the split issued before the
        // first is used: one memory round trip instead of one per 512 slots
        constexpr int kRounds = kMaxSlots / kThr;
        static_assert(kRounds * kThr == kMaxSlots, "slot rounds");
        int* wcnt = sidx + kMaxSlots;                              // per-wave counts
        const int32_t* irow = idx + static_cast<int64_t>(row) * K + j_begin;
        int vv[kRounds];
#pragma unroll
        for (int r = 0; r < kRounds; ++r) vv[r] = irow[min(r * kThr + tid, count - 1)];
#pragma unroll
        for (int r = 0; r < kRounds; ++r) {
            const int p = r * kThr + tid < count ? vv[r] : -1;
            vv[r] = (p >= 0 && p < Lmax) ? (paged ? static_cast<int>(cmap.row(b, p)) : p) : -1;
        }
#pragma unroll
        for (int r = 0; r < kRounds; ++r) {
            if (r * kThr >= count) break;                          // uniform
            const int v = vv[r];
            const uint64_t bal = __ballot(v >= 0);
            const int below = __builtin_amdgcn_mbcnt_hi(static_cast<uint32_t>(bal >> 32),
                                                        __builtin_amdgcn_mbcnt_lo(static_cast<uint32_t>(bal), 0));
            if (lane == 0) wcnt[wave] = __popcll(bal);
            __syncthreads();
            int off = nvalid, tot = 0;
#pragma unroll
            for (int w = 0; w < kRingWaves; ++w) {
                const int c = wcnt[w];
                off += w < wave ? c : 0;
                tot += c;
            }
            if (v >= 0) sidx[off + below] = v;
            nvalid += tot;
            __syncthreads();                                       // wcnt reused
        }
    }
    const int ntiles = (nvalid + kTile - 1) / kTile;
    for (int i = nvalid + tid; i < ntiles * kTile; i += kThr) sidx[i] = -1;

    bf16x8 qreg[kRingGroups][kDq / 32];
#pragma unroll
    for (int j = 0; j < kRingGroups; ++j) mla_load_q(q, row, Hq, (wg0 + j) * 16 + m, g, qreg[j]);
    // q in registers before the ring's loads are issued: the compiler's own
    // waits for the q loads would otherwise count the ring's loads too
#pragma unroll
    for (int j = 0; j < kRingGroups; ++j)
#pragma unroll
        for (int ks = 0; ks < kDq / 32; ++ks) asm volatile("" : "+v"(qreg[j][ks]));
    v4f acc[kRingGroups][kT2];
#pragma unroll
    for (int j = 0; j < kRingGroups; ++j)
#pragma unroll
        for (int t2 = 0; t2 < kT2; ++t2) acc[j][t2] = v4f{0.0f, 0.0f, 0.0f, 0.0f};
    float m_run[kRingGroups], l_run[kRingGroups], lr_run[kRingGroups];
#pragma unroll
    for (int j = 0; j < kRingGroups; ++j) {
        m_run[j] = -INFINITY;
        l_run[j] = 0.0f;
        lr_run[j] = 0.0f;
    }
    const uint64_t lat_b =
        reinterpret_cast<uint64_t>(latent + (paged ? 0 : b * lat_bs));
    const uint64_t rope_b = reinterpret_cast<uint64_t>(rope + (paged ? 0 : b * rope_bs));
    const uint64_t zero = reinterpret_cast<uint64_t>(&mla_zero_kb[0]);
    const int wave_u = __builtin_amdgcn_readfirstlane(wave);
    const uint32_t lds0 = static_cast<uint32_t>(reinterpret_cast<uintptr_t>(smem));
    __syncthreads();                               // sidx ready

    auto issue = [&](int t) {
        const uint32_t st = lds0 + (t % kRingStages) * kRingStageBytes;
        // this wave's four rows: cache rows from one broadcast LDS read
        const int4 pa = *reinterpret_cast<const int4*>(sidx + t * kTile + kRingRows * wave_u);
        const int pr[4] = {pa.x, pa.y, pa.z, pa.w};
        int ln = lane;
        asm volatile("" : "+v"(ln));
        // latent: row 4w + j, lane l reads bytes 16 l .. of the row
#pragma unroll
        for (int j = 0; j < kRingRows; ++j) {
            const int p = __builtin_amdgcn_readfirstlane(pr[j]);
            const uint64_t base =
                p >= 0 ? lat_b + static_cast<uint64_t>(static_cast<uint32_t>(p)) *
                                     static_cast<uint64_t>(lat_rs * 2)
                       : zero;
            ring_load_s(base, 16u * static_cast<uint32_t>(ln),
                        st + (kRingRows * wave_u + j) * (kLatPitch * 2));
        }
        // rotary: lane l (and l + 32) fills chunk c = l % 8 of row 4w + j,
        // j = (l / 8) % 4, from source chunk c ^ (row & 6)
        {
            const int j = (ln >> 3) & 3, c = ln & 7;
            const int p = (j & 2) ? ((j & 1) ? pr[3] : pr[2]) : ((j & 1) ? pr[1] : pr[0]);
            const int sc = c ^ ((kRingRows * wave_u + j) & 6);
            const uint64_t a =
                p >= 0 ? rope_b + static_cast<uint64_t>(static_cast<uint32_t>(p)) *
                                      static_cast<uint64_t>(rope_rs * 2) +
                             16u * static_cast<uint32_t>(sc)
                       : zero + 16u * static_cast<uint32_t>(ln);
            ring_load_v(a, st + kRingLatBytes + 1024 * wave_u);
        }
    };

    // rotary operand offsets (bf16 within a stage) of k-steps 16 and 17 for
    // row m: block m / 4, row m % 4, chunk (4 (ks - 16) + g) ^ (m & 6)
    const int rbase = kRingLatBytes / 2 + (m >> 2) * 512 + (m & 3) * 64;
    const int rope16 = rbase + 8 * (g ^ (m & 6));
    const int rope17 = rbase + 8 * ((4 + g) ^ (m & 6));
    // LDS operand reads in flight (the register budget of two waves per SIMD)
    constexpr int kPipe = 2, kPipeV = 4;
    if (ntiles > 0) issue(0);
    if (ntiles > 1) issue(1);
    for (int t = 0; t < ntiles; ++t) {

        // tile t has landed once only tile t + 1's loads are in flight; the
        // barrier: every wave's loads, and tile t - 1 consumed
        if (t + 1 < ntiles) ring_wait_barrier<kRingLoads>();
        else ring_wait_barrier<0>();
        if (active)
            mla_tile_math<kRingGroups, kPipe, kPipeV, kLatPitch, kRopeHalfRows, 1, true>(
                reinterpret_cast<const uint16_t*>(smem + (t % kRingStages) * kRingStageBytes),
                rope16, rope17, sidx, nvalid - t * kTile, lane, qreg, acc, scale_log2, m_run,
                l_run, lr_run);
        // the loads of tile t + 2 (into tile t - 1's stage) are issued after
        // the tile's math, where the wave would wait at the next barrier
        // anyway: issued during the score MFMAs they held up the MFMA stream
        if (t + 2 < ntiles) issue(t + 2);
    }

    // lane, head group and activity recomputed here (mbcnt, scalars) rather
    // than kept live through the tile loop
    const int lane_e = static_cast<int>(
        __builtin_amdgcn_mbcnt_hi(~0u, __builtin_amdgcn_mbcnt_lo(~0u, 0u)));
    const int m_e = lane_e & 15, g_e = lane_e >> 4;
    const int wg0_e = (hg * kRingWaves + wave_u) * kRingGroups;
    const bool active_e = wg0_e * 16 < Hq;
    if (nsplit == 1) {
        // one split: the normalised rows go out through LDS (the ring's
        // stages are free now), each wave's 16 head rows at a 1,040-byte
        // pitch, then one whole 1 KiB head row per store instruction,
        // streamed past L2 (which keeps the cache rows other blocks gather)
        static_assert(kRingGroups == 1, "one 16-head group per wave");
        constexpr int kOutPitch = kDl + 8;                        // bf16
        static_assert(static_cast<size_t>(kRingWaves) * 16 * kOutPitch * 2 <= kRingLdsBytes,
                      "output staging fits the ring's LDS");
        __syncthreads();                                           // every wave past its last tile
        if (!active_e) return;
        const float l_tot = sum_over_row_groups(l_run[0]);
        const float lr_tot = sum_over_row_groups(lr_run[0]);
        const int h = wg0_e * 16 + m_e;
        if (lse != nullptr && g_e == 0 && h < Hq)
            lse[static_cast<int64_t>(row) * Hq + h] =
                l_tot > 0.0f ? m_run[0] * 0.69314718055994531f + logf(l_tot) : -INFINITY;
        const float inv = lr_tot > 0.0f ? 1.0f / lr_tot : 0.0f;
        uint16_t* stg = reinterpret_cast<uint16_t*>(smem) + wave_u * 16 * kOutPitch;
#pragma unroll
        for (int t2 = 0; t2 < kT2; ++t2)
            *reinterpret_cast<uint2*>(stg + m_e * kOutPitch + 16 * t2 + 4 * g_e) =
                make_uint2(pack_bf16x2(acc[0][t2][0] * inv, acc[0][t2][1] * inv),
                           pack_bf16x2(acc[0][t2][2] * inv, acc[0][t2][3] * inv));
#pragma unroll
        for (int k = 0; k < 16; ++k) {
            if (wg0_e * 16 + k >= Hq) break;                       // wave-uniform
            __builtin_nontemporal_store(
                *reinterpret_cast<const u32x4*>(stg + k * kOutPitch + 8 * lane_e),
                reinterpret_cast<u32x4*>(out + (static_cast<int64_t>(row) * Hq + wg0_e * 16 + k) * kDl +
                                         8 * lane_e));
        }
        return;
    }
    if (!active_e) return;
#pragma unroll
    for (int j = 0; j < kRingGroups; ++j) {
        const float l_tot = sum_over_row_groups(l_run[j]);
        const float lr_tot = sum_over_row_groups(lr_run[j]);
        if ((wg0_e + j) * 16 < Hq)
            mla_store_result<false>(acc[j], m_run[j], l_tot, lr_tot, lane_e, wg0_e + j, Hq, row,
                                    split, nsplit, out, lse, ws_o, ws_ml);
    }
}

// The build for the fewest blocks when every split holds at most 64
// selected slots (one or two rows at K = 2048): 2 waves of 16 heads, and
// all 64 keys of the split at once instead of two 32-key tiles in turn.
// Both tiles' rows are requested together (each thread reads its rows'
// indices itself, so the gather starts as soon as they arrive, without an
// LDS round trip), S^T is computed for the 64 keys, one softmax runs over
// them (no running maximum to carry or rescale: the block sees its keys
// once), and the value product takes two 32-key MFMA steps per feature
// tile. Against the tile loop this removes one gather round trip, one
// softmax and two barriers from each block's dependent chain.
constexpr int kPairKeys = 2 * kTile;
constexpr size_t kPairLdsBytes =
    sizeof(uint16_t) * kPairKeys * kKtStride + sizeof(int) * kPairKeys;

template <int HPB>
__global__ __launch_bounds__(4 * HPB, 1) void sparse_mla_pair_kernel(
    int S, int Hq, int Lmax, int K, int slots_per_split, int nsplit, int nitems, int hgroups,
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ latent, int64_t lat_rs,
    int64_t lat_bs, const uint16_t* __restrict__ rope, int64_t rope_rs, int64_t rope_bs,
    const int32_t* __restrict__ idx, float scale_log2, uint16_t* __restrict__ out,
    float* __restrict__ lse, uint16_t* __restrict__ ws_o, float* __restrict__ ws_ml, CacheMap cmap) {
    extern __shared__ __align__(16) unsigned char smem[];
    uint16_t* Kt = reinterpret_cast<uint16_t*>(smem);
    int* sidx = reinterpret_cast<int*>(Kt + kPairKeys * kKtStride);
    constexpr int kThr = 4 * HPB;                                 // one wave per 16 heads
    constexpr int kRP = kThr / 8;                                 // rows per gather pass
    constexpr int kNP = kPairKeys / kRP;                          // gather passes (4 or 2)

    const int L = blockIdx.x;
    const int item = (L / (8 * hgroups)) * 8 + (L & 7);
    const int hg = (L / 8) % hgroups;
    if (item >= nitems) return;
    const int row = item / nsplit, split = item - row * nsplit;
    const int64_t b = row / S;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int m = lane & 15, g = lane >> 4;
    const int wg = hg * (HPB / 16) + wave;                        // 16-head group
    const int h = wg * 16 + m;
    const bool active = wg * 16 < Hq;
    const int j_begin = split * slots_per_split;
    const int count = min(K, j_begin + slots_per_split) - j_begin;   // 1..64
    const bool paged = cmap.table != nullptr;
    const uint16_t* lat_b = latent + (paged ? 0 : b * lat_bs);
    const uint16_t* rope_b = rope + (paged ? 0 : b * rope_bs);
    const int32_t* irow = idx + static_cast<int64_t>(row) * K + j_begin;

    // Cache rows of the slots (-1: unselected, out of range or page not
    // present). Every index (and page-table) load is issued unconditionally
    // at a clamped address and masked afterwards: a lane-dependent branch
    // around a load makes the compiler wait for it before the next one.
    const int gkey = tid >> 3, gsub = tid & 7;
    constexpr int kNI = kNP + 1;                  // the gather rows, then slot tid
    int sl[kNI], pidx[kNI];
#pragma unroll
    for (int u = 0; u < kNI; ++u) {
        sl[u] = u < kNP ? gkey + kRP * u : tid;
        pidx[u] = irow[min(sl[u], count - 1)];
    }
    if (paged) {
        int pg[kNI];
#pragma unroll
        for (int u = 0; u < kNI; ++u) {
            const int pc = min(max(pidx[u], 0), Lmax - 1);
            pg[u] = cmap.table[b * cmap.max_pages + (pc >> cmap.page_shift)];
        }
#pragma unroll
        for (int u = 0; u < kNI; ++u) {
            const int p = pidx[u];
            const bool ok = sl[u] < count && p >= 0 && p < Lmax && pg[u] >= 0 &&
                            pg[u] < cmap.num_pages;
            pidx[u] = ok ? static_cast<int>((static_cast<int64_t>(pg[u]) << cmap.page_shift) |
                                            (p & ((1 << cmap.page_shift) - 1)))
                         : -1;
        }
    } else {
#pragma unroll
        for (int u = 0; u < kNI; ++u) {
            const int p = pidx[u];
            pidx[u] = (sl[u] < count && p >= 0 && p < Lmax) ? p : -1;
        }
    }
    int prow[kNP];
#pragma unroll
    for (int pp = 0; pp < kNP; ++pp) prow[pp] = pidx[pp];
    if (tid < kPairKeys) sidx[tid] = pidx[kNP];
    uint4 G[kNP][9];
#pragma unroll
    for (int pp = 0; pp < kNP; ++pp) {
        const int pc = prow[pp] >= 0 ? prow[pp] : 0;
        const uint16_t* lrow = lat_b + static_cast<int64_t>(pc) * lat_rs + gsub * 8;
        const uint16_t* rrow = rope_b + static_cast<int64_t>(pc) * rope_rs + gsub * 8;
#pragma unroll
        for (int i = 0; i < 8; ++i) G[pp][i] = *reinterpret_cast<const uint4*>(lrow + 64 * i);
        G[pp][8] = *reinterpret_cast<const uint4*>(rrow);
    }
    // Q^T operand: lane (head h, chunk g) holds q[h][32 ks + 8 g .. +7]
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
#pragma unroll
    for (int pp = 0; pp < kNP; ++pp) {
        const int key = gkey + kRP * pp;
        if (prow[pp] < 0) {
#pragma unroll
            for (int i = 0; i < 9; ++i) G[pp][i] = make_uint4(0u, 0u, 0u, 0u);
        }
        uint16_t* dst = Kt + key * kKtStride + gsub * 8;
#pragma unroll
        for (int i = 0; i < 8; ++i) *reinterpret_cast<uint4*>(dst + 64 * i) = G[pp][i];
        *reinterpret_cast<uint4*>(dst + 512) = G[pp][8];
    }
    __syncthreads();

    float m_tot = -INFINITY, l_tot = 0.0f, lr_tot = 0.0f;
    v4f acc[kT2];
#pragma unroll
    for (int t2 = 0; t2 < kT2; ++t2) acc[t2] = v4f{0.0f, 0.0f, 0.0f, 0.0f};
    if (active) {
        // S^T for keys 16 kt .. 16 kt + 15 (kt < 4); lane holds keys 16 kt + 4 g + i
        v4f s[4];
        {
            v4f c[4][2];
#pragma unroll
            for (int kt = 0; kt < 4; ++kt) c[kt][0] = c[kt][1] = v4f{0.0f, 0.0f, 0.0f, 0.0f};
            constexpr int kPipe = 2;
            bf16x8 a[4][kPipe];
#pragma unroll
            for (int d = 0; d < kPipe; ++d)
#pragma unroll
                for (int kt = 0; kt < 4; ++kt)
                    a[kt][d] = *reinterpret_cast<const bf16x8*>(
                        Kt + (16 * kt + m) * kKtStride + 8 * g + d * 32);
#pragma unroll
            for (int ks = 0; ks < kDq / 32; ++ks) {
                const int sl = ks % kPipe;
#pragma unroll
                for (int kt = 0; kt < 4; ++kt)
                    c[kt][ks & 1] = mfma_bf16_16x16x32(a[kt][sl], qreg[ks], c[kt][ks & 1]);
                if (ks + kPipe < kDq / 32) {
#pragma unroll
                    for (int kt = 0; kt < 4; ++kt)
                        a[kt][sl] = *reinterpret_cast<const bf16x8*>(
                            Kt + (16 * kt + m) * kKtStride + 8 * g + (ks + kPipe) * 32);
                }
            }
#pragma unroll
            for (int kt = 0; kt < 4; ++kt) s[kt] = c[kt][0] + c[kt][1];
        }
        // one softmax over the 64 keys (log2 units)
        float z[16];
        float tmax = -INFINITY;
#pragma unroll
        for (int kt = 0; kt < 4; ++kt)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int key = 16 * kt + 4 * g + i;
                z[4 * kt + i] = sidx[key] >= 0 ? s[kt][i] * scale_log2 : -INFINITY;
                tmax = fmaxf(tmax, z[4 * kt + i]);
            }
        tmax = fmaxf(tmax, __shfl_xor(tmax, 16));
        tmax = fmaxf(tmax, __shfl_xor(tmax, 32));
        m_tot = tmax;
        // P^T operands of the two 32-key steps: step u holds keys
        // 32 u + 4 g + i (i < 4) and 32 u + 16 + 4 g + i, the order of the V^T
        // transposing reads below
        bf16x8 pv[2];
        float psum = 0.0f, prsum = 0.0f;
        const bool live = tmax != -INFINITY;
#pragma unroll
        for (int u = 0; u < 2; ++u)
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                const float pe = live ? __builtin_amdgcn_exp2f(z[8 * u + i] - tmax) : 0.0f;
                const __bf16 pb = static_cast<__bf16>(pe);
                pv[u][i] = pb;
                psum += pe;
                prsum += static_cast<float>(pb);
            }
        l_tot = psum + __shfl_xor(psum, 16);
        l_tot += __shfl_xor(l_tot, 32);
        lr_tot = prsum + __shfl_xor(prsum, 16);
        lr_tot += __shfl_xor(lr_tot, 32);
        // O^T += V^T P^T over the two 32-key steps
        const int tr_off = (4 * g + ((lane >> 2) & 3)) * kKtStride + 4 * (lane & 3);
        auto read_v = [&](int u, int t2) -> bf16x8 {
            const uint16_t* base = Kt + 32 * u * kKtStride + tr_off + 16 * t2;
            const uint2 lo = __builtin_bit_cast(uint2, lds_read_tr16(base));
            const uint2 hi = __builtin_bit_cast(uint2, lds_read_tr16(base + 16 * kKtStride));
            return __builtin_bit_cast(bf16x8, make_uint4(lo.x, lo.y, hi.x, hi.y));
        };
        constexpr int kPipeV = 4;
        bf16x8 va[kPipeV][2];
#pragma unroll
        for (int d = 0; d < kPipeV; ++d) {
            va[d][0] = read_v(0, d);
            va[d][1] = read_v(1, d);
        }
#pragma unroll
        for (int t2 = 0; t2 < kT2; ++t2) {
            const int sl = t2 % kPipeV;
            acc[t2] = mfma_bf16_16x16x32(va[sl][0], pv[0], acc[t2]);
            acc[t2] = mfma_bf16_16x16x32(va[sl][1], pv[1], acc[t2]);
            if (t2 + kPipeV < kT2) {
                va[sl][0] = read_v(0, t2 + kPipeV);
                va[sl][1] = read_v(1, t2 + kPipeV);
            }
        }
    }
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
                l_tot > 0.0f ? m_tot * 0.69314718055994531f + logf(l_tot) : -INFINITY;
    } else {
        const int nwg = (Hq + 15) / 16;
        const int64_t blk = (static_cast<int64_t>(row) * nsplit + split) * nwg + wg;
        uint16_t* wo = ws_o + blk * (kT2 * 64 * 4) + lane * 4;
#pragma unroll
        for (int t2 = 0; t2 < kT2; ++t2) {
            const uint32_t lo = pack_bf16x2(acc[t2][0], acc[t2][1]);
            const uint32_t hi = pack_bf16x2(acc[t2][2], acc[t2][3]);
            __builtin_nontemporal_store(u32x2{lo, hi}, reinterpret_cast<u32x2*>(wo + t2 * 256));
        }
        if (g == 0 && h < Hq)
            *reinterpret_cast<float4*>(ws_ml + ((static_cast<int64_t>(row) * nsplit + split) * Hq + h) * 4) =
                make_float4(m_tot, lr_tot, l_tot, 0.0f);
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
constexpr int kCombineQuarters = 4;         // feature parts per 16-head group
constexpr int kCombineUnroll = 8;           // splits whose loads are in flight together
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
        const float Ls = wave_incl_sum_f(ml.z * e);
        const float Lrs = wave_incl_sum_f(ml.y * e);
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

// The same merge for at most kS splits (the batched-decode plans): the
// block and lane layout of combine_kernel, but each lane loads its head's
// (m, lr, l) triples of every split and its partials of every split at
// once and forms the weights itself, so the merge is one memory round trip
// with no LDS and no barrier. Loads past nsplit repeat the last split and
// are masked after arrival.
template <int kS>
__global__ __launch_bounds__(256) void combine_regs_kernel(int Hq, int nsplit,
                                                           const uint16_t* __restrict__ ws_o,
                                                           const float* __restrict__ ws_ml,
                                                           uint16_t* __restrict__ out,
                                                           float* __restrict__ lse) {
    const int nwg = (Hq + 15) / 16;
    const int quarter = blockIdx.x % kCombineQuarters;
    const int wg = (blockIdx.x / kCombineQuarters) % nwg;
    const int64_t row = blockIdx.x / (kCombineQuarters * nwg);
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int m = lane & 15, g = lane >> 4;
    const int h = wg * 16 + m;
    const int hc = h < Hq ? h : Hq - 1;
    const int t2a = quarter * (kT2 / kCombineQuarters) + kCombineT2 * wave;
    const uint16_t* base = ws_o + (row * nsplit * nwg + wg) * (kT2 * 64 * 4) + lane * 4;
    const int64_t sstride = static_cast<int64_t>(nwg) * kT2 * 64 * 4;
    const float* mb = ws_ml + (row * nsplit * Hq + hc) * 4;
    const int64_t ms = static_cast<int64_t>(Hq) * 4;

    float4 ml[kS];
    uint2 w[kS][kCombineT2];
#pragma unroll
    for (int sp = 0; sp < kS; ++sp) {
        const int sc = min(sp, nsplit - 1);
        ml[sp] = *reinterpret_cast<const float4*>(mb + sc * ms);
#pragma unroll
        for (int u = 0; u < kCombineT2; ++u)
            w[sp][u] = *reinterpret_cast<const uint2*>(base + sc * sstride + (t2a + u) * 256);
    }
    float M = -INFINITY;
#pragma unroll
    for (int sp = 0; sp < kS; ++sp)
        if (sp < nsplit) M = fmaxf(M, ml[sp].x);
    float L = 0.0f, Lr = 0.0f;
    float4 a[kCombineT2];
#pragma unroll
    for (int u = 0; u < kCombineT2; ++u) a[u] = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
#pragma unroll
    for (int sp = 0; sp < kS; ++sp) {
        if (sp < nsplit) {                                         // uniform
            const float e = ml[sp].x == -INFINITY ? 0.0f : exp2f(ml[sp].x - M);
            L += ml[sp].z * e;
            Lr += ml[sp].y * e;
#pragma unroll
            for (int u = 0; u < kCombineT2; ++u) {
                a[u].x += e * __uint_as_float(w[sp][u].x << 16);
                a[u].y += e * __uint_as_float(w[sp][u].x & 0xFFFF0000u);
                a[u].z += e * __uint_as_float(w[sp][u].y << 16);
                a[u].w += e * __uint_as_float(w[sp][u].y & 0xFFFF0000u);
            }
        }
    }
    if (h >= Hq) return;
    const float inv = Lr > 0.0f ? 1.0f / Lr : 0.0f;
    uint16_t* oh = out + (row * Hq + h) * kDl + 4 * g;
#pragma unroll
    for (int u = 0; u < kCombineT2; ++u) {
        const uint32_t lo = pack_bf16x2(a[u].x * inv, a[u].y * inv);
        const uint32_t hi = pack_bf16x2(a[u].z * inv, a[u].w * inv);
        *reinterpret_cast<uint2*>(oh + 16 * (t2a + u)) = make_uint2(lo, hi);
    }
    if (lse != nullptr && quarter == 0 && wave == 0 && g == 0)
        lse[row * Hq + h] = L > 0.0f ? M * 0.69314718055994531f + logf(L) : -INFINITY;
}

// Merge for the fewest rows (the grid of the 32-head builds, at most 32
// splits): one 64-thread block per (row, 16-head group, 16-feature tile t2),
// so that even one row's merge spreads over the whole chip, with no barrier
// across waves. Lane l = 16 g + m reads what lane l of each producing wave
// stored (head m, features 16 t2 + 4 g .. +3). The (m, lr) pairs of head m
// are shared out over its four lanes (lane g loads splits g, g + 4, ...), so
// each pair is read once per block instead of once per lane; the head's
// maximum and its normalisation come from two lane exchanges, and the
// per-split weights 2^(m_s - M) go through LDS to the lanes that scale the
// partials. Every load (pairs and partials) is issued before the first one
// is used: one memory round trip.
constexpr int kMergeMaxSplits = 32;

__global__ __launch_bounds__(64) void merge_few_kernel(int Hq, int nsplit,
                                                       const uint16_t* __restrict__ ws_o,
                                                       const float* __restrict__ ws_ml,
                                                       uint16_t* __restrict__ out,
                                                       float* __restrict__ lse) {
    __shared__ float wgt[16][kMergeMaxSplits + 1];
    constexpr int kPer = kMergeMaxSplits / 4;                    // splits per lane
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
    const bool want_lse = lse != nullptr && t2 == 0;

    // loads at clamped split indices, masked after arrival (a lane-dependent
    // branch around each load would make the compiler wait for every one)
    float2 mlr[kPer];
    float lsum[kPer];
#pragma unroll
    for (int k = 0; k < kPer; ++k) {
        const int sp = min(g + 4 * k, nsplit - 1);
        mlr[k] = *reinterpret_cast<const float2*>(mb + sp * ms);
        lsum[k] = mb[sp * ms + 2];
    }
#pragma unroll
    for (int k = 0; k < kPer; ++k) {
        if (g + 4 * k >= nsplit) {
            mlr[k] = make_float2(-INFINITY, 0.0f);
            lsum[k] = 0.0f;
        }
    }
    uint2 w[kMergeMaxSplits];
#pragma unroll
    for (int sp = 0; sp < kMergeMaxSplits; ++sp)
        w[sp] = *reinterpret_cast<const uint2*>(pb + min(sp, nsplit - 1) * ps);

    float M = -INFINITY;
#pragma unroll
    for (int k = 0; k < kPer; ++k) M = fmaxf(M, mlr[k].x);
    M = fmaxf(M, __shfl_xor(M, 16));
    M = fmaxf(M, __shfl_xor(M, 32));
    float Lr = 0.0f, Ls = 0.0f;
#pragma unroll
    for (int k = 0; k < kPer; ++k) {
        const float e = mlr[k].x == -INFINITY ? 0.0f : exp2f(mlr[k].x - M);
        if (g + 4 * k < nsplit) wgt[m][g + 4 * k] = e;
        Lr += mlr[k].y * e;
        Ls += lsum[k] * e;
    }
    Lr += __shfl_xor(Lr, 16);
    Lr += __shfl_xor(Lr, 32);
    __syncthreads();
    float4 a = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
#pragma unroll
    for (int sp = 0; sp < kMergeMaxSplits; ++sp) {
        if (sp < nsplit) {                      // uniform
            const float e = wgt[m][sp];
            a.x += e * __uint_as_float(w[sp].x << 16);
            a.y += e * __uint_as_float(w[sp].x & 0xFFFF0000u);
            a.z += e * __uint_as_float(w[sp].y << 16);
            a.w += e * __uint_as_float(w[sp].y & 0xFFFF0000u);
        }
    }
    if (want_lse) {
        Ls += __shfl_xor(Ls, 16);
        Ls += __shfl_xor(Ls, 32);
    }
    if (h >= Hq) return;
    const float inv = Lr > 0.0f ? 1.0f / Lr : 0.0f;
    *reinterpret_cast<uint2*>(out + (row * Hq + h) * kDl + 16 * t2 + 4 * g) =
        make_uint2(pack_bf16x2(a.x * inv, a.y * inv), pack_bf16x2(a.z * inv, a.w * inv));
    if (want_lse && g == 0)
        lse[row * Hq + h] = Ls > 0.0f ? M * 0.69314718055994531f + logf(Ls) : -INFINITY;
}

static hipError_t launch_merge_few(hipStream_t stream, int rows, int Hq, int ns,
                                   const uint16_t* ws_o, const float* ws_ml, uint16_t* out,
                                   float* lse) {
    const unsigned blocks = static_cast<unsigned>(rows) * ((Hq + 15) / 16) * kT2;
    hipLaunchKernelGGL(merge_few_kernel, dim3(blocks), dim3(64), 0, stream, Hq, ns, ws_o, ws_ml,
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
    // more than 64 KiB of dynamic LDS (set once per device)
    const hipError_t attr = set_dynamic_lds_limit(
        reinterpret_cast<const void*>(&sparse_mla_kernel<PIPE, HPB>), static_cast<int>(kMlaLdsBytes));
    if (attr != hipSuccess) return attr;
    hipLaunchKernelGGL((sparse_mla_kernel<PIPE, HPB>), grid, dim3(4 * HPB), kMlaLdsBytes, stream, S,
                       Hq, Lmax, K, sps, ns, nitems, hgroups, q, latent, lat_rs, lat_bs, rope,
                       rope_rs, rope_bs, idx, scale_log2, out, lse, ws_o, ws_ml, cmap);
    return hipGetLastError();
}

template <int HPB>
static hipError_t launch_pair(dim3 grid, hipStream_t stream, int S, int Hq, int Lmax, int K,
                              int sps, int ns, int nitems, int hgroups, const uint16_t* q,
                              const uint16_t* latent, int64_t lat_rs, int64_t lat_bs,
                              const uint16_t* rope, int64_t rope_rs, int64_t rope_bs,
                              const int32_t* idx, float scale_log2, uint16_t* out, float* lse,
                              uint16_t* ws_o, float* ws_ml, CacheMap cmap) {
    const hipError_t attr = set_dynamic_lds_limit(
        reinterpret_cast<const void*>(&sparse_mla_pair_kernel<HPB>), static_cast<int>(kPairLdsBytes));
    if (attr != hipSuccess) return attr;
    hipLaunchKernelGGL((sparse_mla_pair_kernel<HPB>), grid, dim3(4 * HPB), kPairLdsBytes, stream, S,
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
    if (few && sps <= kPairKeys) {
        // fewest blocks, splits of at most 64 slots: all of a split's keys at
        // once, 32 heads (2 waves) per block
        e = launch_pair<kHeadsPerBlockFew>(dim3(nb_few), stream, S, Hq, Lmax, K, sps, ns, nitems,
                                           hg_few, q, latent, lat_rs, lat_bs, rope, rope_rs,
                                           rope_bs, idx, scale_log2, out, lse, ws_o, ws_ml, cmap);
    } else if (nblocks <= 256 && sps <= kPairKeys) {
        // at most one block per CU, splits of at most 64 slots: the same with
        // 64 heads (4 waves) per block
        e = launch_pair<kHeadsPerBlock>(dim3(nblocks), stream, S, Hq, Lmax, K, sps, ns, nitems,
                                        hgroups, q, latent, lat_rs, lat_bs, rope, rope_rs,
                                        rope_bs, idx, scale_log2, out, lse, ws_o, ws_ml, cmap);
    } else if (few) {
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
    } else if (Hq > kHeadsPerBlock) {
        // more than one block per CU and more than 64 heads: 128-head
        // blocks, each row gathered once, the gather two tiles ahead
        const int hg_ring = (Hq + kRingHeads - 1) / kRingHeads;
        // whole groups of 8 rows' splits (the launch-to-item map above)
        const int nb_ring = ((nitems + 8 * ns - 1) / (8 * ns)) * 8 * ns * hg_ring;
        e = set_dynamic_lds_limit(reinterpret_cast<const void*>(&sparse_mla_ring_kernel),
                                  static_cast<int>(kRingLdsBytes));
        if (e != hipSuccess) return e;
        hipLaunchKernelGGL(sparse_mla_ring_kernel, dim3(nb_ring), dim3(64 * kRingWaves),
                           kRingLdsBytes, stream, S, Hq, Lmax, K, sps, ns, nitems, hg_ring, q,
                           latent, lat_rs, lat_bs, rope, rope_rs, rope_bs, idx, scale_log2, out,
                           lse, ws_o, ws_ml, cmap);
        e = hipGetLastError();
    } else {
        e = launch_mla_kernel<false, kHeadsPerBlock>(
            dim3(nblocks), stream, S, Hq, Lmax, K, sps, ns, nitems, hgroups, q, latent, lat_rs,
            lat_bs, rope, rope_rs, rope_bs, idx, scale_log2, out, lse, ws_o, ws_ml, cmap);
    }
    if (e != hipSuccess) return e;
    if (ns > 1) {
        const int64_t merge_blocks = static_cast<int64_t>(rows) * nwg * kT2;
        if (ns <= kMergeMaxSplits && merge_blocks <= 2048) {
            e = launch_merge_few(stream, rows, Hq, ns, ws_o, ws_ml, out, lse);
        } else {
            const dim3 grid(rows * nwg * kCombineQuarters);
            if (ns <= 4)
                hipLaunchKernelGGL(combine_regs_kernel<4>, grid, dim3(256), 0, stream, Hq, ns,
                                   ws_o, ws_ml, out, lse);
            else if (ns <= 8)
                hipLaunchKernelGGL(combine_regs_kernel<8>, grid, dim3(256), 0, stream, Hq, ns,
                                   ws_o, ws_ml, out, lse);
            else if (ns <= 16)
                hipLaunchKernelGGL(combine_regs_kernel<16>, grid, dim3(256), 0, stream, Hq, ns,
                                   ws_o, ws_ml, out, lse);
            else
                hipLaunchKernelGGL(combine_kernel, grid, dim3(256), 0, stream, Hq, ns, ws_o, ws_ml,
                                   out, lse);
            e = hipGetLastError();
        }
    }
    return e;
}

}  // namespace dsa
