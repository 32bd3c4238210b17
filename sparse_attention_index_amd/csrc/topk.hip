// topk.hip -- per-query causal top-k for gfx950.
//
// Method (page "Sparse latent attention": the lightning indexer chooses up
// to 2,048 positions per query, a selection over top_2048 of the causally
// masked score; page "Rotate first features": topk(min(index_topk,
// end_pos))). Row r has n_valid = pos[r] + 1 candidates and keeps
// k_eff = min(K, n_valid) of them under (score desc, position asc), written
// in ascending position order and padded with -1.
//
// One 1024-thread block per row; rows of up to kLdsKeys scores are cached
// in LDS, longer rows are re-read from global memory by each walk.
//  1. min/max of the row.
//  2. Bucket pass: bucket(v) = floor((v - min) * 2048 / (max - min)), a
//     monotone non-decreasing map, so every score in a higher bucket is
//     larger than every score in a lower one. Score rows are smooth, so the
//     LDS histogram sees little atomic contention (the bits of a float's
//     exponent, by contrast, pile most scores into a few bins).
//  3. The bucket holding the k_eff-th largest score is found by a block
//     scan; its members (few) are collected and an exact three-pass radix
//     select (11/11/10-bit digits of the order-preserving uint32 key, -0.0
//     folded into +0.0) over them gives the threshold key T and how many
//     keys equal to T are taken. Degenerate rows (all equal, infinities, an
//     overfull bucket) run the radix select over the whole row instead.
//  4. Compaction in position order: each wave owns a contiguous run and
//     ranks ties and selections with ballots; two scans over the wave totals
//     give each wave its starting ranks. Ascending output falls out.
#include "dsa_common.h"

namespace dsa {

constexpr int kTopkThreads = 1024;
constexpr int kTopkWaves = kTopkThreads / 64;
constexpr int kLdsKeys = 16384;
constexpr int kBuckets = 2048;
constexpr int kCandCap = 4096;

struct TopkShared {
    uint32_t hist[2048];
    int wsum[kTopkWaves];
    float wmin[kTopkWaves];
    float wmax[kTopkWaves];
    uint32_t digit;
    int above;
    int ccount;
};

// Exclusive scan of one int per thread across the block (two barriers).
__device__ __forceinline__ int block_exclusive_scan(int v, int* wsum) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    int incl = v;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
        const int t = __shfl_up(incl, o);
        if (lane >= o) incl += t;
    }
    if (lane == 63) wsum[wave] = incl;
    __syncthreads();
    int before = 0;
#pragma unroll
    for (int i = 0; i < kTopkWaves; ++i) before += (i < wave) ? wsum[i] : 0;
    __syncthreads();
    return before + incl - v;
}

// Largest `want`-th key among n keys get(i): returns T and how many of the
// keys equal to T belong to the top `want` (1 <= want <= n).
template <typename Get>
__device__ void radix_select(int n, Get get, int want, TopkShared& sh, uint32_t& T,
                             int& remaining) {
    const int tid = threadIdx.x;
    uint32_t prefix = 0, mask = 0;
    remaining = want;
    const int shifts[3] = {21, 10, 0};
    const uint32_t dmasks[3] = {0x7FFu, 0x7FFu, 0x3FFu};
#pragma unroll
    for (int pass = 0; pass < 3; ++pass) {
        const int shift = shifts[pass];
        const uint32_t dmask = dmasks[pass];
        sh.hist[tid] = 0u;
        sh.hist[tid + 1024] = 0u;
        __syncthreads();
        for (int i = tid; i < n; i += kTopkThreads) {
            const uint32_t u = get(i);
            if ((u & mask) == prefix) atomicAdd(&sh.hist[(u >> shift) & dmask], 1u);
        }
        __syncthreads();
        // thread t owns digits hi = 2047-2t and lo = 2046-2t (descending)
        const uint32_t hi = 2047u - 2u * tid, lo = hi - 1u;
        const int chi = static_cast<int>(sh.hist[hi]), clo = static_cast<int>(sh.hist[lo]);
        const int above = block_exclusive_scan(chi + clo, sh.wsum);
        if (above < remaining && above + chi + clo >= remaining) {
            if (above + chi >= remaining) {
                sh.digit = hi;
                sh.above = above;
            } else {
                sh.digit = lo;
                sh.above = above + chi;
            }
        }
        __syncthreads();
        prefix |= sh.digit << shift;
        mask |= dmask << shift;
        remaining -= sh.above;
        __syncthreads();
    }
    T = prefix;
}

__device__ __forceinline__ int bucket_of(float v, float vmin, float scale) {
    const float f = (v - vmin) * scale;
    const int b = static_cast<int>(f);
    return b < kBuckets - 1 ? b : kBuckets - 1;
}

template <bool IN_LDS>
__global__ __launch_bounds__(kTopkThreads) void topk_kernel(
    int Lmax, int K, const float* __restrict__ scores, int64_t ld,
    const int32_t* __restrict__ pos, int32_t* __restrict__ idx, int32_t* __restrict__ count) {
    __shared__ TopkShared sh;
    extern __shared__ uint32_t dyn[];
    uint32_t* cand = dyn;                                        // [kCandCap]
    float* lvals = reinterpret_cast<float*>(dyn + kCandCap);     // [Lmax] when IN_LDS

    const int row = blockIdx.x;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const uint64_t lt_mask = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
    const int p = pos[row];
    const int n = (p >= 0 && p < Lmax) ? p + 1 : 0;
    const int keff = n < K ? n : K;
    int32_t* out = idx + static_cast<int64_t>(row) * K;
    const float* srow = scores + static_cast<int64_t>(row) * ld;
    if (count != nullptr && tid == 0) count[row] = keff;

    if (keff == n) {                        // everything causal is selected
        for (int i = tid; i < K; i += kTopkThreads) out[i] = i < n ? i : -1;
        return;
    }
    auto val = [&](int i) -> float { return IN_LDS ? lvals[i] : srow[i] + 0.0f; };
    auto key = [&](int i) -> uint32_t { return float_order_key(val(i)); };

    // 1. load (adding +0.0 folds -0.0 into +0.0) and min/max
    float vmin = INFINITY, vmax = -INFINITY;
    for (int i = tid; i < n; i += kTopkThreads) {
        const float v = srow[i] + 0.0f;
        if (IN_LDS) lvals[i] = v;
        vmin = fminf(vmin, v);
        vmax = fmaxf(vmax, v);
    }
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) {
        vmin = fminf(vmin, __shfl_xor(vmin, o));
        vmax = fmaxf(vmax, __shfl_xor(vmax, o));
    }
    if (lane == 0) {
        sh.wmin[wave] = vmin;
        sh.wmax[wave] = vmax;
    }
    if (tid == 0) sh.ccount = 0;
    __syncthreads();
    vmin = sh.wmin[0];
    vmax = sh.wmax[0];
#pragma unroll
    for (int i = 1; i < kTopkWaves; ++i) {
        vmin = fminf(vmin, sh.wmin[i]);
        vmax = fmaxf(vmax, sh.wmax[i]);
    }

    uint32_t T = 0;
    int remaining = 0;
    bool done = false;
    if (!(vmax > vmin)) {                   // all scores equal
        T = float_order_key(vmax);
        remaining = keff;
        done = true;
    } else {
        const float range = vmax - vmin;
        const float scale = static_cast<float>(kBuckets) / range;
        if (isfinite(range) && isfinite(scale) && scale > 0.0f) {
            // 2. bucket histogram
            sh.hist[tid] = 0u;
            sh.hist[tid + 1024] = 0u;
            __syncthreads();
            for (int i = tid; i < n; i += kTopkThreads)
                atomicAdd(&sh.hist[bucket_of(val(i), vmin, scale)], 1u);
            __syncthreads();
            // 3. bucket of the k_eff-th largest score
            const uint32_t hi = 2047u - 2u * tid, lo = hi - 1u;
            const int chi = static_cast<int>(sh.hist[hi]), clo = static_cast<int>(sh.hist[lo]);
            const int above = block_exclusive_scan(chi + clo, sh.wsum);
            if (above < keff && above + chi + clo >= keff) {
                if (above + chi >= keff) {
                    sh.digit = hi;
                    sh.above = above;
                } else {
                    sh.digit = lo;
                    sh.above = above + chi;
                }
            }
            __syncthreads();
            const int bstar = static_cast<int>(sh.digit);
            const int rem = keff - sh.above;
            const int c = static_cast<int>(sh.hist[bstar]);
            __syncthreads();
            if (c <= kCandCap) {
                for (int i0 = 0; i0 < n; i0 += kTopkThreads) {
                    const int i = i0 + tid;
                    const float v = i < n ? val(i) : 0.0f;
                    const bool is_c = i < n && bucket_of(v, vmin, scale) == bstar;
                    const uint64_t m = __ballot(is_c);
                    int base = 0;
                    if (lane == 0 && m) base = atomicAdd(&sh.ccount, __popcll(m));
                    base = __shfl(base, 0);
                    if (is_c) cand[base + __popcll(m & lt_mask)] = float_order_key(v);
                }
                __syncthreads();
                radix_select(c, [&](int i) { return cand[i]; }, rem, sh, T, remaining);
                done = true;
            }
        }
    }
    if (!done) radix_select(n, key, keff, sh, T, remaining);

    // 4. compaction in position order
    const int wseg = ((n + kTopkWaves - 1) / kTopkWaves + 63) & ~63;
    const int w0 = wave * wseg;
    const int w1 = (w0 + wseg < n) ? w0 + wseg : n;
    int eq_wave = 0;
    for (int c = w0; c < w1; c += 64) {
        const int i = c + lane;
        const bool eq = i < w1 && key(i) == T;
        eq_wave += __popcll(__ballot(eq));
    }
    const int eq_base0 = __shfl(block_exclusive_scan(lane == 0 ? eq_wave : 0, sh.wsum), 0);
    int sel_wave = 0;
    {
        int e = eq_base0;
        for (int c = w0; c < w1; c += 64) {
            const int i = c + lane;
            const uint32_t u = i < w1 ? key(i) : 0u;
            const bool eq = i < w1 && u == T;
            const uint64_t eqm = __ballot(eq);
            const int rank = e + __popcll(eqm & lt_mask);
            const bool take = i < w1 && (u > T || (eq && rank < remaining));
            sel_wave += __popcll(__ballot(take));
            e += __popcll(eqm);
        }
    }
    int o = __shfl(block_exclusive_scan(lane == 0 ? sel_wave : 0, sh.wsum), 0);
    {
        int e = eq_base0;
        for (int c = w0; c < w1; c += 64) {
            const int i = c + lane;
            const uint32_t u = i < w1 ? key(i) : 0u;
            const bool eq = i < w1 && u == T;
            const uint64_t eqm = __ballot(eq);
            const int rank = e + __popcll(eqm & lt_mask);
            const bool take = i < w1 && (u > T || (eq && rank < remaining));
            const uint64_t tm = __ballot(take);
            const int slot = o + __popcll(tm & lt_mask);
            if (take && slot < keff) out[slot] = i;
            o += __popcll(tm);
            e += __popcll(eqm);
        }
    }
    for (int i = keff + tid; i < K; i += kTopkThreads) out[i] = -1;
}

hipError_t launch_topk(int rows, int Lmax, int K, const float* scores, int64_t ld,
                       const int32_t* pos, int32_t* idx, int32_t* count, hipStream_t stream) {
    const size_t cand_bytes = sizeof(uint32_t) * kCandCap;
    if (Lmax <= kLdsKeys) {
        const size_t bytes = cand_bytes + sizeof(float) * static_cast<size_t>(Lmax);
        // thread-safe one-time opt-in to more than 64 KiB of LDS
        static const hipError_t attr = hipFuncSetAttribute(
            reinterpret_cast<const void*>(&topk_kernel<true>),
            hipFuncAttributeMaxDynamicSharedMemorySize,
            static_cast<int>(cand_bytes + sizeof(float) * kLdsKeys));
        if (attr != hipSuccess) return attr;
        hipLaunchKernelGGL((topk_kernel<true>), dim3(rows), dim3(kTopkThreads), bytes, stream,
                           Lmax, K, scores, ld, pos, idx, count);
    } else {
        hipLaunchKernelGGL((topk_kernel<false>), dim3(rows), dim3(kTopkThreads), cand_bytes,
                           stream, Lmax, K, scores, ld, pos, idx, count);
    }
    return hipGetLastError();
}

}  // namespace dsa
