// topk.hip -- per-query causal top-k for gfx950.
//
// Method (page "Sparse latent attention": the lightning indexer chooses up
// to 2,048 positions per query, a selection over top_2048 of the causally
// masked score; page "Rotate first features": topk(min(index_topk,
// end_pos))). Row r has n_valid = pos[r] + 1 candidates and keeps
// k_eff = min(K, n_valid) of them under (score desc, position asc), written
// in ascending position order and padded with -1.
//
// One 1024-thread block per row. Scores become order-preserving uint32
// keys (-0.0 folded into +0.0). A three-pass radix select (11, 11, 10-bit
// digits, LDS histograms) finds the k_eff-th largest key T and how many of
// the keys equal to T are needed. A compaction then walks the row in
// position order: each wave owns a contiguous run, ballots rank ties and
// selections inside the wave, two scans over the wave totals give each wave
// its earlier ties and selections, and each selected position is written
// at its rank -- ascending order falls out of the walk. Rows of up to kLdsKeys keys are cached in LDS; longer
// rows are re-read from global memory on each pass.
#include "dsa_common.h"

namespace dsa {

constexpr int kTopkThreads = 1024;
constexpr int kTopkWaves = kTopkThreads / 64;
constexpr int kLdsKeys = 16384;

// Exclusive scan of one int per thread across the block; also returns the
// block total. Uses two barriers; `wsum` holds kTopkWaves ints.
__device__ __forceinline__ int block_exclusive_scan(int v, int* wsum, int& total) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    int incl = v;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
        const int t = __shfl_up(incl, o);
        if (lane >= o) incl += t;
    }
    if (lane == 63) wsum[wave] = incl;
    __syncthreads();
    int before = 0, all = 0;
#pragma unroll
    for (int i = 0; i < kTopkWaves; ++i) {
        const int s = wsum[i];
        before += (i < wave) ? s : 0;
        all += s;
    }
    __syncthreads();
    total = all;
    return before + incl - v;
}

template <bool IN_LDS>
__device__ __forceinline__ uint32_t row_key(const uint32_t* lkeys, const float* srow, int i) {
    return IN_LDS ? lkeys[i] : float_order_key(srow[i]);
}

template <bool IN_LDS>
__global__ __launch_bounds__(kTopkThreads) void topk_kernel(
    int Lmax, int K, const float* __restrict__ scores, int64_t ld,
    const int32_t* __restrict__ pos, int32_t* __restrict__ idx, int32_t* __restrict__ count) {
    __shared__ uint32_t hist[2048];
    __shared__ int wsum[kTopkWaves];
    __shared__ uint32_t s_digit;
    __shared__ int s_above;
    extern __shared__ uint32_t lkeys[];

    const int row = blockIdx.x;
    const int tid = threadIdx.x;
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
    if (IN_LDS) {
        for (int i = tid; i < n; i += kTopkThreads) lkeys[i] = float_order_key(srow[i]);
    }

    uint32_t prefix = 0, mask = 0;
    int remaining = keff;
    const int shifts[3] = {21, 10, 0};
    const uint32_t dmasks[3] = {0x7FFu, 0x7FFu, 0x3FFu};
#pragma unroll
    for (int pass = 0; pass < 3; ++pass) {
        const int shift = shifts[pass];
        const uint32_t dmask = dmasks[pass];
        hist[tid] = 0u;
        hist[tid + 1024] = 0u;
        __syncthreads();
        for (int i = tid; i < n; i += kTopkThreads) {
            const uint32_t u = row_key<IN_LDS>(lkeys, srow, i);
            if ((u & mask) == prefix) atomicAdd(&hist[(u >> shift) & dmask], 1u);
        }
        __syncthreads();
        // thread t owns digits hi = 2047-2t and lo = 2046-2t (descending order)
        const uint32_t hi = 2047u - 2u * tid, lo = hi - 1u;
        const int chi = static_cast<int>(hist[hi]), clo = static_cast<int>(hist[lo]);
        int tot;
        const int above = block_exclusive_scan(chi + clo, wsum, tot);
        if (above < remaining && above + chi + clo >= remaining) {
            if (above + chi >= remaining) {
                s_digit = hi;
                s_above = above;
            } else {
                s_digit = lo;
                s_above = above + chi;
            }
        }
        __syncthreads();
        prefix |= s_digit << shift;
        mask |= dmask << shift;
        remaining -= s_above;
        __syncthreads();
    }
    const uint32_t T = prefix;

    // compaction in position order: wave w owns a contiguous run of the row
    // and walks it 64 positions at a time; ballots give in-wave ranks, a
    // scan over the 16 wave totals gives each wave its starting rank.
    const int lane = tid & 63, wave = tid >> 6;
    const uint64_t lt_mask = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
    const int wseg = ((n + kTopkWaves - 1) / kTopkWaves + 63) & ~63;
    const int w0 = wave * wseg;
    const int w1 = (w0 + wseg < n) ? w0 + wseg : n;
    int eq_wave = 0;
    for (int c = w0; c < w1; c += 64) {
        const int i = c + lane;
        const bool eq = i < w1 && row_key<IN_LDS>(lkeys, srow, i) == T;
        eq_wave += __popcll(__ballot(eq));
    }
    int tot;
    const int eq_before = block_exclusive_scan(lane == 0 ? eq_wave : 0, wsum, tot);
    const int eq_base0 = __shfl(eq_before, 0);
    int sel_wave = 0;
    {
        int e = eq_base0;
        for (int c = w0; c < w1; c += 64) {
            const int i = c + lane;
            const uint32_t u = i < w1 ? row_key<IN_LDS>(lkeys, srow, i) : 0u;
            const bool eq = i < w1 && u == T;
            const uint64_t eqm = __ballot(eq);
            const int rank = e + __popcll(eqm & lt_mask);
            const bool take = i < w1 && (u > T || (eq && rank < remaining));
            sel_wave += __popcll(__ballot(take));
            e += __popcll(eqm);
        }
    }
    const int sel_before = block_exclusive_scan(lane == 0 ? sel_wave : 0, wsum, tot);
    {
        int e = eq_base0;
        int o = __shfl(sel_before, 0);
        for (int c = w0; c < w1; c += 64) {
            const int i = c + lane;
            const uint32_t u = i < w1 ? row_key<IN_LDS>(lkeys, srow, i) : 0u;
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
    if (Lmax <= kLdsKeys) {
        // thread-safe one-time opt-in to more than 64 KiB of LDS (row cache + histogram)
        static const hipError_t attr = hipFuncSetAttribute(
            reinterpret_cast<const void*>(&topk_kernel<true>),
            hipFuncAttributeMaxDynamicSharedMemorySize,
            static_cast<int>(sizeof(uint32_t) * kLdsKeys));
        if (attr != hipSuccess) return attr;
        hipLaunchKernelGGL((topk_kernel<true>), dim3(rows), dim3(kTopkThreads),
                           sizeof(uint32_t) * static_cast<size_t>(Lmax), stream, Lmax, K, scores,
                           ld, pos, idx, count);
    } else {
        hipLaunchKernelGGL((topk_kernel<false>), dim3(rows), dim3(kTopkThreads), 0, stream, Lmax,
                           K, scores, ld, pos, idx, count);
    }
    return hipGetLastError();
}

}  // namespace dsa
