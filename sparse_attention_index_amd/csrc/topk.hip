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
    __shared__ int w_gt[kTopkWaves], w_eq[kTopkWaves], w_off[kTopkWaves], w_eqb[kTopkWaves];
    __shared__ uint32_t s_T;
    __shared__ int s_rem;
    extern __shared__ uint32_t dyn[];
    uint32_t* ckey = dyn;                                         // [kCandCap]
    int* cpos = reinterpret_cast<int*>(dyn + kCandCap);           // [kCandCap]
    float* lvals = reinterpret_cast<float*>(dyn + 2 * kCandCap);  // [Lmax] when IN_LDS

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

    // every walk uses the same mapping: wave w owns the contiguous run
    // [w0, w1) of the row and steps through it 64 positions at a time
    const int wseg = ((n + kTopkWaves - 1) / kTopkWaves + 63) & ~63;
    const int w0 = wave * wseg;
    const int w1 = (w0 + wseg < n) ? w0 + wseg : n;

    // walk 1: load (adding +0.0 folds -0.0 into +0.0), min/max; the loads of
    // 16 steps are issued together so their latencies overlap
    float vmin = INFINITY, vmax = -INFINITY;
    for (int cb = w0; cb < w1; cb += 16 * 64) {
        float v[16];
#pragma unroll
        for (int j = 0; j < 16; ++j) {
            const int i = cb + 64 * j + lane;
            v[j] = i < w1 ? srow[i] : 0.0f;
        }
#pragma unroll
        for (int j = 0; j < 16; ++j) {
            const int i = cb + 64 * j + lane;
            if (i < w1) {
                const float x = v[j] + 0.0f;
                if (IN_LDS) lvals[i] = x;
                vmin = fminf(vmin, x);
                vmax = fmaxf(vmax, x);
            }
        }
    }
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) {
        vmin = fminf(vmin, __shfl_xor(vmin, o));
        vmax = fmaxf(vmax, __shfl_xor(vmax, o));
    }
    if (lane == 0) {
        sh.wmin[wave] = vmin;
        sh.wmax[wave] = vmax;
        w_eq[wave] = 0;
        w_gt[wave] = 0;
    }
    if (tid == 0) sh.ccount = 0;
    sh.hist[tid] = 0u;
    sh.hist[tid + 1024] = 0u;
    __syncthreads();
    vmin = sh.wmin[0];
    vmax = sh.wmax[0];
#pragma unroll
    for (int i = 1; i < kTopkWaves; ++i) {
        vmin = fminf(vmin, sh.wmin[i]);
        vmax = fmaxf(vmax, sh.wmax[i]);
    }
    const float range = vmax - vmin;
    const float scale = static_cast<float>(kBuckets) / range;
    const bool bucketed = vmax > vmin && isfinite(range) && isfinite(scale) && scale > 0.0f;

    uint32_t T = 0;
    int remaining = 0;
    int bstar = -1;                         // bucketed rows: the threshold bucket
    if (bucketed) {
        // walk 2: bucket histogram
        for (int c = w0; c < w1; c += 64) {
            const int i = c + lane;
            if (i < w1) atomicAdd(&sh.hist[bucket_of(val(i), vmin, scale)], 1u);
        }
        __syncthreads();
        // bucket of the k_eff-th largest score (thread t owns 2047-2t, 2046-2t)
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
        bstar = static_cast<int>(sh.digit);
        const int rem = keff - sh.above;
        const int c = static_cast<int>(sh.hist[bstar]);
        if (c <= kCandCap) {
            // walk 3: per-wave count above b*, members of b* to the list
            int gt = 0;
            for (int c0 = w0; c0 < w1; c0 += 64) {
                const int i = c0 + lane;
                const float v = i < w1 ? val(i) : 0.0f;
                const int bk = i < w1 ? bucket_of(v, vmin, scale) : -1;
                gt += bk > bstar ? 1 : 0;
                const bool is_c = bk == bstar;
                const uint64_t m = __ballot(is_c);
                int base = 0;
                if (lane == 0 && m) base = atomicAdd(&sh.ccount, __popcll(m));
                base = __shfl(base, 0);
                if (is_c) {
                    ckey[base + __popcll(m & lt_mask)] = float_order_key(v);
                    cpos[base + __popcll(m & lt_mask)] = i;
                }
            }
#pragma unroll
            for (int o = 32; o >= 1; o >>= 1) gt += __shfl_xor(gt, o);
            if (lane == 0) w_gt[wave] = gt;
            __syncthreads();
            if (c <= 64) {
                // exact ranking inside one wave: (key desc, position asc)
                if (wave == 0) {
                    const uint32_t k = lane < c ? ckey[lane] : 0u;
                    const int ps = lane < c ? cpos[lane] : 0x7FFFFFFF;
                    int rank = 0, gtk = 0;
                    for (int j = 0; j < c; ++j) {
                        const uint32_t kj = __shfl(k, j);
                        const int pj = __shfl(ps, j);
                        rank += (kj > k || (kj == k && pj < ps)) ? 1 : 0;
                    }
                    const uint64_t hit = __ballot(lane < c && rank == rem - 1);
                    const int src = __ffsll(static_cast<unsigned long long>(hit)) - 1;
                    const uint32_t Tk = __shfl(k, src);
                    gtk = (lane < c && k > Tk) ? 1 : 0;
#pragma unroll
                    for (int o = 32; o >= 1; o >>= 1) gtk += __shfl_xor(gtk, o);
                    if (lane == 0) {
                        s_T = Tk;
                        s_rem = rem - gtk;
                    }
                }
                __syncthreads();
                T = s_T;
                remaining = s_rem;
            } else {
                radix_select(c, [&](int i) { return ckey[i]; }, rem, sh, T, remaining);
            }
            // per-wave keys above T / equal to T inside bucket b*
            for (int i = tid; i < c; i += kTopkThreads) {
                const int wv = cpos[i] / wseg;
                if (ckey[i] > T) atomicAdd(&w_gt[wv], 1);
                else if (ckey[i] == T) atomicAdd(&w_eq[wv], 1);
            }
            __syncthreads();
        } else {
            bstar = -1;                     // overfull bucket: plain compaction below
        }
    }
    if (bstar < 0) {
        if (!bucketed) {
            if (!(vmax > vmin)) {           // all scores equal
                T = float_order_key(vmax);
                remaining = keff;
            } else {
                radix_select(n, key, keff, sh, T, remaining);
            }
        } else {
            radix_select(n, key, keff, sh, T, remaining);
        }
        // counting walk: per-wave keys above T / equal to T
        int gt = 0, eq = 0;
        for (int c0 = w0; c0 < w1; c0 += 64) {
            const int i = c0 + lane;
            const uint32_t u = i < w1 ? key(i) : 0u;
            gt += (i < w1 && u > T) ? 1 : 0;
            eq += (i < w1 && u == T) ? 1 : 0;
        }
#pragma unroll
        for (int o = 32; o >= 1; o >>= 1) {
            gt += __shfl_xor(gt, o);
            eq += __shfl_xor(eq, o);
        }
        if (lane == 0) {
            w_gt[wave] = gt;
            w_eq[wave] = eq;
        }
        __syncthreads();
    }
    // output start of every wave's run and its earlier ties
    if (tid == 0) {
        int o = 0, eb = 0;
        for (int w = 0; w < kTopkWaves; ++w) {
            w_off[w] = o;
            w_eqb[w] = eb;
            o += w_gt[w] + min(max(remaining - eb, 0), w_eq[w]);
            eb += w_eq[w];
        }
    }
    __syncthreads();
    // walk 4: write the taken positions in order
    {
        int e = w_eqb[wave];
        int o = w_off[wave];
        for (int c0 = w0; c0 < w1; c0 += 64) {
            const int i = c0 + lane;
            bool take = false, eq = false;
            if (i < w1) {
                if (bstar >= 0) {
                    const float v = val(i);
                    const int bk = bucket_of(v, vmin, scale);
                    if (bk > bstar) {
                        take = true;
                    } else if (bk == bstar) {
                        const uint32_t u = float_order_key(v);
                        take = u > T;
                        eq = u == T;
                    }
                } else {
                    const uint32_t u = key(i);
                    take = u > T;
                    eq = u == T;
                }
            }
            const uint64_t eqm = __ballot(eq);
            if (eq) take = e + __popcll(eqm & lt_mask) < remaining;
            e += __popcll(eqm);
            const uint64_t tm = __ballot(take);
            const int slot = o + __popcll(tm & lt_mask);
            if (take && slot < keff) out[slot] = i;
            o += __popcll(tm);
        }
    }
    for (int i = keff + tid; i < K; i += kTopkThreads) out[i] = -1;
}

// ---------------------------------------------------------------------------
// Multi-block path for long rows: chunks of kChunk scores, one 256-thread
// block per (chunk, row), three launches:
//   T1  per-chunk LDS histogram of the top 11 bits of the order key, added to
//       the row's global histogram; the last chunk to finish (atomic counter
//       after a fence) finds the bucket b* holding the k_eff-th largest key
//       and the count above it.
//   T2  per chunk: count of keys in buckets above b*; keys of bucket b* are
//       appended (key, position) to the row's candidate list. The last chunk
//       selects exactly among the candidates (radix select; a whole-row radix
//       select when the list overflowed), derives for every chunk how many
//       of its keys are taken and where its output run starts, and clears the
//       row's histogram and counters for the next call.
//   T3  per chunk: ordered compaction of its taken positions into idx.
// Workspace per row (zero on the first call, left zero by every call):
//   hist[2048] | state[8] | per-chunk gt/eq/off/eqb | candidates[kCandRow] x2
// ---------------------------------------------------------------------------
constexpr int kChunk = 2048;
constexpr int kMbThreads = 256;
constexpr int kMbPer = kChunk / kMbThreads;     // 8 scores per thread
constexpr int kCandRow = 8192;                  // candidate list capacity per row
constexpr int kMbMinLmax = kLdsKeys + 1;       // rows longer than the LDS row cache
constexpr int kCandLds = 4096;                  // candidates staged in LDS by the last chunk
constexpr int kMaxChunks = 1024;                // chunks per row (rows up to 2M keys)

struct MbLayout {
    int nch;                 // chunks per row (Lmax / kChunk rounded up)
    size_t row_bytes;        // bytes per row
    size_t off_state, off_gt, off_eq, off_off, off_eqb, off_ckey, off_cpos;
};

__host__ __device__ inline MbLayout mb_layout(int Lmax) {
    MbLayout L;
    L.nch = (Lmax + kChunk - 1) / kChunk;
    size_t o = 2048 * 4;
    L.off_state = o; o += 8 * 4;
    L.off_gt = o; o += static_cast<size_t>(L.nch) * 4;
    L.off_eq = o; o += static_cast<size_t>(L.nch) * 4;
    L.off_off = o; o += static_cast<size_t>(L.nch) * 4;
    L.off_eqb = o; o += static_cast<size_t>(L.nch) * 4;
    o = (o + 15) & ~static_cast<size_t>(15);
    L.off_ckey = o; o += static_cast<size_t>(kCandRow) * 4;
    L.off_cpos = o; o += static_cast<size_t>(kCandRow) * 4;
    L.row_bytes = (o + 255) & ~static_cast<size_t>(255);
    return L;
}

enum { ST_DONE1 = 0, ST_DONE2, ST_NCAND, ST_BSTAR, ST_ABOVE, ST_T, ST_REM };

struct MbRow {
    uint32_t* hist; int* st; int* gt; int* eq; int* off; int* eqb; uint32_t* ckey; int* cpos;
};

__device__ __forceinline__ MbRow mb_row(unsigned char* ws, const MbLayout& L, int row) {
    unsigned char* base = ws + static_cast<size_t>(row) * L.row_bytes;
    MbRow R;
    R.hist = reinterpret_cast<uint32_t*>(base);
    R.st = reinterpret_cast<int*>(base + L.off_state);
    R.gt = reinterpret_cast<int*>(base + L.off_gt);
    R.eq = reinterpret_cast<int*>(base + L.off_eq);
    R.off = reinterpret_cast<int*>(base + L.off_off);
    R.eqb = reinterpret_cast<int*>(base + L.off_eqb);
    R.ckey = reinterpret_cast<uint32_t*>(base + L.off_ckey);
    R.cpos = reinterpret_cast<int*>(base + L.off_cpos);
    return R;
}

// exclusive scan across a 256-thread block; `ws` holds 4 ints
__device__ __forceinline__ int block256_scan(int v, int* ws, int& total) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    int incl = v;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
        const int t = __shfl_up(incl, o);
        if (lane >= o) incl += t;
    }
    if (lane == 63) ws[wave] = incl;
    __syncthreads();
    int before = 0;
    total = 0;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        before += i < wave ? ws[i] : 0;
        total += ws[i];
    }
    __syncthreads();
    return before + incl - v;
}

__device__ __forceinline__ int row_nvalid(const int32_t* pos, int row, int Lmax) {
    const int p = pos[row];
    return (p >= 0 && p < Lmax) ? p + 1 : 0;
}

// Bucket b and count above it from a 2048-bin histogram (descending scan),
// for the want-th largest (1 <= want <= total count).
__device__ void find_bucket(const uint32_t* hist, int want, int* ws, int* s_b, int* s_above) {
    const int tid = threadIdx.x;
    int c[8];
    int sum = 0;
#pragma unroll
    for (int j = 0; j < 8; ++j) {             // thread t owns digits 2047-8t-j
        c[j] = static_cast<int>(hist[2047 - 8 * tid - j]);
        sum += c[j];
    }
    int tot;
    int above = block256_scan(sum, ws, tot);
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        if (above < want && above + c[j] >= want) {
            *s_b = 2047 - 8 * tid - j;
            *s_above = above;
        }
        above += c[j];
    }
    __syncthreads();
}

__global__ __launch_bounds__(kMbThreads) void topk_mb_hist(int Lmax, int K,
                                                           const float* __restrict__ scores,
                                                           int64_t ld, const int32_t* __restrict__ pos,
                                                           unsigned char* __restrict__ ws) {
    __shared__ uint32_t lh[2048];
    __shared__ int wsc[4];
    __shared__ int s_last, s_b, s_above;
    const int row = blockIdx.y, ch = blockIdx.x, tid = threadIdx.x;
    const int n = row_nvalid(pos, row, Lmax);
    const int keff = n < K ? n : K;
    if (keff == n || ch * kChunk >= n) return;
    const MbLayout L = mb_layout(Lmax);
    const MbRow R = mb_row(ws, L, row);
    const int nch = (n + kChunk - 1) / kChunk;
    for (int i = tid; i < 2048; i += kMbThreads) lh[i] = 0u;
    __syncthreads();
    const float* src = scores + static_cast<int64_t>(row) * ld + ch * kChunk;
    const int lim = min(kChunk, n - ch * kChunk);
#pragma unroll
    for (int j = 0; j < kMbPer; ++j) {
        const int i = tid + j * kMbThreads;
        if (i < lim) atomicAdd(&lh[float_order_key(src[i]) >> 21], 1u);
    }
    __syncthreads();
    for (int i = tid; i < 2048; i += kMbThreads)
        if (lh[i]) atomicAdd(&R.hist[i], lh[i]);
    __threadfence();
    __syncthreads();
    if (tid == 0) s_last = atomicAdd(&R.st[ST_DONE1], 1) == nch - 1;
    __syncthreads();
    if (!s_last) return;
    __threadfence();
    find_bucket(R.hist, keff, wsc, &s_b, &s_above);
    if (tid == 0) {
        R.st[ST_BSTAR] = s_b;
        R.st[ST_ABOVE] = s_above;
    }
}

__global__ __launch_bounds__(kMbThreads) void topk_mb_cand(int Lmax, int K,
                                                           const float* __restrict__ scores,
                                                           int64_t ld, const int32_t* __restrict__ pos,
                                                           unsigned char* __restrict__ ws) {
    __shared__ int wsc[4];
    __shared__ int s_last;
    __shared__ uint32_t hist[2048];
    __shared__ int s_b, s_above;
    __shared__ uint32_t ckey_l[kCandLds];
    __shared__ uint8_t cch_l[kCandLds];
    const int row = blockIdx.y, ch = blockIdx.x, tid = threadIdx.x;
    const int lane = tid & 63;
    const uint64_t lt_mask = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
    const int n = row_nvalid(pos, row, Lmax);
    const int keff = n < K ? n : K;
    if (keff == n || ch * kChunk >= n) return;
    const MbLayout L = mb_layout(Lmax);
    const MbRow R = mb_row(ws, L, row);
    const int nch = (n + kChunk - 1) / kChunk;
    const uint32_t bstar = static_cast<uint32_t>(R.st[ST_BSTAR]);
    const float* srow = scores + static_cast<int64_t>(row) * ld;
    const float* src = srow + ch * kChunk;
    const int lim = min(kChunk, n - ch * kChunk);
    int gt = 0;
#pragma unroll
    for (int j = 0; j < kMbPer; ++j) {
        const int i = tid + j * kMbThreads;
        const uint32_t u = i < lim ? float_order_key(src[i]) : 0u;
        const uint32_t d = u >> 21;
        gt += (i < lim && d > bstar) ? 1 : 0;
        const bool c = i < lim && d == bstar;
        const uint64_t m = __ballot(c);
        int base = 0;
        if (lane == 0 && m) base = atomicAdd(&R.st[ST_NCAND], __popcll(m));
        base = __shfl(base, 0);
        const int slot = base + __popcll(m & lt_mask);
        if (c && slot < kCandRow) {
            R.ckey[slot] = u;
            R.cpos[slot] = ch * kChunk + i;
        }
    }
    int tot;
    block256_scan(gt, wsc, tot);
    if (tid == 0) R.gt[ch] = tot;
    __threadfence();
    __syncthreads();
    if (tid == 0) s_last = atomicAdd(&R.st[ST_DONE2], 1) == nch - 1;
    __syncthreads();
    if (!s_last) return;
    __threadfence();

    // ---- last chunk of the row: exact threshold among the candidates ----
    const int ncand = R.st[ST_NCAND];
    const int rem = keff - R.st[ST_ABOVE];
    uint32_t prefix = 0, mask = 0;
    int remaining = rem;
    const bool from_list = ncand <= kCandRow;
    const int nsrc = from_list ? ncand : n;
    if (!from_list) remaining = keff;              // overflow: whole-row select
    const bool in_lds = from_list && ncand <= kCandLds;
    if (in_lds)
        for (int i = tid; i < ncand; i += kMbThreads) {
            ckey_l[i] = R.ckey[i];
            cch_l[i] = static_cast<uint8_t>(R.cpos[i] / kChunk);
        }
    auto getk = [&](int i) -> uint32_t {
        return in_lds ? ckey_l[i] : (from_list ? R.ckey[i] : float_order_key(srow[i]));
    };
    auto getc = [&](int i) -> int {
        return in_lds ? static_cast<int>(cch_l[i]) : (from_list ? R.cpos[i] / kChunk : i / kChunk);
    };
    const int shifts[3] = {21, 10, 0};
    const uint32_t dmasks[3] = {0x7FFu, 0x7FFu, 0x3FFu};
    if (from_list) {                               // the list shares bucket b*'s 11 bits
        prefix = static_cast<uint32_t>(R.st[ST_BSTAR]) << 21;
        mask = 0x7FFu << 21;
    }
    for (int pass = from_list ? 1 : 0; pass < 3; ++pass) {
        const int shift = shifts[pass];
        const uint32_t dmask = dmasks[pass];
        for (int i = tid; i < 2048; i += kMbThreads) hist[i] = 0u;
        __syncthreads();
        for (int i = tid; i < nsrc; i += kMbThreads) {
            const uint32_t u = getk(i);
            if ((u & mask) == prefix) atomicAdd(&hist[(u >> shift) & dmask], 1u);
        }
        __syncthreads();
        find_bucket(hist, remaining, wsc, &s_b, &s_above);
        prefix |= static_cast<uint32_t>(s_b) << shift;
        mask |= dmask << shift;
        remaining -= s_above;
        __syncthreads();
    }
    const uint32_t T = prefix;
    // per chunk: taken = (keys above T) + (keys equal to T, lowest positions
    // first); counted in LDS from the candidates (every key >= T outside the
    // buckets above b* is one) or, after an overflow, from the whole row
    int* c_gt = reinterpret_cast<int*>(hist);          // hist is free now
    int* c_eq = c_gt + kMaxChunks;
    for (int c2 = tid; c2 < 2 * kMaxChunks; c2 += kMbThreads) c_gt[c2] = 0;
    __syncthreads();
    for (int i = tid; i < nsrc; i += kMbThreads) {
        const uint32_t u = getk(i);
        if (u > T) atomicAdd(&c_gt[getc(i)], 1);
        else if (u == T) atomicAdd(&c_eq[getc(i)], 1);
    }
    __syncthreads();
    if (tid == 0) {
        int o = 0, eb = 0;
        for (int c2 = 0; c2 < nch; ++c2) {
            const int gtc = (from_list ? R.gt[c2] : 0) + c_gt[c2];
            const int eqc = c_eq[c2];
            const int take_eq = min(max(remaining - eb, 0), eqc);
            R.eqb[c2] = eb;                    // keys equal to T in earlier chunks
            R.off[c2] = o;                     // output start of the chunk
            o += gtc + take_eq;
            eb += eqc;
        }
        R.st[ST_T] = static_cast<int>(T);
        R.st[ST_REM] = remaining;
        R.st[ST_DONE1] = 0;
        R.st[ST_DONE2] = 0;
        R.st[ST_NCAND] = 0;
    }
    for (int i = tid; i < 2048; i += kMbThreads) R.hist[i] = 0u;
}

__global__ __launch_bounds__(kMbThreads) void topk_mb_write(int Lmax, int K,
                                                            const float* __restrict__ scores,
                                                            int64_t ld, const int32_t* __restrict__ pos,
                                                            unsigned char* __restrict__ ws,
                                                            int32_t* __restrict__ idx,
                                                            int32_t* __restrict__ count) {
    __shared__ int wsc[4];
    const int row = blockIdx.y, ch = blockIdx.x, tid = threadIdx.x;
    const int lane = tid & 63;
    const uint64_t lt_mask = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
    const int n = row_nvalid(pos, row, Lmax);
    const int keff = n < K ? n : K;
    int32_t* out = idx + static_cast<int64_t>(row) * K;
    if (ch == 0) {
        for (int i = keff + tid; i < K; i += kMbThreads) out[i] = -1;
        if (count != nullptr && tid == 0) count[row] = keff;
    }
    if (ch * kChunk >= n) return;
    const int lim = min(kChunk, n - ch * kChunk);
    if (keff == n) {                               // every causal key is taken
        for (int i = tid; i < lim; i += kMbThreads) out[ch * kChunk + i] = ch * kChunk + i;
        return;
    }
    const MbLayout L = mb_layout(Lmax);
    const MbRow R = mb_row(ws, L, row);
    const uint32_t T = static_cast<uint32_t>(R.st[ST_T]);
    const int remaining = R.st[ST_REM];
    const float* src = scores + static_cast<int64_t>(row) * ld + ch * kChunk;
    // thread t owns scores [8t, 8t+8) of the chunk (position order)
    uint32_t u[kMbPer];
    int eqn = 0, seln = 0;
#pragma unroll
    for (int j = 0; j < kMbPer; ++j) {
        const int i = tid * kMbPer + j;
        u[j] = i < lim ? float_order_key(src[i]) : 0u;
        eqn += (i < lim && u[j] == T) ? 1 : 0;
    }
    int tot;
    int e = R.eqb[ch] + block256_scan(eqn, wsc, tot);
#pragma unroll
    for (int j = 0; j < kMbPer; ++j) {
        const int i = tid * kMbPer + j;
        if (i < lim) {
            if (u[j] > T) ++seln;
            else if (u[j] == T) { if (e < remaining) ++seln; ++e; }
        }
    }
    int o = R.off[ch] + block256_scan(seln, wsc, tot);
    e = R.eqb[ch] + block256_scan(eqn, wsc, tot);
#pragma unroll
    for (int j = 0; j < kMbPer; ++j) {
        const int i = tid * kMbPer + j;
        if (i < lim) {
            bool take = false;
            if (u[j] > T) take = true;
            else if (u[j] == T) { take = e < remaining; ++e; }
            if (take && o < keff) out[o++] = ch * kChunk + i;
        }
    }
    (void)lt_mask;
}

size_t topk_workspace_bytes(int rows, int Lmax) {
    if (Lmax < kMbMinLmax) return 0;
    return static_cast<size_t>(rows) * mb_layout(Lmax).row_bytes;
}

hipError_t launch_topk(int rows, int Lmax, int K, const float* scores, int64_t ld,
                       const int32_t* pos, int32_t* idx, int32_t* count, void* workspace,
                       hipStream_t stream) {
    if (Lmax >= kMbMinLmax) {
        unsigned char* ws = static_cast<unsigned char*>(workspace);
        const dim3 grid((Lmax + kChunk - 1) / kChunk, rows);
        hipLaunchKernelGGL(topk_mb_hist, grid, dim3(kMbThreads), 0, stream, Lmax, K, scores, ld,
                           pos, ws);
        hipLaunchKernelGGL(topk_mb_cand, grid, dim3(kMbThreads), 0, stream, Lmax, K, scores, ld,
                           pos, ws);
        hipLaunchKernelGGL(topk_mb_write, grid, dim3(kMbThreads), 0, stream, Lmax, K, scores, ld,
                           pos, ws, idx, count);
        return hipGetLastError();
    }
    const size_t bytes = sizeof(uint32_t) * (2 * kCandCap + static_cast<size_t>(Lmax));
    // thread-safe one-time opt-in to more than 64 KiB of LDS
    static const hipError_t attr = hipFuncSetAttribute(
        reinterpret_cast<const void*>(&topk_kernel<true>),
        hipFuncAttributeMaxDynamicSharedMemorySize,
        static_cast<int>(sizeof(uint32_t) * (2 * kCandCap + kLdsKeys)));
    if (attr != hipSuccess) return attr;
    hipLaunchKernelGGL((topk_kernel<true>), dim3(rows), dim3(kTopkThreads), bytes, stream, Lmax, K,
                       scores, ld, pos, idx, count);
    return hipGetLastError();
}

}  // namespace dsa
