// topk.hip -- per-query causal top-k for gfx950.
//
// Method (page "Sparse latent attention": the lightning indexer chooses up
// to 2,048 positions per query, a selection over top_2048 of the causally
// masked score; page "Rotate first features": topk(min(index_topk,
// end_pos))). Row r has n_valid = pos[r] + 1 candidates and keeps
// k_eff = min(K, n_valid) of them under (score desc, position asc), written
// in ascending position order and padded with -1.
//
// Rows of up to 16,384 scores: one block per row, the row held in
// registers (16 scores per thread; wave w owns the contiguous run
// [1024 w, 1024 w + 1024), lane l item j at 1024 w + 64 j + l).
//  1. Load (adding +0.0 folds -0.0 into +0.0) and the row's min/max.
//  2. Bucket pass: bucket(v) = floor((v - min) * 2048 / (max - min)), a
//     monotone non-decreasing map, so every score in a higher bucket is
//     larger than every score in a lower one. An LDS histogram, scanned by
//     one wave with DPP prefix sums, gives the bucket b* holding the
//     k_eff-th largest score and the count G above it.
//  3. Threshold key T (the k_eff-th largest order key, counted with
//     multiplicity): when b* holds at most 64 scores one wave ranks them;
//     otherwise an exact three-pass radix select (11/11/10-bit digits of the
//     order key) runs over the scores of b*. Rows whose min/max give no
//     usable bucket map (all equal, infinities) run it over the whole row.
//     Every key above T is taken, and of the keys equal to T the ones with
//     the lowest positions, as many as k_eff leaves.
//  4. Ordered compaction: per-wave counts of keys above / equal to T (taken
//     during step 3 when one wave ranked b*, else by a ballot pass) give each
//     wave its output start, and each wave writes its taken positions in
//     order. Ascending output falls out of the position order of the runs.
#include "dsa_common.h"

namespace dsa {

constexpr int kRegItems = 16;                           // scores per thread
constexpr int kRegMaxThreads = 1024;
constexpr int kRegMaxWaves = kRegMaxThreads / kWave;
constexpr int kLdsKeys = kRegItems * kRegMaxThreads;    // longest row of the one-block path
constexpr int kBuckets = 2048;
constexpr int kRankCap = kWave;                         // bucket sizes ranked by one wave

struct alignas(16) RegShared {
    uint32_t hist[kBuckets];
    uint32_t cand[kRankCap];
    int cand_wave[kRankCap];
    int wa[kRegMaxWaves];                   // per wave: keys above T
    int wb[kRegMaxWaves];                   // per wave: keys equal to T
    float wmin[kRegMaxWaves];
    float wmax[kRegMaxWaves];
    uint32_t digit;
    int above;
    int ccount;
    uint32_t T;
    int gtc;
};

// Over hist[0..nbins) (nbins = 1024 or 2048): the bin holding the want-th
// largest entry, counting from the top bin down, and how many entries lie in
// higher bins, written to sh.digit / sh.above by wave 0 alone
// (1 <= want <= total). Lane l sums the bins [nbins - nb (l+1), nbins - nb l);
// a DPP prefix sum over the lanes finds the lane whose range holds the
// want-th entry, and a second one over that range's bins (one per lane, top
// first) finds the bin. The caller synchronises the block afterwards.
template <int NBINS>
__device__ __forceinline__ void find_digit_wave0(RegShared& sh, int want) {
    constexpr int nb = NBINS / kWave;
    const int lane = threadIdx.x & 63;
    const int lo = NBINS - nb * (lane + 1);
    int sum = 0;
#pragma unroll
    for (int b = 0; b < nb; b += 4) {
        const uint4 v = *reinterpret_cast<const uint4*>(&sh.hist[lo + b]);
        sum += static_cast<int>(v.x + v.y + v.z + v.w);
    }
    const int incl = wave_incl_scan_add(sum);
    const int excl = incl - sum;
    // the lane whose range holds the want-th entry (exactly one: counts are
    // non-negative and the total is at least want)
    const uint64_t hit = __ballot(excl < want && incl >= want);
    const int src = __ffsll(static_cast<unsigned long long>(hit)) - 1;
    const int lo_s = NBINS - nb * (src + 1);
    const int ex_s = __builtin_amdgcn_readlane(excl, src);
    // its nb bins, top one first, one per lane; a second prefix sum finds the bin
    const int cb = lane < nb ? static_cast<int>(sh.hist[lo_s + nb - 1 - lane]) : 0;
    const int in2 = ex_s + wave_incl_scan_add(cb);
    const uint64_t hit2 = __ballot(lane < nb && in2 >= want && in2 - cb < want);
    const int l2 = __ffsll(static_cast<unsigned long long>(hit2)) - 1;
    if (lane == l2) {
        sh.digit = static_cast<uint32_t>(lo_s + nb - 1 - lane);
        sh.above = in2 - cb;
    }
}

__device__ __forceinline__ void clear_hist(RegShared& sh) {
    for (int b = threadIdx.x; b < kBuckets; b += blockDim.x) sh.hist[b] = 0u;
}

__device__ __forceinline__ int bucket_of(float v, float vmin, float scale) {
    const float f = (v - vmin) * scale;
    const int b = static_cast<int>(f);
    return b < kBuckets - 1 ? b : kBuckets - 1;
}

// blockDim.x: a power of two from 64 to 1024 with 16 * blockDim.x >= Lmax.
// speculative: issue the score loads of the whole row before pos[row] is
// known (lower latency for a few rows; rows that turn out to keep all their
// keys waste the loads, so many-row launches pass false).
__global__ __launch_bounds__(kRegMaxThreads) void topk_kernel(
    int Lmax, int K, int speculative, const float* __restrict__ scores, int64_t ld,
    const int32_t* __restrict__ pos, int32_t* __restrict__ idx, int32_t* __restrict__ count) {
    __shared__ RegShared sh;
    const int row = blockIdx.x;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int nw = static_cast<int>(blockDim.x) >> 6;
    const uint64_t lt_mask = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
    const float* srow = scores + static_cast<int64_t>(row) * ld;
    const int base = wave * (kWave * kRegItems) + lane;

    // 1. load the scores (speculatively: every in-row score, before pos is
    // known; scores past the causal end are masked below), min/max of the
    // causal ones
    float v[kRegItems];
    if (speculative) {
#pragma unroll
        for (int j = 0; j < kRegItems; ++j) {
            const int i = base + kWave * j;
            v[j] = i < Lmax ? srow[i] : 0.0f;
        }
    }
    const int p = pos[row];
    const int n = (p >= 0 && p < Lmax) ? p + 1 : 0;
    const int keff = n < K ? n : K;
    int32_t* out = idx + static_cast<int64_t>(row) * K;
    if (count != nullptr && tid == 0) count[row] = keff;
    if (keff == n) {                        // everything causal is selected
        for (int i = tid; i < K; i += blockDim.x) out[i] = i < n ? i : -1;
        return;
    }
    if (!speculative) {
#pragma unroll
        for (int j = 0; j < kRegItems; ++j) {
            const int i = base + kWave * j;
            v[j] = i < n ? srow[i] : 0.0f;
        }
    }
    float vmin = INFINITY, vmax = -INFINITY;
#pragma unroll
    for (int j = 0; j < kRegItems; ++j) {
        v[j] = v[j] + 0.0f;
        if (base + kWave * j < n) {
            vmin = fminf(vmin, v[j]);
            vmax = fmaxf(vmax, v[j]);
        }
    }
    vmin = wave_min_dpp(vmin);
    vmax = wave_max_dpp(vmax);
    if (lane == 0) {
        sh.wmin[wave] = vmin;
        sh.wmax[wave] = vmax;
        sh.wa[wave] = 0;
        sh.wb[wave] = 0;
    }
    if (tid == 0) sh.ccount = 0;
    clear_hist(sh);
    __syncthreads();
    vmin = sh.wmin[0];
    vmax = sh.wmax[0];
    for (int w = 1; w < nw; ++w) {
        vmin = fminf(vmin, sh.wmin[w]);
        vmax = fmaxf(vmax, sh.wmax[w]);
    }

    uint32_t T;                             // threshold order key
    int eq_take;                            // keys equal to T that are taken
    bool counted = false;                   // sh.wa / sh.wb already hold the per-wave counts
    if (!(vmax > vmin)) {                   // all causal scores equal
        T = float_order_key(vmax);
        eq_take = keff;
    } else {
        const float range = vmax - vmin;
        const float scale = static_cast<float>(kBuckets) / range;
        const bool bucketed = isfinite(range) && isfinite(scale) && scale > 0.0f;
        int want = keff;
        int bstar = -1;
        if (bucketed) {
            // 2. bucket histogram, threshold bucket (-1: not causal)
            int bk[kRegItems];
#pragma unroll
            for (int j = 0; j < kRegItems; ++j) {
                bk[j] = base + kWave * j < n ? bucket_of(v[j], vmin, scale) : -1;
                if (bk[j] >= 0) atomicAdd(&sh.hist[bk[j]], 1u);
            }
            __syncthreads();
            if (wave == 0) find_digit_wave0<kBuckets>(sh, keff);
            __syncthreads();
            bstar = static_cast<int>(sh.digit);
            want = keff - sh.above;
            const int c = static_cast<int>(sh.hist[bstar]);
            if (c <= kRankCap) {
                // 3a. per wave: keys in buckets above b* (all above T);
                // members of b* (key, wave) to LDS; one wave ranks them and
                // adds their counts above / equal to T to their waves
                int above_w = 0;
#pragma unroll
                for (int j = 0; j < kRegItems; ++j) {
                    above_w += __popcll(__ballot(bk[j] > bstar));
                    const bool is_c = bk[j] == bstar;
                    const uint64_t m = __ballot(is_c);
                    if (m != 0ull) {
                        int at = 0;
                        if (lane == 0) at = atomicAdd(&sh.ccount, __popcll(m));
                        at = __shfl(at, 0);
                        if (is_c) {
                            const int slot = at + __popcll(m & lt_mask);
                            sh.cand[slot] = float_order_key(v[j]);
                            sh.cand_wave[slot] = wave;
                        }
                    }
                }
                if (lane == 0) atomicAdd(&sh.wa[wave], above_w);
                __syncthreads();
                if (wave == 0) {
                    const uint32_t k = lane < c ? sh.cand[lane] : 0u;
                    int rank = 0;
                    for (int jj = 0; jj < c; ++jj) {
                        const uint32_t kj = static_cast<uint32_t>(
                            __builtin_amdgcn_readlane(static_cast<int>(k), jj));
                        rank += (kj > k || (kj == k && jj < lane)) ? 1 : 0;
                    }
                    const uint64_t hit = __ballot(lane < c && rank == want - 1);
                    const int src = __ffsll(static_cast<unsigned long long>(hit)) - 1;
                    const uint32_t Tk = static_cast<uint32_t>(
                        __builtin_amdgcn_readlane(static_cast<int>(k), src));
                    if (lane < c) {
                        if (k > Tk) atomicAdd(&sh.wa[sh.cand_wave[lane]], 1);
                        else if (k == Tk) atomicAdd(&sh.wb[sh.cand_wave[lane]], 1);
                    }
                    const int gtc = __popcll(__ballot(lane < c && k > Tk));
                    if (lane == 0) {
                        sh.T = Tk;
                        sh.gtc = gtc;
                    }
                }
                __syncthreads();
                T = sh.T;
                eq_take = want - sh.gtc;
                counted = true;
            }
        }
        if (!counted) {
            // 3b. radix select over the scores of b* (or of the whole row)
            uint32_t memb = 0u;
#pragma unroll
            for (int j = 0; j < kRegItems; ++j) {
                const bool in = base + kWave * j < n &&
                                (bstar < 0 || bucket_of(v[j], vmin, scale) == bstar);
                memb |= in ? (1u << j) : 0u;
            }
            uint32_t prefix = 0u, mask = 0u;
#pragma unroll 1
            for (int pass = 0; pass < 3; ++pass) {
                const int shift = pass == 0 ? 21 : (pass == 1 ? 10 : 0);
                const uint32_t dmask = pass == 2 ? 0x3FFu : 0x7FFu;
                __syncthreads();            // previous readers of hist / digit are done
                clear_hist(sh);
                __syncthreads();
#pragma unroll
                for (int j = 0; j < kRegItems; ++j) {
                    const uint32_t uj = float_order_key(v[j]);
                    if (((memb >> j) & 1u) && (uj & mask) == prefix)
                        atomicAdd(&sh.hist[(uj >> shift) & dmask], 1u);
                }
                __syncthreads();
                if (wave == 0) {
                    if (pass == 2) find_digit_wave0<1024>(sh, want);
                    else find_digit_wave0<kBuckets>(sh, want);
                }
                __syncthreads();
                prefix |= sh.digit << shift;
                mask |= dmask << shift;
                want -= sh.above;
            }
            T = prefix;
            eq_take = want;
        }
    }

    // 4. ordered compaction
    if (!counted) {
        int gtw = 0, eqw = 0;
#pragma unroll
        for (int j = 0; j < kRegItems; ++j) {
            const bool ok = base + kWave * j < n;
            const uint32_t uk = float_order_key(v[j]);
            gtw += __popcll(__ballot(ok && uk > T));
            eqw += __popcll(__ballot(ok && uk == T));
        }
        if (lane == 0) {
            sh.wa[wave] = gtw;
            sh.wb[wave] = eqw;
        }
        __syncthreads();
    }
    int gp = 0, ep = 0;
    for (int w = 0; w < wave; ++w) {
        gp += sh.wa[w];
        ep += sh.wb[w];
    }
    int o = gp + (ep < eq_take ? ep : eq_take);
    int e = ep;
#pragma unroll
    for (int j = 0; j < kRegItems; ++j) {
        const int i = base + kWave * j;
        const bool ok = i < n;
        const uint32_t uk = float_order_key(v[j]);
        const bool eq = ok && uk == T;
        const uint64_t eqm = __ballot(eq);
        const bool take = (ok && uk > T) || (eq && e + __popcll(eqm & lt_mask) < eq_take);
        e += __popcll(eqm);
        const uint64_t tm = __ballot(take);
        const int slot = o + __popcll(tm & lt_mask);
        if (take && slot < K) out[slot] = i;
        o += __popcll(tm);
    }
    for (int i = keff + tid; i < K; i += blockDim.x) out[i] = -1;
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
    int nt = kWave;
    while (nt * kRegItems < Lmax) nt <<= 1;
    const int speculative = rows <= 256 ? 1 : 0;
    hipLaunchKernelGGL(topk_kernel, dim3(rows), dim3(nt), 0, stream, Lmax, K, speculative, scores,
                       ld, pos, idx, count);
    return hipGetLastError();
}

}  // namespace dsa
