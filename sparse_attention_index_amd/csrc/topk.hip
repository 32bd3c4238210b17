// topk.hip -- per-query causal top-k for gfx950.
//
// Method (page "Sparse latent attention": the lightning indexer chooses up
// to 2,048 positions per query, a selection over top_2048 of the causally
// masked score; page "Rotate first features": topk(min(index_topk,
// end_pos))). Row r has n_valid = pos[r] + 1 candidates and keeps
// k_eff = min(K, n_valid) of them under (score desc, position asc), written
// in ascending position order and padded with -1.
//
// The selection block: up to 16,384 items held in registers (16 per thread;
// wave w owns the contiguous run [1024 w, 1024 w + 1024), in four groups of
// 256: lane l holds items 1024 w + 256 g + 4 l + q, q < 4, of group g, so
// every load is 16 bytes), of which the valid ones are ranked; it keeps
// k = min(K, valid count) of them.
//  1. Load (adding +0.0 folds -0.0 into +0.0) and the min/max of the valid
//     items.
//  2. Bucket pass: bucket(v) = floor((v - min) * 2048 / (max - min)), a
//     monotone non-decreasing map, so every score in a higher bucket is
//     larger than every score in a lower one. An LDS histogram, scanned by
//     one wave with DPP prefix sums, gives the bucket b* holding the k-th
//     largest score and the count G above it.
//  3. Threshold key T (the k-th largest order key, counted with
//     multiplicity): when b* holds at most 64 scores one wave ranks them;
//     otherwise an exact three-pass radix select (11/11/10-bit digits of the
//     order key) runs over the scores of b*. Blocks whose min/max give no
//     usable bucket map (all equal, infinities) run it over all items.
//     Every key above T is taken, and of the keys equal to T the ones with
//     the lowest item indices, as many as k leaves.
//  4. Ordered compaction: per-wave counts of keys above / equal to T (taken
//     during step 3 when one wave ranked b*, else by a ballot pass) give each
//     wave its output start; per group, a DPP prefix sum of the lanes' taken
//     counts places each lane's items, so each wave writes its taken items in
//     item order.
//
// Rows of up to 16,384 scores: one selection block per row over the row
// itself. Longer rows: a tournament. Level 0 splits the row into chunks of
// 16,384 scores and keeps each chunk's top k as a candidate list (score,
// position) in ascending position order; each further level merges groups of
// consecutive lists (16,384 items per block) into one list, and the last
// level writes the row's indices. A key of the row's top k is in the top k
// of every subset that holds it (fewer keys of the subset beat it), so no
// level drops it. Item order equals position order at every level, so the
// tie rule (lower position first) and the ascending output carry through.
#include "dsa_common.h"

#include <type_traits>

namespace dsa {

constexpr int kRegItems = 16;                           // scores per thread
constexpr int kRegMaxThreads = 1024;
constexpr int kRegMaxWaves = kRegMaxThreads / kWave;
constexpr int kBlockItems = kRegItems * kRegMaxThreads; // items of one selection block
constexpr int kBuckets = 2048;
constexpr int kRankCap = kWave;                         // bucket sizes ranked by one wave

struct alignas(16) RegShared {
    uint32_t hist[kBuckets];
    uint32_t cand[kRankCap];
    int cand_wave[kRankCap];
    int wa[kRegMaxWaves];                   // per wave: keys above T
    int wb[kRegMaxWaves];                   // per wave: keys equal to T
    int wn[kRegMaxWaves];                   // per wave: valid items
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

// Number of lanes below this one whose bit is set in m.
__device__ __forceinline__ int lanes_below(uint64_t m) {
    return static_cast<int>(__builtin_amdgcn_mbcnt_hi(
        static_cast<uint32_t>(m >> 32), __builtin_amdgcn_mbcnt_lo(static_cast<uint32_t>(m), 0u)));
}

// The float with order key k (the inverse of float_order_key; key
// 0x80000000 gives +0.0). The key map is strictly monotone and maps -0 and +0
// alike, so for non-NaN x: key(x) > k iff x > value(k), key(x) == k iff
// x == value(k).
__device__ __forceinline__ float order_key_value(uint32_t k) {
    return __uint_as_float((k & 0x80000000u) ? (k & 0x7FFFFFFFu) : ~k);
}

__device__ __forceinline__ void clear_hist(RegShared& sh) {
    for (int b = threadIdx.x; b < kBuckets; b += blockDim.x) sh.hist[b] = 0u;
}

// Bucket of v under the map floor(v * scale + off) (off = -vmin * scale),
// clamped to [0, kBuckets - 1]: one fma, correctly rounded, so the map is
// monotone non-decreasing in v (the histogram and every later membership
// test use this one function). At v = vmin the fma gives the tiny rounding
// residual of vmin * scale, which truncates to bucket 0.
__device__ __forceinline__ int bucket_of(float v, float scale, float off) {
    const int b = static_cast<int>(__builtin_fmaf(v, scale, off));
    return b < kBuckets - 1 ? b : kBuckets - 1;
}

// Arguments of one selection launch. Block x covers part x % nparts of row
// x / nparts: a chunk of blockDim.x * 16 scores of the row (score source) or
// a group of consecutive candidate lists (candidate source).
struct SelectArgs {
    int Lmax, K;
    int nparts;                 // blocks per row
    int speculative;            // score source: load before pos[row] is known
    int kp_shift;               // candidate list stride Kp = 2^kp_shift >= K
    // score source
    const float* scores;
    int64_t ld;
    const int32_t* pos;
    // candidate source: row r's list s at ((r * in_lists + s) << kp_shift)
    const float* in_key;
    const int32_t* in_pos;
    const int32_t* in_cnt;      // [rows][in_lists]
    int in_lists;
    // index output
    int32_t* idx;
    int32_t* count;
    // candidate output: list (row, part), nparts lists per row
    float* out_key;
    int32_t* out_pos;
    int32_t* out_cnt;
};

// blockDim.x: a power of two from 64 to 1024; with the score source the row
// chunk of part x starts at x * blockDim.x * 16 and 16 * blockDim.x >= Lmax
// when nparts == 1.
template <bool CAND_IN, bool CAND_OUT>
__global__ __launch_bounds__(kRegMaxThreads) void topk_select_kernel(SelectArgs a) {
    __shared__ RegShared sh;
    const int row = static_cast<int>(blockIdx.x) / a.nparts;
    const int part = static_cast<int>(blockIdx.x) - row * a.nparts;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int nw = static_cast<int>(blockDim.x) >> 6;
    const int nitems = static_cast<int>(blockDim.x) * kRegItems;
    const int base4 = wave * (kWave * kRegItems) + lane * 4;
    // block-local index of this thread's item j (group j / 4, element j % 4)
    auto item = [&](int j) -> int { return base4 + (j >> 2) * (kWave * 4) + (j & 3); };
    const int kps = a.kp_shift;
    const int K = a.K;

    // 1. load the items
    float v[kRegItems];
    int32_t pv[CAND_IN ? kRegItems : 1];     // candidate source: positions of the items
    uint32_t vmask = 0u;                     // candidate source: bit j = item j is valid
    int M = 0;                               // valid items of the block
    int start = 0;                           // score source: chunk start in the row
    int64_t cbase = 0;                       // candidate source: first item of the group
    if constexpr (!CAND_IN) {
        start = part * nitems;
        const float* src = a.scores + static_cast<int64_t>(row) * a.ld + start;
        const int lim = min(a.Lmax - start, nitems);
        const bool vec = (reinterpret_cast<uintptr_t>(src) & 15u) == 0u;
        // items [i, i + 4) of the chunk, those at or past `bound` read as 0
        auto load_group = [&](int g4, int bound) {
            const int i = base4 + g4 * (kWave * 4);
            if (vec && i + 3 < bound) {
                const float4 t = *reinterpret_cast<const float4*>(src + i);
                v[4 * g4] = t.x;
                v[4 * g4 + 1] = t.y;
                v[4 * g4 + 2] = t.z;
                v[4 * g4 + 3] = t.w;
            } else {
#pragma unroll
                for (int q = 0; q < 4; ++q) v[4 * g4 + q] = i + q < bound ? src[i + q] : 0.0f;
            }
        };
        if (a.speculative) {
#pragma unroll
            for (int g4 = 0; g4 < kRegItems / 4; ++g4) load_group(g4, lim);
        }
        const int p = a.pos[row];
        const int n = (p >= 0 && p < a.Lmax) ? p + 1 : 0;
        M = min(max(n - start, 0), nitems);
        const int keff0 = M < K ? M : K;
        if (keff0 == M) {                    // every valid item is selected
            if constexpr (CAND_OUT) {
                const int64_t ob = (static_cast<int64_t>(row) * a.nparts + part) << kps;
                for (int i = tid; i < M; i += blockDim.x) {
                    a.out_key[ob + i] = src[i] + 0.0f;
                    a.out_pos[ob + i] = start + i;
                }
                if (tid == 0) a.out_cnt[static_cast<int64_t>(row) * a.nparts + part] = M;
            } else {
                int32_t* out = a.idx + static_cast<int64_t>(row) * K;
                for (int i = tid; i < K; i += blockDim.x) out[i] = i < M ? i : -1;
                if (a.count != nullptr && tid == 0) a.count[row] = M;
            }
            return;
        }
        if (!a.speculative) {
#pragma unroll
            for (int g4 = 0; g4 < kRegItems / 4; ++g4) load_group(g4, M);
        }
    } else {
        const int kpm = (1 << kps) - 1;
        const int slot0 = part * (nitems >> kps);
        const int nsl = min(nitems >> kps, a.in_lists - slot0);   // lists in the group
        cbase = (static_cast<int64_t>(row) * a.in_lists + slot0) << kps;
        const int32_t* cnt = a.in_cnt + static_cast<int64_t>(row) * a.in_lists + slot0;
        // all loads first (keys, positions, list counts), then the valid
        // bits. Lists of at least 4 entries keep a group of 4 in one list and
        // 16-byte aligned (the workspace is 256-byte aligned).
        int cj[kRegItems];
        if (kps >= 2) {
#pragma unroll
            for (int g4 = 0; g4 < kRegItems / 4; ++g4) {
                const int i = base4 + g4 * (kWave * 4);
                const int s = i >> kps;
                float4 kv = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
                int4 pq = make_int4(0, 0, 0, 0);
                int c = 0;
                if (s < nsl) {
                    kv = *reinterpret_cast<const float4*>(a.in_key + cbase + i);
                    pq = *reinterpret_cast<const int4*>(a.in_pos + cbase + i);
                    c = cnt[s];
                }
                v[4 * g4] = kv.x;
                v[4 * g4 + 1] = kv.y;
                v[4 * g4 + 2] = kv.z;
                v[4 * g4 + 3] = kv.w;
                pv[4 * g4] = pq.x;
                pv[4 * g4 + 1] = pq.y;
                pv[4 * g4 + 2] = pq.z;
                pv[4 * g4 + 3] = pq.w;
#pragma unroll
                for (int q = 0; q < 4; ++q) cj[4 * g4 + q] = c;
            }
        } else {
#pragma unroll
            for (int j = 0; j < kRegItems; ++j) {
                const int i = item(j);
                const int s = i >> kps;
                const bool in = s < nsl;
                v[j] = in ? a.in_key[cbase + i] : 0.0f;
                pv[j] = in ? a.in_pos[cbase + i] : 0;
                cj[j] = in ? cnt[s] : 0;
            }
        }
#pragma unroll
        for (int j = 0; j < kRegItems; ++j) vmask |= (item(j) & kpm) < cj[j] ? (1u << j) : 0u;
    }
    // item j of this thread is valid: a prefix of the chunk (score source,
    // one compare against M) or the per-list counts (candidate source)
    auto valid = [&](int j) -> bool {
        if constexpr (CAND_IN) return (vmask >> j) & 1u;
        else return item(j) < M;
    };
    // every item of the wave is valid (wave-uniform): the per-item loops
    // below then skip the validity tests (the work is VALU-bound: 16 waves
    // of one CU run every per-item instruction)
    bool wave_full;
    if constexpr (CAND_IN) wave_full = __ballot(vmask != 0xFFFFu) == 0ull;
    else wave_full = (wave + 1) * (kWave * kRegItems) <= M;
    float vmin = INFINITY, vmax = -INFINITY;
    if (wave_full) {
#pragma unroll
        for (int j = 0; j < kRegItems; ++j) {
            v[j] = v[j] + 0.0f;
            vmin = fminf(vmin, v[j]);
            vmax = fmaxf(vmax, v[j]);
        }
    } else {
#pragma unroll
        for (int j = 0; j < kRegItems; ++j) {
            v[j] = v[j] + 0.0f;
            if (valid(j)) {
                vmin = fminf(vmin, v[j]);
                vmax = fmaxf(vmax, v[j]);
            }
        }
    }
    vmin = wave_min_dpp(vmin);
    vmax = wave_max_dpp(vmax);
    int wn = 0;
    if constexpr (CAND_IN) {
#pragma unroll
        for (int j = 0; j < kRegItems; ++j) wn += __popcll(__ballot(valid(j)));
    }
    if (lane == 0) {
        sh.wmin[wave] = vmin;
        sh.wmax[wave] = vmax;
        sh.wn[wave] = wn;
        sh.wa[wave] = 0;
        sh.wb[wave] = 0;
    }
    if (tid == 0) sh.ccount = 0;
    clear_hist(sh);
    __syncthreads();
    // block totals: lane l < nw reads wave l's figures and wave reductions
    // combine them (one LDS round trip instead of one per wave)
    const bool wl_ok = lane < nw;
    const int wl = wl_ok ? lane : 0;
    vmin = wave_min_dpp(wl_ok ? sh.wmin[wl] : INFINITY);
    vmax = wave_max_dpp(wl_ok ? sh.wmax[wl] : -INFINITY);
    if constexpr (CAND_IN)
        M = __builtin_amdgcn_readlane(wave_incl_scan_add(wl_ok ? sh.wn[wl] : 0), 63);
    const int keff = M < K ? M : K;

    uint32_t T = 0u;                        // threshold order key
    int eq_take = 0;                        // keys equal to T that are taken
    bool counted = false;                   // sh.wa / sh.wb already hold the per-wave counts
    const bool take_all = keff == M;        // every valid item is selected
    if (take_all) {
    } else if (!(vmax > vmin)) {            // all valid scores equal
        T = float_order_key(vmax);
        eq_take = keff;
    } else {
        const float range = vmax - vmin;
        const float scale = static_cast<float>(kBuckets) / range;
        const float off = -vmin * scale;
        const bool bucketed = isfinite(range) && isfinite(scale) && scale > 0.0f &&
                              isfinite(off);
        int want = keff;
        int bstar = -1;
        if (bucketed) {
            // 2. bucket histogram, threshold bucket (-1: not valid)
            int bk[kRegItems];
            if (wave_full) {
#pragma unroll
                for (int j = 0; j < kRegItems; ++j) {
                    bk[j] = bucket_of(v[j], scale, off);
                    atomicAdd(&sh.hist[bk[j]], 1u);
                }
            } else {
#pragma unroll
                for (int j = 0; j < kRegItems; ++j) {
                    bk[j] = valid(j) ? bucket_of(v[j], scale, off) : -1;
                    if (bk[j] >= 0) atomicAdd(&sh.hist[bk[j]], 1u);
                }
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
                            const int slot = at + lanes_below(m);
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
            // 3b. radix select over the scores of b* (or over all valid items)
            uint32_t memb = 0u;
#pragma unroll
            for (int j = 0; j < kRegItems; ++j) {
                const bool in = valid(j) &&
                                (bstar < 0 || bucket_of(v[j], scale, off) == bstar);
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

    // 4. ordered compaction: taken are the valid items above T and, of those
    // equal to T, the first eq_take in item order (compared as floats against
    // the value of T)
    const float Tf = order_key_value(T);
    auto above = [&](int j) -> bool { return valid(j) && (take_all || v[j] > Tf); };
    auto equal = [&](int j) -> bool { return !take_all && valid(j) && v[j] == Tf; };
    if (!counted) {
        int gtw = 0, eqw = 0;
#pragma unroll
        for (int j = 0; j < kRegItems; ++j) {
            gtw += __popcll(__ballot(above(j)));
            eqw += __popcll(__ballot(equal(j)));
        }
        if (lane == 0) {
            sh.wa[wave] = gtw;
            sh.wb[wave] = eqw;
        }
        __syncthreads();
    }
    // counts of the waves before this one: lane l reads wave l's, an
    // exclusive prefix sum over the lanes, read at lane `wave`
    int gp, ep;
    {
        const int ga = wl_ok ? sh.wa[wl] : 0, gb = wl_ok ? sh.wb[wl] : 0;
        gp = __builtin_amdgcn_readlane(wave_incl_scan_add(ga) - ga, wave);
        ep = __builtin_amdgcn_readlane(wave_incl_scan_add(gb) - gb, wave);
    }
    int o = gp + (ep < eq_take ? ep : eq_take);
    int e = ep;
    int32_t* out = nullptr;
    int64_t ob = 0;
    if constexpr (CAND_OUT) ob = (static_cast<int64_t>(row) * a.nparts + part) << kps;
    else out = a.idx + static_cast<int64_t>(row) * K;
    // Item order within a wave is (group, lane, element). Each lane turns its
    // 16 items into bit masks (taken / equal to T), counts each group's
    // nibble, and two DPP prefix sums over the lanes of the counts packed in
    // 16-bit fields (at most 256 per field) give every lane its first slot
    // in each group; the lane then stores its taken items in order. Ties at
    // T (rare; wave-uniform test) are ranked the same way among the equal
    // items before the taken counts are formed.
    auto nib = [](uint32_t m, int g) { return __popc((m >> (4 * g)) & 0xFu); };
    auto field = [](int lo, int hi, int g) {
        const int x = g < 2 ? lo : hi;
        return (g & 1) ? (x >> 16) : (x & 0xFFFF);
    };
    auto compact = [&](auto full_tag) {
        constexpr bool FULL = decltype(full_tag)::value;
        uint32_t tkm = 0u, eqm = 0u;
#pragma unroll
        for (int j = 0; j < kRegItems; ++j) {
            const bool ok = FULL || valid(j);
            tkm |= (ok && (take_all || v[j] > Tf)) ? (1u << j) : 0u;
            eqm |= (ok && !take_all && v[j] == Tf) ? (1u << j) : 0u;
        }
        if (__ballot(eqm != 0u) != 0ull) {
            const int lo = nib(eqm, 0) | (nib(eqm, 1) << 16), hi = nib(eqm, 2) | (nib(eqm, 3) << 16);
            const int ilo = wave_incl_scan_add(lo), ihi = wave_incl_scan_add(hi);
            const int tlo = __builtin_amdgcn_readlane(ilo, 63), thi = __builtin_amdgcn_readlane(ihi, 63);
            int er = e;
#pragma unroll
            for (int g4 = 0; g4 < kRegItems / 4; ++g4) {
                int r = er + field(ilo - lo, ihi - hi, g4);
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const int j = 4 * g4 + q;
                    if ((eqm >> j) & 1u) {
                        tkm |= r < eq_take ? (1u << j) : 0u;
                        ++r;
                    }
                }
                er += field(tlo, thi, g4);
            }
            e = er;
        }
        const int lo = nib(tkm, 0) | (nib(tkm, 1) << 16), hi = nib(tkm, 2) | (nib(tkm, 3) << 16);
        const int ilo = wave_incl_scan_add(lo), ihi = wave_incl_scan_add(hi);
        const int tlo = __builtin_amdgcn_readlane(ilo, 63), thi = __builtin_amdgcn_readlane(ihi, 63);
#pragma unroll
        for (int g4 = 0; g4 < kRegItems / 4; ++g4) {
            int slot = o + field(ilo - lo, ihi - hi, g4);
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const int j = 4 * g4 + q;
                if ((tkm >> j) & 1u) {
                    if (slot < keff) {
                        int32_t p;
                        if constexpr (CAND_IN) p = pv[j];
                        else p = start + item(j);
                        if constexpr (CAND_OUT) {
                            a.out_key[ob + slot] = v[j];
                            a.out_pos[ob + slot] = p;
                        } else {
                            out[slot] = p;
                        }
                    }
                    ++slot;
                }
            }
            o += field(tlo, thi, g4);
        }
    };
    if (wave_full) compact(std::true_type{});
    else compact(std::false_type{});
    if constexpr (CAND_OUT) {
        if (tid == 0) a.out_cnt[static_cast<int64_t>(row) * a.nparts + part] = keff;
    } else {
        for (int i = keff + tid; i < K; i += blockDim.x) out[i] = -1;
        if (a.count != nullptr && tid == 0) a.count[row] = keff;
    }
}

// ---------------------------------------------------------------------------
// Tournament plan for rows longer than one selection block. Candidate lists
// have stride Kp = K rounded up to a power of two; a merge block takes
// 16,384 / Kp consecutive lists. Buffer A holds the level-0 lists (one per
// 16,384-score chunk), buffer B the level-1 lists; later levels alternate.
// Each buffer: keys [rows][lists][Kp] f32 | positions (same) i32 |
// counts [rows][lists] i32, each part 256-byte aligned. No initial contents
// are needed: every list a launch reads was written by the previous one.
// ---------------------------------------------------------------------------
struct TourPlan {
    int kp_shift, group, lists0, lists1;
    size_t a_key, a_pos, a_cnt, b_key, b_pos, b_cnt, bytes;
};

static size_t align256(size_t x) { return (x + 255) & ~static_cast<size_t>(255); }

static TourPlan tour_plan(int rows, int Lmax, int K) {
    TourPlan t;
    t.kp_shift = 0;
    while ((1 << t.kp_shift) < K) ++t.kp_shift;
    t.group = kBlockItems >> t.kp_shift;
    t.lists0 = (Lmax + kBlockItems - 1) / kBlockItems;
    t.lists1 = t.lists0 > t.group ? (t.lists0 + t.group - 1) / t.group : 0;
    const size_t r = static_cast<size_t>(rows);
    const size_t kp = static_cast<size_t>(1) << t.kp_shift;
    size_t o = 0;
    t.a_key = o; o += align256(r * t.lists0 * kp * 4);
    t.a_pos = o; o += align256(r * t.lists0 * kp * 4);
    t.a_cnt = o; o += align256(r * t.lists0 * 4);
    t.b_key = o; o += align256(r * t.lists1 * kp * 4);
    t.b_pos = o; o += align256(r * t.lists1 * kp * 4);
    t.b_cnt = o; o += align256(r * t.lists1 * 4);
    t.bytes = o;
    return t;
}

size_t topk_workspace_bytes(int rows, int Lmax, int K) {
    if (Lmax <= kBlockItems) return 0;
    return tour_plan(rows, Lmax, K).bytes;
}

// Blocks of the largest launch (level 0), for the grid-size check.
int64_t topk_max_blocks(int rows, int Lmax) {
    return static_cast<int64_t>(rows) * ((Lmax + kBlockItems - 1) / kBlockItems);
}

hipError_t launch_topk(int rows, int Lmax, int K, const float* scores, int64_t ld,
                       const int32_t* pos, int32_t* idx, int32_t* count, void* workspace,
                       hipStream_t stream) {
    SelectArgs a{};
    a.Lmax = Lmax;
    a.K = K;
    a.scores = scores;
    a.ld = ld;
    a.pos = pos;
    a.idx = idx;
    a.count = count;
    a.speculative = rows <= 256 ? 1 : 0;
    if (Lmax <= kBlockItems) {
        int nt = kWave;
        while (nt * kRegItems < Lmax) nt <<= 1;
        a.nparts = 1;
        hipLaunchKernelGGL((topk_select_kernel<false, false>), dim3(rows), dim3(nt), 0, stream, a);
        return hipGetLastError();
    }
    const TourPlan t = tour_plan(rows, Lmax, K);
    unsigned char* ws = static_cast<unsigned char*>(workspace);
    float* key[2] = {reinterpret_cast<float*>(ws + t.a_key), reinterpret_cast<float*>(ws + t.b_key)};
    int32_t* cpos[2] = {reinterpret_cast<int32_t*>(ws + t.a_pos),
                        reinterpret_cast<int32_t*>(ws + t.b_pos)};
    int32_t* cnt[2] = {reinterpret_cast<int32_t*>(ws + t.a_cnt),
                       reinterpret_cast<int32_t*>(ws + t.b_cnt)};
    a.kp_shift = t.kp_shift;
    // level 0: row chunks -> candidate lists in A
    a.nparts = t.lists0;
    a.out_key = key[0];
    a.out_pos = cpos[0];
    a.out_cnt = cnt[0];
    hipLaunchKernelGGL((topk_select_kernel<false, true>), dim3(rows * t.lists0),
                       dim3(kRegMaxThreads), 0, stream, a);
    int cur = 0, lists = t.lists0;
    while (lists > t.group) {                // merge levels
        const int nout = (lists + t.group - 1) / t.group;
        a.in_key = key[cur];
        a.in_pos = cpos[cur];
        a.in_cnt = cnt[cur];
        a.in_lists = lists;
        a.nparts = nout;
        a.out_key = key[cur ^ 1];
        a.out_pos = cpos[cur ^ 1];
        a.out_cnt = cnt[cur ^ 1];
        hipLaunchKernelGGL((topk_select_kernel<true, true>), dim3(rows * nout),
                           dim3(kRegMaxThreads), 0, stream, a);
        cur ^= 1;
        lists = nout;
    }
    // last level: the row's remaining lists -> indices
    a.in_key = key[cur];
    a.in_pos = cpos[cur];
    a.in_cnt = cnt[cur];
    a.in_lists = lists;
    a.nparts = 1;
    int nt = kWave;
    while (nt * kRegItems < (lists << t.kp_shift)) nt <<= 1;
    hipLaunchKernelGGL((topk_select_kernel<true, false>), dim3(rows), dim3(nt), 0, stream, a);
    return hipGetLastError();
}

}  // namespace dsa
