// sparse_mha.hip -- sparse attention in the multi-head (non-absorbed) prefill
// form, gfx950.
//
// Method (page "RoPE coefficients", MLA prefill excerpt): every head has its
// own key [k_nope (128) ; k_pe (64, shared by the heads)] and value (128)
// from the up-projection of the latent rows; the scores q . k are scaled,
// the index mask (0 where the top-k list scatters, -inf elsewhere) and the
// causal mask are added, and the softmax over positions weights the values.
// For row r = (b, s), head h:
//   z_p   = scale * (q[r][h][0:128] . kv[b][p][h][0:128] + q[r][h][128:192] . rope[b][p])
//   out[r][h] = sum_p softmax(z)_p kv[b][p][h][128:256]
// over the positions p in the row's list (a repeat counts once, as in a
// scattered mask) with 0 <= p < Lmax and p <= pos[r] when positions are
// given.
//
// Design. The masked dense form is computed, tile by tile, only where the
// mask has something:
//  1. selection_rows_kernel turns each row's list into a bit mask over
//     positions (two 32-bit words per 64-position tile, one wave per row);
//     tile_lists_kernel lists, for every 128-row query tile, the
//     64-position key tiles that any of its rows selects, with the union of
//     the rows' bits.
//  2. sparse_mha_kernel: one block of 4 waves per (query tile, head); wave w
//     serves rows 32w..32w+31 as two 16-row groups. The head's 64 key/value
//     rows of each listed key tile go straight from global memory into one
//     of two LDS tile buffers (direct loads, no registers; positions no row
//     selects load zeros): the next tile's loads are issued before the
//     current tile is computed. Per wave and tile:
//       S^T = K Q^T    bf16 MFMA 16x16x32, keys x rows, Q^T held in VGPRs,
//                      each K operand read once for both row groups;
//       online softmax per row (masked scores are -inf; a wave whose rows
//                      select the whole tile skips the mask tests), in log2
//                      units with the scale folded into the exponent's fma,
//                      against a reference maximum that moves only when the
//                      running maximum passes it by 8;
//       O^T += V^T P^T P^T straight from the S^T registers (the key order
//                      inside the MFMA's K dimension only has to agree
//                      between the operands), V^T by the transposing LDS
//                      read from the row-major value rows.
//     Tile rows are stored with XOR-swizzled 16-byte chunks so the operand
//     reads hit distinct banks. Launch order: the heads of a query tile are
//     adjacent, query tiles with the longest causal extent first (measured
//     7% faster than giving each XCD whole heads).
#include "dsa_common.h"

namespace dsa {

constexpr int kMhaRows = 128;           // query rows per block
constexpr int kMhaKeys = 64;            // positions per key tile
constexpr int kMhaThreads = 256;
// LDS tile buffer: k_nope [64][256 B], k_pe [64][128 B], v [64][256 B]
constexpr int kMhaKP = 64 * 256, kMhaV = kMhaKP + 64 * 128;
constexpr int kMhaTileBytes = kMhaV + 64 * 256;
constexpr int kMhaLoads = kMhaTileBytes / 1024 / 4;   // direct loads per thread per tile (10)
constexpr size_t kMhaLds = 2 * static_cast<size_t>(kMhaTileBytes);
constexpr int kMaskThreads = 256;

// ---- 1. bit masks and key-tile lists ---------------------------------------
// 1a. One wave per query row: the row's list becomes a bit mask over
// positions, built in LDS (one row per wave) and written out whole.
constexpr int kMaskRowsPerBlock = kMaskThreads / 64;

__global__ __launch_bounds__(kMaskThreads) void selection_rows_kernel(
    int S, int Lmax, int K, int nw, int64_t nrows, const int32_t* __restrict__ idx,
    const int32_t* __restrict__ pos, uint32_t* __restrict__ mask, uint16_t* __restrict__ zeros) {
    extern __shared__ uint32_t msm[];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int64_t r = static_cast<int64_t>(blockIdx.x) * kMaskRowsPerBlock + wave;
    const bool valid = r < nrows;
    // 256 zero bytes: the source of unselected positions in the attention gather
    if (blockIdx.x == 0 && tid < 16) reinterpret_cast<uint4*>(zeros)[tid] = make_uint4(0u, 0u, 0u, 0u);
    uint32_t* rb = msm + wave * nw;
    for (int i = lane; i < nw; i += 64) rb[i] = 0u;
    __syncthreads();
    if (valid) {
        const int pr = pos != nullptr ? pos[r] : 0x7FFFFFFF;
        const int32_t* sel = idx + r * K;
        for (int j0 = 0; j0 < K; j0 += 64) {
            const int j = j0 + lane;
            const int p = j < K ? sel[j] : -1;
            const bool ok = p >= 0 && p < Lmax && p <= pr;
            // lanes holding the same word OR their bits towards the first
            // lane of each run of equal words, which alone writes (fewer LDS
            // atomics on one address); any order of the list is correct
            int w = ok ? (p >> 5) : -1 - lane;
            uint32_t bit = ok ? (1u << (p & 31)) : 0u;
#pragma unroll
            for (int d = 1; d < 64; d <<= 1) {
                const uint32_t ob = static_cast<uint32_t>(__shfl_down(static_cast<int>(bit), d));
                const int ow = __shfl_down(w, d);
                if (ow == w) bit |= ob;
            }
            const int prev = __shfl_up(w, 1);
            if (ok && (lane == 0 || prev != w)) atomicOr(&rb[w], bit);
        }
    }
    __syncthreads();
    if (valid) {
        uint32_t* mrow = mask + r * nw;
        for (int i = lane; i < nw; i += 64) mrow[i] = rb[i];
    }
}

// 1b. One block per 128-row query tile: the union of its rows' masks, then
// the list of 64-position tiles with any bit set (entry 0: the count; then
// (tile, union bits low, union bits high, 0) in ascending order).
__global__ __launch_bounds__(kMaskThreads) void tile_lists_kernel(
    int S, int nkt, int ntq, const uint32_t* __restrict__ mask, int4* __restrict__ tiles) {
    extern __shared__ uint32_t tun[];
    const int nw = 2 * nkt;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int qt = blockIdx.x;
    const int64_t b = qt / ntq;
    const int t0 = (qt % ntq) * kMhaRows;
    const int t1 = min(S, t0 + kMhaRows);
    const uint32_t* m0 = mask + (b * S + t0) * nw;
    for (int i = tid; i < nw; i += kMaskThreads) tun[i] = 0u;
    __syncthreads();
    // G row groups per word when the words are fewer than the threads
    const int G = max(1, kMaskThreads / nw);
    for (int x = tid; x < nw * G; x += kMaskThreads) {
        const int i = x % nw, g0 = x / nw;
        uint32_t u = 0u;
        for (int t = g0; t < t1 - t0; t += G) u |= m0[static_cast<int64_t>(t) * nw + i];
        if (u) atomicOr(&tun[i], u);
    }
    __syncthreads();
    if (wave == 0) {
        int4* tl = tiles + static_cast<int64_t>(qt) * (nkt + 1);
        int base = 0;
        for (int k0 = 0; k0 < nkt; k0 += 64) {
            const int kt = k0 + lane;
            const uint32_t lo = kt < nkt ? tun[2 * kt] : 0u;
            const uint32_t hi = kt < nkt ? tun[2 * kt + 1] : 0u;
            const bool nz = (lo | hi) != 0u;
            const uint64_t bal = __ballot(nz);
            const int rank = __popcll(bal & ((uint64_t(1) << lane) - 1));
            if (nz) tl[1 + base + rank] = make_int4(kt, static_cast<int>(lo), static_cast<int>(hi), 0);
            base += __popcll(bal);
        }
        if (lane == 0) tl[0] = make_int4(base, 0, 0, 0);
    }
}

// ---- 2. attention over the listed key tiles ---------------------------------
__global__ __launch_bounds__(kMhaThreads, 2) void sparse_mha_kernel(
    int S, int Hq, int Lmax, int nkt, int ntq, int nqt, const uint16_t* __restrict__ q,
    const uint16_t* __restrict__ kv, const uint16_t* __restrict__ rope, int64_t rope_rs,
    int64_t rope_bs, const uint32_t* __restrict__ mask, const int4* __restrict__ tiles,
    const uint16_t* __restrict__ zeros, float scale_log2, uint16_t* __restrict__ out) {
    extern __shared__ __align__(16) unsigned char kvs[];     // two tile buffers

    // launch index -> (head, query tile): the heads of one query tile are
    // adjacent (they share its mask rows and tile list); longest causal
    // extent first
    const int L = blockIdx.x;
    const int h = L % Hq;
    const int qtg = nqt - 1 - L / Hq;
    const int64_t b = qtg / ntq;
    const int t0 = (qtg % ntq) * kMhaRows;
    const int nw = 2 * nkt;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int m = lane & 15, g = lane >> 4;

    // rows of this lane's two groups: t0 + 32 wave + 16 qg + m
    int64_t rr[2];
    bool rv[2];
#pragma unroll
    for (int qg = 0; qg < 2; ++qg) {
        const int t = t0 + 32 * wave + 16 * qg + m;
        rv[qg] = t < S;
        rr[qg] = b * S + (rv[qg] ? t : 0);
    }
    // Q^T operands: lane (row m, chunk g) holds q[row][h][32 ks + 8 g .. +7]
    bf16x8 qreg[2][6];
#pragma unroll
    for (int qg = 0; qg < 2; ++qg) {
        const uint16_t* qh = q + (rr[qg] * Hq + h) * 192 + 8 * g;
#pragma unroll
        for (int ks = 0; ks < 6; ++ks) {
            uint4 v = *reinterpret_cast<const uint4*>(qh + 32 * ks);
            if (!rv[qg]) v = make_uint4(0u, 0u, 0u, 0u);
            qreg[qg][ks] = __builtin_bit_cast(bf16x8, v);
        }
    }
    v4f acc[2][8];
#pragma unroll
    for (int qg = 0; qg < 2; ++qg)
#pragma unroll
        for (int t2 = 0; t2 < 8; ++t2) acc[qg][t2] = v4f{0.0f, 0.0f, 0.0f, 0.0f};
    float m_run[2] = {-INFINITY, -INFINITY}, l_run[2] = {0.0f, 0.0f};

    const int4* tl = tiles + static_cast<int64_t>(qtg) * (nkt + 1);
    const int ntile = tl[0].x;

    // Gather: direct global-to-LDS loads (lane l of a wave instruction
    // writes bytes 16 l .. +15 of that instruction's 1 KiB). Regions of a
    // tile buffer, with 16-byte chunk c of row r stored at position c ^ f(r):
    //   k_nope rows of 16 chunks, f = r & 15            (instructions 0..15, 4 rows each)
    //   k_pe   rows of  8 chunks, f = (r >> 1) & 7      (16..23, 8 rows each)
    //   v      rows of 16 chunks, f = 2 (r & 3) | 8 ((r >> 2) & 1)   (24..39)
    // so that the 16 rows of a K operand read, and the rows of a transposing
    // V read, fall on distinct banks. Wave w issues instructions w + 4 i;
    // the chunk a lane loads does not depend on i. Positions no row of the
    // query tile selects load 16 zero bytes.
    const int rq = lane >> 4, r8 = lane >> 3;
    const int cKN = (lane & 15) ^ ((4 * wave + rq) & 15);
    const int cKP = (lane & 7) ^ ((4 * wave + rq) & 7);
    const int cV = (lane & 15) ^ (2 * rq | 8 * (wave & 1));
    uint2 mw[2];
    const uint16_t* kv_bh = kv + (b * Lmax * Hq + h) * 256;
    const uint16_t* rope_b = rope + b * rope_bs;
    const int64_t kv_rs = static_cast<int64_t>(Hq) * 256;
    auto issue = [&](int it) {
        const int4 e = tl[1 + it];
        const int kt = e.x;
        unsigned char* buf = kvs + (it & 1) * kMhaTileBytes;
        const int64_t s0 = static_cast<int64_t>(kt) * kMhaKeys;
        // the source, or the zero bytes for a position no row selects (a
        // select on the address, so every lane issues the same loads)
        auto pick = [&](int r, const uint16_t* src) {
            const uint32_t bit = (r < 32 ? static_cast<uint32_t>(e.y) >> r
                                         : static_cast<uint32_t>(e.z) >> (r - 32)) & 1u;
            const uint64_t a = reinterpret_cast<uint64_t>(src), zz = reinterpret_cast<uint64_t>(zeros);
            return reinterpret_cast<const uint16_t*>(zz ^ ((a ^ zz) & (0ull - bit)));
        };
#pragma unroll
        for (int i = 0; i < 4; ++i) {                     // k_nope: rows 4 n + lane / 16
            const int r = 4 * wave + 16 * i + rq;
            const uint16_t* src = kv_bh + (s0 + r) * kv_rs + 8 * cKN;
            load_to_lds(pick(r, src), buf + 1024 * (wave + 4 * i));
        }
#pragma unroll
        for (int i = 0; i < 2; ++i) {                     // k_pe: rows 8 n' + lane / 8
            const int r = 8 * wave + 32 * i + r8;
            const uint16_t* src = rope_b + (s0 + r) * rope_rs + 8 * cKP;
            load_to_lds(pick(r, src), buf + kMhaKP + 1024 * (wave + 4 * i));
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) {                     // v: rows 4 n'' + lane / 16
            const int r = 4 * wave + 16 * i + rq;
            const uint16_t* src = kv_bh + (s0 + r) * kv_rs + 128 + 8 * cV;
            load_to_lds(pick(r, src), buf + kMhaV + 1024 * (wave + 4 * i));
        }
#pragma unroll
        for (int qg = 0; qg < 2; ++qg)
            mw[qg] = rv[qg] ? *reinterpret_cast<const uint2*>(mask + rr[qg] * nw + 2 * kt)
                            : make_uint2(0u, 0u);
    };

    // operand reads: K rows 16 st + m; V^T transposing reads, lane 4e+q of
    // group g: rows 4g + e (+16) of a 32-key half, value chunk 2 t2 + q/2,
    // half q % 2
    const int e4 = (lane >> 2) & 3, q4 = lane & 3;
    const int fv = 2 * e4 | 8 * (g & 1);
    const int vrow = kMhaV + (4 * g + e4) * 256 + 8 * (q4 & 1);

    if (ntile > 0) issue(0);
    for (int it = 0; it < ntile; ++it) {
        wait_vmcnt<0>();                                 // this tile's loads (own)
        __builtin_amdgcn_s_barrier();                  // everyone's; previous tile consumed
        const uint2 mcur[2] = {mw[0], mw[1]};
        if (it + 1 < ntile) issue(it + 1);
        const unsigned char* Kt = kvs + (it & 1) * kMhaTileBytes;

        // S^T: s[qg][st] for keys 16 st + 4 g + i, row m of group qg
        v4f s[2][4];
#pragma unroll
        for (int qg = 0; qg < 2; ++qg)
#pragma unroll
            for (int st = 0; st < 4; ++st) s[qg][st] = v4f{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
        for (int ks = 0; ks < 6; ++ks) {
#pragma unroll
            for (int st = 0; st < 4; ++st) {
                const int row = 16 * st + m;
                const unsigned char* kp =
                    ks < 4 ? Kt + row * 256 + 16 * ((4 * ks + g) ^ m)
                           : Kt + kMhaKP + row * 128 + 16 * ((4 * (ks - 4) + g) ^ ((m >> 1) & 7));
                const bf16x8 kop = *reinterpret_cast<const bf16x8*>(kp);
                s[0][st] = mfma_bf16_16x16x32(kop, qreg[0][ks], s[0][st]);
                s[1][st] = mfma_bf16_16x16x32(kop, qreg[1][ks], s[1][st]);
            }
        }

        bf16x8 pv[2][2];
#pragma unroll
        for (int qg = 0; qg < 2; ++qg) {
            // raw scores (the scale goes into the exponent's fma); positions
            // the row does not select are -inf
            float z[16];
            const uint32_t gm = 0x000F000Fu << (4 * g);
            const bool full = ((mcur[qg].x & gm) == gm) && ((mcur[qg].y & gm) == gm);
            if (__ballot(!full) == 0) {
#pragma unroll
                for (int st = 0; st < 4; ++st)
#pragma unroll
                    for (int i = 0; i < 4; ++i) z[4 * st + i] = s[qg][st][i];
            } else {
#pragma unroll
                for (int st = 0; st < 4; ++st) {
                    const uint32_t word = st < 2 ? mcur[qg].x : mcur[qg].y;
                    const uint32_t nib = (word >> ((16 * st + 4 * g) & 31)) & 0xFu;
#pragma unroll
                    for (int i = 0; i < 4; ++i)
                        z[4 * st + i] = (nib >> i) & 1u ? s[qg][st][i] : -INFINITY;
                }
            }
            float zmax = z[0];
#pragma unroll
            for (int i = 1; i < 16; ++i) zmax = fmaxf(zmax, z[i]);
            zmax = fmaxf(zmax, __shfl_xor(zmax, 16));
            zmax = fmaxf(zmax, __shfl_xor(zmax, 32));
            const float tmax = zmax * scale_log2;
            if (tmax > m_run[qg] + 8.0f) {
                const float corr = (m_run[qg] == -INFINITY) ? 0.0f : exp2f(m_run[qg] - tmax);
                l_run[qg] *= corr;
                m_run[qg] = tmax;
                if (__ballot(corr != 1.0f)) {
#pragma unroll
                    for (int t2 = 0; t2 < 8; ++t2) acc[qg][t2] *= corr;
                }
            }
            // exp2(scale z - m); before any selected position m is -inf and
            // every z is -inf: an offset of 0 keeps p = 0
            const float moff = m_run[qg] == -INFINITY ? 0.0f : -m_run[qg];
            float psum = 0.0f;
#pragma unroll
            for (int kk = 0; kk < 2; ++kk) {
#pragma unroll
                for (int i = 0; i < 8; i += 2) {
                    // k slot 8g + i of the value product: key 32 kk + 4 g + i
                    // (i < 4) or 32 kk + 16 + 4 g + i - 4
                    const float z0 = z[4 * (2 * kk + (i >> 2)) + (i & 3)];
                    const float z1 = z[4 * (2 * kk + (i >> 2)) + (i & 3) + 1];
                    const float p0 = __builtin_amdgcn_exp2f(fmaf(z0, scale_log2, moff));
                    const float p1 = __builtin_amdgcn_exp2f(fmaf(z1, scale_log2, moff));
                    const bf16x2 pb = __builtin_bit_cast(bf16x2, pack_bf16x2(p0, p1));
                    pv[qg][kk][i] = pb[0];
                    pv[qg][kk][i + 1] = pb[1];
                    psum += p0 + p1;
                }
            }
            l_run[qg] += psum;
        }

        // O^T += V^T P^T
#pragma unroll
        for (int kk = 0; kk < 2; ++kk) {
#pragma unroll
            for (int t2 = 0; t2 < 8; ++t2) {
                const int c = 2 * t2 + (q4 >> 1);
                const unsigned char* p = Kt + 32 * kk * 256 + vrow + 16 * (c ^ fv);
                const uint2 lo = __builtin_bit_cast(uint2, lds_read_tr16(reinterpret_cast<const uint16_t*>(p)));
                const uint2 hi = __builtin_bit_cast(uint2, lds_read_tr16(
                    reinterpret_cast<const uint16_t*>(p + 16 * 256)));
                const bf16x8 va = __builtin_bit_cast(bf16x8, make_uint4(lo.x, lo.y, hi.x, hi.y));
                acc[0][t2] = mfma_bf16_16x16x32(va, pv[0][kk], acc[0][t2]);
                acc[1][t2] = mfma_bf16_16x16x32(va, pv[1][kk], acc[1][t2]);
            }
        }
    }

    // lane holds O^T[16 t2 + 4 g + i][row m of group qg]
#pragma unroll
    for (int qg = 0; qg < 2; ++qg) {
        float lr_tot = l_run[qg] + __shfl_xor(l_run[qg], 16);
        lr_tot += __shfl_xor(lr_tot, 32);
        if (!rv[qg]) continue;
        const float inv = lr_tot > 0.0f ? 1.0f / lr_tot : 0.0f;
        uint16_t* oh = out + (rr[qg] * Hq + h) * 128 + 4 * g;
#pragma unroll
        for (int t2 = 0; t2 < 8; ++t2) {
            const uint32_t lo = pack_bf16x2(acc[qg][t2][0] * inv, acc[qg][t2][1] * inv);
            const uint32_t hi = pack_bf16x2(acc[qg][t2][2] * inv, acc[qg][t2][3] * inv);
            *reinterpret_cast<uint2*>(oh + 16 * t2) = make_uint2(lo, hi);
        }
    }
}

// Workspace: bit masks [B*S][2*nkt] words, then (256-byte aligned) the tile
// lists [B*ntq][nkt + 1] of int4.
size_t mha_workspace_bytes(int B, int S, int Lmax) {
    const int64_t nkt = (Lmax + kMhaKeys - 1) / kMhaKeys;
    const int64_t ntq = (S + kMhaRows - 1) / kMhaRows;
    const size_t maskb = static_cast<size_t>(B) * S * 2 * nkt * sizeof(uint32_t);
    const size_t tl = static_cast<size_t>(B) * ntq * (nkt + 1) * sizeof(int4);
    return (maskb + 255) / 256 * 256 + (tl + 255) / 256 * 256 + 256;
}

hipError_t launch_sparse_mha(int B, int S, int Hq, int Lmax, int K, const uint16_t* q,
                             const uint16_t* kv, const uint16_t* rope, int64_t rope_rs,
                             int64_t rope_bs, const int32_t* idx, const int32_t* pos, float scale,
                             uint16_t* out, void* workspace, hipStream_t stream) {
    // more than 64 KiB of dynamic LDS (set once per device)
    const hipError_t attr = set_dynamic_lds_limit(
        reinterpret_cast<const void*>(&sparse_mha_kernel), static_cast<int>(kMhaLds));
    if (attr != hipSuccess) return attr;
    const int nkt = (Lmax + kMhaKeys - 1) / kMhaKeys;
    const int ntq = (S + kMhaRows - 1) / kMhaRows;
    const int nqt = B * ntq;
    const size_t maskb = static_cast<size_t>(B) * S * 2 * nkt * sizeof(uint32_t);
    const size_t tlb = static_cast<size_t>(nqt) * (nkt + 1) * sizeof(int4);
    char* ws = static_cast<char*>(workspace);
    uint32_t* mask = reinterpret_cast<uint32_t*>(ws);
    int4* tiles = reinterpret_cast<int4*>(ws + (maskb + 255) / 256 * 256);
    uint16_t* zeros = reinterpret_cast<uint16_t*>(ws + (maskb + 255) / 256 * 256 + (tlb + 255) / 256 * 256);
    const int nw = 2 * nkt;
    const int64_t nrows = static_cast<int64_t>(B) * S;
    hipLaunchKernelGGL(selection_rows_kernel,
                       dim3(static_cast<unsigned>((nrows + kMaskRowsPerBlock - 1) / kMaskRowsPerBlock)),
                       dim3(kMaskThreads), sizeof(uint32_t) * kMaskRowsPerBlock * nw, stream, S, Lmax,
                       K, nw, nrows, idx, pos, mask, zeros);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(tile_lists_kernel, dim3(static_cast<unsigned>(nqt)), dim3(kMaskThreads),
                       sizeof(uint32_t) * nw, stream, S, nkt, ntq, mask, tiles);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    const float scale_log2 = scale * 1.4426950408889634f;
    hipLaunchKernelGGL(sparse_mha_kernel, dim3(static_cast<unsigned>(nqt * Hq)), dim3(kMhaThreads),
                       kMhaLds, stream, S, Hq, Lmax, nkt, ntq, nqt, q, kv, rope, rope_rs, rope_bs,
                       mask, tiles, zeros, scale_log2, out);
    return hipGetLastError();
}

}  // namespace dsa
