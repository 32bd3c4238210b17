// sparse_mla.hip -- sparse latent attention, absorbed (MQA) form, gfx950.
//
// Method (page "Similarities", MLA decode excerpt; page "Sparse latent
// attention", S' = S m^2/sqrt(192), softmax, O = AV, attention over the
// selected positions alone): for query row r and head h, over the selected
// positions p_j,
//   z_j = scale * (q[h][0:512] . latent[p_j] + q[h][512:576] . rope[p_j])
//   out[h] = sum_j softmax(z)_j latent[p_j],  lse[h] = log sum_j exp(z_j).
//
// Design: one block serves 16*NW heads of one query row over a contiguous
// range ("split") of its selected positions. Selected rows are gathered 32
// at a time into LDS: K tile [32][576] row-major (padded) and a transposed
// copy of the latent part, V^T [512][32]. Per wave (16 heads):
//   S^T = K Q^T       bf16 MFMA 16x16x32, M = keys, N = heads, K = features;
//                     the wave's Q^T operands stay in registers.
//   online softmax    per head (one head per lane column), in log2 units.
//   O^T += V^T P^T    bf16 MFMA, M = 16 latent features, N = heads,
//                     K = the 32 keys; P^T comes straight from the S^T
//                     result registers (the key order inside the MFMA K
//                     dimension is free as long as both operands agree).
// With several splits per row the unnormalised partials (O, m, l) go to the
// workspace and combine_kernel merges them with the log-sum-exp rule.
#include "dsa_common.h"

namespace dsa {

constexpr int kDl = 512, kDr = 64, kDq = 576;
constexpr int kTile = 32;
constexpr int kKtStride = kDq + 8;      // bf16 per K-tile row (1168 B, staggers banks)
constexpr int kVtStride = kTile + 4;    // bf16 per V^T row (72 B)
constexpr size_t kMlaLdsBytes =
    sizeof(uint16_t) * (kTile * kKtStride + kDl * kVtStride) + sizeof(int) * kTile;

template <int NW>
__global__ __launch_bounds__(NW * 64) void sparse_mla_kernel(
    int S, int Hq, int Lmax, int K, int slots_per_split, int nsplit,
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ latent, int64_t lat_rs,
    int64_t lat_bs, const uint16_t* __restrict__ rope, int64_t rope_rs, int64_t rope_bs,
    const int32_t* __restrict__ idx, float scale_log2, uint16_t* __restrict__ out,
    float* __restrict__ lse, float* __restrict__ ws_o, float* __restrict__ ws_ml) {
    extern __shared__ __align__(16) unsigned char smem[];
    uint16_t* Kt = reinterpret_cast<uint16_t*>(smem);
    uint16_t* Vt = Kt + kTile * kKtStride;
    int* tile_pos = reinterpret_cast<int*>(Vt + kDl * kVtStride);

    constexpr int kThreads = NW * 64;
    const int row = blockIdx.y, split = blockIdx.x;
    const int64_t b = row / S;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int m = lane & 15, g = lane >> 4;
    const int h = wave * 16 + m;

    // Q^T operand: lane (n = head h, g) holds q[h][32 ks + 8 g .. +7].
    bf16x8 qreg[kDq / 32];
    {
        const uint16_t* qh = q + (static_cast<int64_t>(row) * Hq + (h < Hq ? h : 0)) * kDq + 8 * g;
#pragma unroll
        for (int ks = 0; ks < kDq / 32; ++ks) {
            uint4 v = *reinterpret_cast<const uint4*>(qh + ks * 32);
            if (h >= Hq) v = make_uint4(0u, 0u, 0u, 0u);
            qreg[ks] = __builtin_bit_cast(bf16x8, v);
        }
    }

    v4f acc[kDl / 16];
#pragma unroll
    for (int t = 0; t < kDl / 16; ++t) acc[t] = v4f{0.0f, 0.0f, 0.0f, 0.0f};
    // l_run sums the float32 probabilities (for lse); lr_run sums the bf16
    // values that actually weight the latent rows (for the normalisation).
    float m_run = -INFINITY, l_run = 0.0f, lr_run = 0.0f;

    const int j_begin = split * slots_per_split;
    const int j_end = min(K, j_begin + slots_per_split);
    const int32_t* irow = idx + static_cast<int64_t>(row) * K;
    const uint16_t* lat_b = latent + b * lat_bs;
    const uint16_t* rope_b = rope + b * rope_bs;

    for (int j0 = j_begin; j0 < j_end; j0 += kTile) {
        __syncthreads();                     // previous tile fully consumed
        if (tid < kTile) {
            const int j = j0 + tid;
            int p = j < j_end ? irow[j] : -1;
            if (p < 0 || p >= Lmax) p = -1;
            tile_pos[tid] = p;
        }
        __syncthreads();
        // gather: 32 rows x 72 chunks of 16 B (64 latent + 8 rope chunks)
        for (int c = tid; c < kTile * 72; c += kThreads) {
            const int key = c / 72, part = c - key * 72;
            const int p = tile_pos[key];
            uint4 v = make_uint4(0u, 0u, 0u, 0u);
            if (p >= 0) {
                const uint16_t* src = part < 64 ? lat_b + p * lat_rs + part * 8
                                                : rope_b + p * rope_rs + (part - 64) * 8;
                v = *reinterpret_cast<const uint4*>(src);
            }
            *reinterpret_cast<uint4*>(Kt + key * kKtStride + part * 8) = v;
        }
        __syncthreads();
        // transposed copy of the latent part: Vt[d][key]
        for (int c = tid; c < kTile * 64; c += kThreads) {
            const int key = c & 31, ch = c >> 5;
            const uint4 v = *reinterpret_cast<const uint4*>(Kt + key * kKtStride + ch * 8);
            const uint32_t w4[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                Vt[(ch * 8 + 2 * e) * kVtStride + key] = static_cast<uint16_t>(w4[e] & 0xFFFFu);
                Vt[(ch * 8 + 2 * e + 1) * kVtStride + key] = static_cast<uint16_t>(w4[e] >> 16);
            }
        }
        __syncthreads();

        // S^T for keys 0..15 (s0) and 16..31 (s1); lane holds keys 4g+i.
        v4f s0 = {0.0f, 0.0f, 0.0f, 0.0f}, s1 = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
        for (int ks = 0; ks < kDq / 32; ++ks) {
            const bf16x8 a0 =
                *reinterpret_cast<const bf16x8*>(Kt + m * kKtStride + ks * 32 + 8 * g);
            const bf16x8 a1 =
                *reinterpret_cast<const bf16x8*>(Kt + (16 + m) * kKtStride + ks * 32 + 8 * g);
            s0 = mfma_bf16_16x16x32(a0, qreg[ks], s0);
            s1 = mfma_bf16_16x16x32(a1, qreg[ks], s1);
        }
        float z[8];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            z[i] = tile_pos[4 * g + i] >= 0 ? s0[i] * scale_log2 : -INFINITY;
            z[4 + i] = tile_pos[16 + 4 * g + i] >= 0 ? s1[i] * scale_log2 : -INFINITY;
        }
        float tmax = z[0];
#pragma unroll
        for (int i = 1; i < 8; ++i) tmax = fmaxf(tmax, z[i]);
        tmax = fmaxf(tmax, __shfl_xor(tmax, 16));
        tmax = fmaxf(tmax, __shfl_xor(tmax, 32));
        const float m_new = fmaxf(m_run, tmax);
        const bool live = m_new != -INFINITY;
        const float corr = live ? exp2f(m_run - m_new) : 1.0f;
        bf16x8 pv;
        float psum = 0.0f, prsum = 0.0f;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const float pe = live ? exp2f(z[i] - m_new) : 0.0f;
            const __bf16 pb = static_cast<__bf16>(pe);
            pv[i] = pb;
            psum += pe;
            prsum += static_cast<float>(pb);
        }
        l_run = l_run * corr + psum;
        lr_run = lr_run * corr + prsum;
        m_run = m_new;
#pragma unroll
        for (int t = 0; t < kDl / 16; ++t) {
            acc[t] *= corr;
            const int d = 16 * t + m;
            const uint2 lo = *reinterpret_cast<const uint2*>(Vt + d * kVtStride + 4 * g);
            const uint2 hi = *reinterpret_cast<const uint2*>(Vt + d * kVtStride + 16 + 4 * g);
            const uint4 v = make_uint4(lo.x, lo.y, hi.x, hi.y);
            acc[t] = mfma_bf16_16x16x32(__builtin_bit_cast(bf16x8, v), pv, acc[t]);
        }
    }

    float l_tot = l_run + __shfl_xor(l_run, 16);
    l_tot += __shfl_xor(l_tot, 32);
    float lr_tot = lr_run + __shfl_xor(lr_run, 16);
    lr_tot += __shfl_xor(lr_tot, 32);
    if (h >= Hq) return;
    if (nsplit == 1) {
        const float inv = lr_tot > 0.0f ? 1.0f / lr_tot : 0.0f;
        uint16_t* oh = out + (static_cast<int64_t>(row) * Hq + h) * kDl + 4 * g;
#pragma unroll
        for (int t = 0; t < kDl / 16; ++t) {
            const uint32_t lo = static_cast<uint32_t>(float_to_bf16_bits(acc[t][0] * inv)) |
                                (static_cast<uint32_t>(float_to_bf16_bits(acc[t][1] * inv)) << 16);
            const uint32_t hi = static_cast<uint32_t>(float_to_bf16_bits(acc[t][2] * inv)) |
                                (static_cast<uint32_t>(float_to_bf16_bits(acc[t][3] * inv)) << 16);
            *reinterpret_cast<uint2*>(oh + 16 * t) = make_uint2(lo, hi);
        }
        if (lse != nullptr && g == 0)
            lse[static_cast<int64_t>(row) * Hq + h] =
                l_tot > 0.0f ? m_run * 0.69314718055994531f + logf(l_tot) : -INFINITY;
    } else {
        const int64_t slot = (static_cast<int64_t>(row) * nsplit + split) * Hq + h;
        float* wo = ws_o + slot * kDl + 4 * g;
#pragma unroll
        for (int t = 0; t < kDl / 16; ++t)
            *reinterpret_cast<float4*>(wo + 16 * t) =
                make_float4(acc[t][0], acc[t][1], acc[t][2], acc[t][3]);
        if (g == 0)
            *reinterpret_cast<float4*>(ws_ml + slot * 4) = make_float4(m_run, l_tot, lr_tot, 0.0f);
    }
}

// Merge of key-split partials: block per (row, head), 128 threads x 4
// features. The (m, l, lr) triples of all splits are staged in LDS first so
// the partial-output loads below are independent and overlap.
constexpr int kMaxSplits = 64;

__global__ __launch_bounds__(128) void combine_kernel(int Hq, int nsplit,
                                                      const float* __restrict__ ws_o,
                                                      const float* __restrict__ ws_ml,
                                                      uint16_t* __restrict__ out,
                                                      float* __restrict__ lse) {
    __shared__ float4 ml[kMaxSplits];
    __shared__ float wgt[kMaxSplits];
    __shared__ float s_M, s_L, s_Lr;
    const int rh = blockIdx.x;
    const int64_t row = rh / Hq;
    const int h = rh - static_cast<int>(row * Hq);
    const int tid = threadIdx.x;
    const int d = tid * 4;
    if (tid < nsplit)
        ml[tid] = *reinterpret_cast<const float4*>(ws_ml + ((row * nsplit + tid) * Hq + h) * 4);
    __syncthreads();
    if (tid < 64) {
        float M = -INFINITY;
        for (int s = tid; s < nsplit; s += 64) M = fmaxf(M, ml[s].x);
#pragma unroll
        for (int o = 32; o >= 1; o >>= 1) M = fmaxf(M, __shfl_xor(M, o));
        float L = 0.0f, Lr = 0.0f;
        for (int s = tid; s < nsplit; s += 64) {
            const float e = (ml[s].x == -INFINITY) ? 0.0f : exp2f(ml[s].x - M);
            wgt[s] = e;
            L += ml[s].y * e;
            Lr += ml[s].z * e;
        }
#pragma unroll
        for (int o = 32; o >= 1; o >>= 1) {
            L += __shfl_xor(L, o);
            Lr += __shfl_xor(Lr, o);
        }
        if (tid == 0) {
            s_M = M;
            s_L = L;
            s_Lr = Lr;
        }
    }
    __syncthreads();
    const float* base = ws_o + (row * nsplit * Hq + h) * kDl + d;
    const int64_t sstride = static_cast<int64_t>(Hq) * kDl;
    float4 acc = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
#pragma unroll 8
    for (int s = 0; s < nsplit; ++s) {
        const float e = wgt[s];
        const float4 v = *reinterpret_cast<const float4*>(base + s * sstride);
        acc.x += e * v.x;
        acc.y += e * v.y;
        acc.z += e * v.z;
        acc.w += e * v.w;
    }
    const float Lr = s_Lr;
    const float inv = Lr > 0.0f ? 1.0f / Lr : 0.0f;
    uint16_t* oh = out + (row * Hq + h) * kDl + d;
    const uint32_t lo = static_cast<uint32_t>(float_to_bf16_bits(acc.x * inv)) |
                        (static_cast<uint32_t>(float_to_bf16_bits(acc.y * inv)) << 16);
    const uint32_t hi = static_cast<uint32_t>(float_to_bf16_bits(acc.z * inv)) |
                        (static_cast<uint32_t>(float_to_bf16_bits(acc.w * inv)) << 16);
    *reinterpret_cast<uint2*>(oh) = make_uint2(lo, hi);
    if (lse != nullptr && tid == 0)
        lse[row * Hq + h] = s_L > 0.0f ? s_M * 0.69314718055994531f + logf(s_L) : -INFINITY;
}

// Split plan: enough (row, split) blocks to occupy the chip, each split a
// whole number of 32-key tiles.
void mla_plan(int rows, int K, int* nsplit, int* slots_per_split) {
    const int tiles = (K + kTile - 1) / kTile;
    int ns = (256 + rows - 1) / rows;
    int cap = tiles >= 2 ? tiles / 2 : 1;
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
    const size_t slots = static_cast<size_t>(rows) * ns * Hq;
    return slots * kDl * sizeof(float) + slots * 4 * sizeof(float) + 256;
}

template <int NW>
static hipError_t launch_mla_nw(dim3 grid, hipStream_t stream, int S, int Hq, int Lmax, int K,
                                int sps, int ns, const uint16_t* q, const uint16_t* latent,
                                int64_t lat_rs, int64_t lat_bs, const uint16_t* rope,
                                int64_t rope_rs, int64_t rope_bs, const int32_t* idx,
                                float scale_log2, uint16_t* out, float* lse, float* ws_o,
                                float* ws_ml) {
    // thread-safe one-time opt-in to more than 64 KiB of dynamic LDS
    static const hipError_t attr = hipFuncSetAttribute(
        reinterpret_cast<const void*>(&sparse_mla_kernel<NW>),
        hipFuncAttributeMaxDynamicSharedMemorySize, static_cast<int>(kMlaLdsBytes));
    if (attr != hipSuccess) return attr;
    hipLaunchKernelGGL((sparse_mla_kernel<NW>), grid, dim3(NW * 64), kMlaLdsBytes, stream, S, Hq,
                       Lmax, K, sps, ns, q, latent, lat_rs, lat_bs, rope, rope_rs, rope_bs, idx,
                       scale_log2, out, lse, ws_o, ws_ml);
    return hipGetLastError();
}

hipError_t launch_sparse_mla(int B, int S, int Hq, int Lmax, int K, const uint16_t* q,
                             const uint16_t* latent, int64_t lat_rs, int64_t lat_bs,
                             const uint16_t* rope, int64_t rope_rs, int64_t rope_bs,
                             const int32_t* idx, float scale, uint16_t* out, float* lse,
                             void* workspace, hipStream_t stream) {
    const int rows = B * S;
    int ns, sps;
    mla_plan(rows, K, &ns, &sps);
    float* ws_o = nullptr;
    float* ws_ml = nullptr;
    if (ns > 1) {
        ws_o = static_cast<float*>(workspace);
        ws_ml = ws_o + static_cast<size_t>(rows) * ns * Hq * kDl;
    }
    const float scale_log2 = scale * 1.4426950408889634f;
    const dim3 grid(ns, rows);
    const int nw = (Hq + 15) / 16;
    hipError_t e;
#define DSA_MLA(NWV)                                                                           \
    e = launch_mla_nw<NWV>(grid, stream, S, Hq, Lmax, K, sps, ns, q, latent, lat_rs, lat_bs,   \
                           rope, rope_rs, rope_bs, idx, scale_log2, out, lse, ws_o, ws_ml)
    if (nw <= 1) DSA_MLA(1);
    else if (nw <= 2) DSA_MLA(2);
    else if (nw <= 4) DSA_MLA(4);
    else DSA_MLA(8);
#undef DSA_MLA
    if (e != hipSuccess) return e;
    if (ns > 1) {
        hipLaunchKernelGGL(combine_kernel, dim3(rows * Hq), dim3(128), 0, stream, Hq, ns, ws_o,
                           ws_ml, out, lse);
        e = hipGetLastError();
    }
    return e;
}

}  // namespace dsa
