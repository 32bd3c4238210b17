// mla_append.hip -- MLA-side cache append for gfx950.
//
// Method (page "DeepSeek-V3.2-Exp . RoPE coefficients", MLA prefill
// excerpt: the new latent rows go to the latent cache and the rotated
// rotary keys to the rope cache at their positions; aipricedb update note
// of 2025.11.17: the MLA rotary embedding pairs features 2j and 2j+1, the
// indexer's j and j+32): for query row r = (b, s) at position p,
//   latent[b][p][:]  = latent_new[r][:]                      (bf16 copy)
//   rope[b][p][2j], rope[b][p][2j+1] = bf16(a c - b s), bf16(a s + b c)
// with (a, b) = kpe_new[r][2j], kpe_new[r][2j+1] and (c, s) the table entry
// (p, j); products and the sum or difference each rounded in float32 (no
// fused multiply-add). Optionally the rope part q[r][h][512:576] of every
// head is rotated in place the same way.
//
// One block of 256 threads per query row: 64 threads copy the 1 KiB latent
// row (16 B each), 32 threads rotate the rotary key (one pair each), and all
// threads rotate the query heads' pairs (Hq x 32 pairs).
#include "dsa_common.h"

namespace dsa {

__device__ __forceinline__ uint32_t rotate_pair_bf16(uint32_t ab, float c, float s) {
#pragma clang fp contract(off)
    const float a = bf16_bits_to_float(static_cast<uint16_t>(ab & 0xFFFFu));
    const float b = bf16_bits_to_float(static_cast<uint16_t>(ab >> 16));
    const float ac = a * c, bs = b * s, as = a * s, bc = b * c;
    const float ya = ac - bs, yb = as + bc;
    return static_cast<uint32_t>(float_to_bf16_bits(ya)) |
           (static_cast<uint32_t>(float_to_bf16_bits(yb)) << 16);
}

__global__ __launch_bounds__(256) void mla_append_kernel(
    int S, int Hq, int Lmax, int P, const uint16_t* __restrict__ latent_new,
    const uint16_t* __restrict__ kpe_new, const int32_t* __restrict__ pos,
    const float* __restrict__ cos_t, const float* __restrict__ sin_t,
    uint16_t* __restrict__ latent, int64_t lat_rs, int64_t lat_bs, uint16_t* __restrict__ rope,
    int64_t rope_rs, int64_t rope_bs, uint16_t* __restrict__ q, CacheMap cmap) {
    const int64_t r = blockIdx.x;
    const int tid = threadIdx.x;
    const int p = pos[r];
    if (p < 0 || p >= Lmax || p >= P) return;
    const int64_t b = r / S;
    // cache row of (b, p): dense strides, or the pool row of p's page
    int64_t lat_off, rope_off;
    bool present = true;
    if (cmap.table == nullptr) {
        lat_off = b * lat_bs + static_cast<int64_t>(p) * lat_rs;
        rope_off = b * rope_bs + static_cast<int64_t>(p) * rope_rs;
    } else {
        const int64_t prow = cmap.row(b, p);
        present = prow >= 0;                         // no page: no cache write
        lat_off = prow * lat_rs;
        rope_off = prow * rope_rs;
    }
    if (present && tid < 64) {
        const uint4 v = reinterpret_cast<const uint4*>(latent_new + r * 512)[tid];
        reinterpret_cast<uint4*>(latent + lat_off)[tid] = v;
    }
    const float* cr = cos_t + static_cast<int64_t>(p) * 32;
    const float* sr = sin_t + static_cast<int64_t>(p) * 32;
    if (present && tid >= 64 && tid < 96) {
        const int j = tid - 64;
        const uint32_t ab = reinterpret_cast<const uint32_t*>(kpe_new + r * 64)[j];
        reinterpret_cast<uint32_t*>(rope + rope_off)[j] = rotate_pair_bf16(ab, cr[j], sr[j]);
    }
    if (q != nullptr) {
        for (int i = tid; i < Hq * 32; i += 256) {
            const int h = i >> 5, j = i & 31;
            uint32_t* qp = reinterpret_cast<uint32_t*>(q + (r * Hq + h) * 576 + 512) + j;
            *qp = rotate_pair_bf16(*qp, cr[j], sr[j]);
        }
    }
}

hipError_t launch_mla_append(int B, int S, int Hq, int Lmax, int P, const uint16_t* latent_new,
                             const uint16_t* kpe_new, const int32_t* pos, const float* cos_t,
                             const float* sin_t, uint16_t* latent, int64_t lat_rs, int64_t lat_bs,
                             uint16_t* rope, int64_t rope_rs, int64_t rope_bs, uint16_t* q,
                             CacheMap cmap, hipStream_t stream) {
    const int64_t rows = static_cast<int64_t>(B) * S;
    hipLaunchKernelGGL(mla_append_kernel, dim3(static_cast<unsigned>(rows)), dim3(256), 0, stream,
                       S, Hq, Lmax, P, latent_new, kpe_new, pos, cos_t, sin_t, latent, lat_rs,
                       lat_bs, rope, rope_rs, rope_bs, q, cmap);
    return hipGetLastError();
}

}  // namespace dsa
