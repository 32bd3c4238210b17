// mla_proj.hip -- the MLA projections around the attention, gfx950:
// the key/value up-projection of the multi-head prefill form and the two
// absorption products of the absorbed form.
//
// Method (page "RoPE coefficients", MLA prefill excerpt: wkv_b applied to
// the latent rows and viewed per head as a 128-feature non-rotary key then a
// 128-feature value; page "Similarities", MQA decode excerpt: the query's
// non-rotary part times W_UK[h] gives a 512-feature latent query, and the
// latent attention output times W_UV[h]^T gives the head's value output).
// wkv_b is [Hq][256][512]: rows 0..127 of head h are W_UK[h], rows 128..255
// W_UV[h].
//
// All three are bf16 matrix products with float32 accumulation, run by one
// tiled MFMA kernel computing C[z] = A[z] B[z]^T over a batch z:
//   kv_up     A = latent rows [rows][512], B = wkv_b as [Hq*256][512]   (B is N x K)
//   absorb_q  per (b, h): A = q_nope [rows][128], B = W_UK[h] [128][512] (B is K x N)
//   absorb_o  per (b, h): A = x [rows][512],      B = W_UV[h] [128][512] (B is N x K)
// Block tile 128 x 128 x 64, 4 waves of 64 x 64 (4 x 4 MFMA 16x16x32
// tiles); A and B tiles pass through double-buffered LDS, the next k-slice
// is loaded into registers while the current one is multiplied. Each MFMA
// computes a tile of C^T (B rows as the first operand), so a lane ends with
// four consecutive output columns of one row: 8-byte stores. A B operand
// stored K x N is read column-wise from its row-major LDS tile by the
// transposing LDS read.
#include "dsa_common.h"

namespace dsa {

constexpr int kGM = 128, kGN = 128, kGK = 64;
constexpr int kGThreads = 256;
constexpr int kGAStride = kGK + 8;      // bf16 per LDS row of an A (or N x K B) tile
constexpr int kGBnStride = kGN + 8;     // bf16 per LDS row of a K x N B tile
constexpr size_t kGemmLds =
    sizeof(uint16_t) * 2 * (kGM * kGAStride + kGN * kGAStride);   // both buffers, both tiles

struct GemmArgs {
    int M, N, K;
    int zdiv;                         // batch z -> (z / zdiv, z % zdiv)
    int mtiles;
    const uint16_t* A;
    int64_t lda, a_s1, a_s2;          // element offsets per z / zdiv and z % zdiv
    const uint16_t* B;
    int64_t ldb, b_s1, b_s2;
    uint16_t* C;
    int64_t ldc, c_s1, c_s2;
};

template <bool B_KN>
__global__ __launch_bounds__(kGThreads, 2) void gemm_bf16_kernel(GemmArgs a) {
    extern __shared__ __align__(16) unsigned char smem[];
    uint16_t* As = reinterpret_cast<uint16_t*>(smem);                 // [2][128][72]
    uint16_t* Bs = As + 2 * kGM * kGAStride;                          // [2][128][72] / [2][64][136]
    constexpr int kBBuf = B_KN ? kGK * kGBnStride : kGN * kGAStride;

    const int z = blockIdx.y;
    const int z1 = z / a.zdiv, z2 = z - z1 * a.zdiv;
    const int mt = blockIdx.x % a.mtiles, nt = blockIdx.x / a.mtiles;
    const int m0 = mt * kGM, n0 = nt * kGN;
    const uint16_t* A = a.A + z1 * a.a_s1 + z2 * a.a_s2;
    const uint16_t* B = a.B + z1 * a.b_s1 + z2 * a.b_s2;
    uint16_t* C = a.C + z1 * a.c_s1 + z2 * a.c_s2;

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wm = wave >> 1, wn = wave & 1;
    const int m = lane & 15, g = lane >> 4;

    // Staging: A (and an N x K B) rows tid/8 + 32 i, 8 elements at (tid%8)*8;
    // a K x N B: k-rows tid/16 + 16 i, 8 columns at (tid%16)*8. Rows of A
    // past M are zero.
    const int ar = tid >> 3, ac = (tid & 7) * 8;
    const int br = tid >> 4, bc = (tid & 15) * 8;
    const uint16_t* arow[4];
    bool aval[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int row = m0 + ar + 32 * i;
        aval[i] = row < a.M;
        arow[i] = A + static_cast<int64_t>(aval[i] ? row : 0) * a.lda + ac;
    }
    u32x4 ga[4], gb[4];
    auto load = [&](int k0) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            ga[i] = *reinterpret_cast<const u32x4*>(arow[i] + k0);   // row 0 past M
            if (!aval[i]) ga[i] = u32x4{0u, 0u, 0u, 0u};
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            if (!B_KN)
                gb[i] = *reinterpret_cast<const u32x4*>(
                    B + static_cast<int64_t>(n0 + ar + 32 * i) * a.ldb + k0 + ac);
            else
                gb[i] = *reinterpret_cast<const u32x4*>(
                    B + static_cast<int64_t>(k0 + br + 16 * i) * a.ldb + n0 + bc);
        }
    };
    auto store = [&](int buf) {
        uint16_t* as = As + buf * kGM * kGAStride;
        uint16_t* bs = Bs + buf * kBBuf;
#pragma unroll
        for (int i = 0; i < 4; ++i)
            *reinterpret_cast<u32x4*>(as + (ar + 32 * i) * kGAStride + ac) = ga[i];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            if (!B_KN)
                *reinterpret_cast<u32x4*>(bs + (ar + 32 * i) * kGAStride + ac) = gb[i];
            else
                *reinterpret_cast<u32x4*>(bs + (br + 16 * i) * kGBnStride + bc) = gb[i];
        }
    };

    v4f acc[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = v4f{0.0f, 0.0f, 0.0f, 0.0f};

    // transposing-read address inside a 4 x 16 block (K x N tiles)
    const int tr_off = ((lane >> 2) & 3) * kGBnStride + 4 * (lane & 3);
    const int nk = a.K / kGK;
    load(0);
    store(0);
    __syncthreads();
    for (int kt = 0; kt < nk; ++kt) {
        const int buf = kt & 1;
        // the last step reloads its own slice (no branch around the loads)
        load(min(kt + 1, nk - 1) * kGK);
        const uint16_t* as = As + buf * kGM * kGAStride;
        const uint16_t* bs = Bs + buf * kBBuf;
#pragma unroll
        for (int ks = 0; ks < kGK / 32; ++ks) {
            bf16x8 av[4], bv[4];
#pragma unroll
            for (int i = 0; i < 4; ++i)
                av[i] = *reinterpret_cast<const bf16x8*>(as + (64 * wm + 16 * i + m) * kGAStride +
                                                         32 * ks + 8 * g);
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                if (!B_KN) {
                    bv[j] = *reinterpret_cast<const bf16x8*>(
                        bs + (64 * wn + 16 * j + m) * kGAStride + 32 * ks + 8 * g);
                } else {
                    // lane (column n, group g) gets k = 8g..8g+3, then 8g+4..8g+7
                    const uint16_t* p = bs + (32 * ks + 8 * g) * kGBnStride + 64 * wn + 16 * j + tr_off;
                    const uint2 lo = __builtin_bit_cast(uint2, lds_read_tr16(p));
                    const uint2 hi = __builtin_bit_cast(uint2, lds_read_tr16(p + 4 * kGBnStride));
                    bv[j] = __builtin_bit_cast(bf16x8, make_uint4(lo.x, lo.y, hi.x, hi.y));
                }
            }
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int j = 0; j < 4; ++j) acc[i][j] = mfma_bf16_16x16x32(bv[j], av[i], acc[i][j]);
        }
        store(buf ^ 1);
        __syncthreads();
    }

    // lane holds C[64 wm + 16 i + m][64 wn + 16 j + 4 g + 0..3]
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int row = m0 + 64 * wm + 16 * i + m;
        if (row >= a.M) continue;
        uint16_t* crow = C + static_cast<int64_t>(row) * a.ldc + n0 + 64 * wn + 4 * g;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const uint32_t lo = pack_bf16x2(acc[i][j][0], acc[i][j][1]);
            const uint32_t hi = pack_bf16x2(acc[i][j][2], acc[i][j][3]);
            *reinterpret_cast<uint2*>(crow + 16 * j) = make_uint2(lo, hi);
        }
    }
}

template <bool B_KN>
static hipError_t run_gemm(const GemmArgs& a, int nbatch, hipStream_t stream) {
    static const hipError_t attr = hipFuncSetAttribute(
        reinterpret_cast<const void*>(&gemm_bf16_kernel<B_KN>),
        hipFuncAttributeMaxDynamicSharedMemorySize, static_cast<int>(kGemmLds));
    if (attr != hipSuccess) return attr;
    const int ntiles = a.N / kGN;
    hipLaunchKernelGGL(gemm_bf16_kernel<B_KN>, dim3(static_cast<unsigned>(a.mtiles * ntiles),
                                                    static_cast<unsigned>(nbatch)),
                       dim3(kGThreads), kGemmLds, stream, a);
    return hipGetLastError();
}

// mode 0: kv_up, 1: absorb_q, 2: absorb_o (argument checks are the caller's)
hipError_t launch_mla_proj(int mode, int B, int rows, int Hq, const uint16_t* wkv_b,
                           const uint16_t* x, int64_t xrs, int64_t xbs, int64_t xhs, uint16_t* y,
                           int64_t yrs, int64_t ybs, int64_t yhs, hipStream_t stream) {
    GemmArgs a{};
    a.M = rows;
    a.mtiles = (rows + kGM - 1) / kGM;
    a.A = x;
    a.lda = xrs;
    a.C = y;
    a.ldc = yrs;
    a.ldb = 512;
    if (mode == 0) {
        a.N = Hq * 256;
        a.K = 512;
        a.zdiv = 1;
        a.a_s1 = xbs;
        a.B = wkv_b;
        a.c_s1 = ybs;
        return run_gemm<false>(a, B, stream);
    }
    a.zdiv = Hq;
    a.a_s1 = xbs;
    a.a_s2 = xhs;
    a.c_s1 = ybs;
    a.c_s2 = yhs;
    a.b_s2 = 256 * 512;
    if (mode == 1) {
        a.N = 512;
        a.K = 128;
        a.B = wkv_b;                      // W_UK[h]: [128 (k)][512 (n)]
        return run_gemm<true>(a, B * Hq, stream);
    }
    a.N = 128;
    a.K = 512;
    a.B = wkv_b + 128 * 512;              // W_UV[h]: [128 (n)][512 (k)]
    return run_gemm<false>(a, B * Hq, stream);
}

}  // namespace dsa
