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
// Block tile 128 x 128, 4 waves of 64 x 64 (4 x 4 MFMA 16x16x32 tiles),
// k-slices of 32. The slices stream through a ring of LDS stages filled
// straight from global memory (global_load_lds, 16 bytes per lane, no
// registers), the next slice loading while the current one is multiplied;
// raw barriers and explicit vector-memory waits order them. (Two stages
// leave room for four blocks per CU, which hides more latency than a
// deeper ring.)
// Tiles are stored with XOR-swizzled 16-byte chunks so the operand reads
// of one MFMA hit distinct banks. Each MFMA computes a tile of C^T (B rows
// as the first operand), so a lane ends with four consecutive output
// columns of one row; the bf16 tile is staged through LDS and written in
// 16-byte pieces, whole 256-byte rows per 16 threads. A B operand stored
// K x N is read column-wise by the transposing LDS read.
#include "dsa_common.h"

namespace dsa {

constexpr int kGM = 128, kGN = 128, kGK = 32;
constexpr int kGStages = 2;                          // k-slices in the LDS ring
constexpr int kGThreads = 256;
constexpr int kGTileBytes = 128 * kGK * 2;           // one 128 x 32 (or 32 x 128) bf16 tile
constexpr int kGStageBytes = 2 * kGTileBytes;        // A tile + B tile
constexpr size_t kGCTileBytes = sizeof(uint16_t) * kGM * (kGN + 8);   // staged output tile
constexpr size_t kGemmLds = static_cast<size_t>(kGStages) * kGStageBytes > kGCTileBytes
                                ? static_cast<size_t>(kGStages) * kGStageBytes
                                : kGCTileBytes;
constexpr int kGLoads = 4;                           // 16-byte loads per thread per slice

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

// MODE 0: kv up-projection, 1: query absorption (B stored K x N),
// 2: output absorption; one instantiation each, so profiles tell them apart
template <int MODE>
__global__ __launch_bounds__(kGThreads, 2) void gemm_bf16_kernel(GemmArgs a) {
    constexpr bool B_KN = MODE == 1;
    extern __shared__ __align__(16) unsigned char smem[];

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

    // LDS tiles, filled straight from global memory (lane l of a wave
    // instruction writes bytes 16 l .. 16 l + 15 of that instruction's 1 KiB).
    //  - 128 x 32 tiles (A; B stored N x K): 64-byte rows of four 16-byte
    //    chunks, chunk c of row r at position c ^ (2 ((r >> 2) & 1)).
    //    Instruction j of wave w fills rows 16 (4 j + w) .. +15.
    //  - 32 x 128 tiles (B stored K x N): 256-byte rows of sixteen chunks,
    //    chunk c of row r at position c ^ (2 (r & 3)) ^ (8 ((r >> 3) & 1));
    //    instruction j of wave w fills rows 4 (4 j + w) .. +3.
    //  Both keep every operand read free of LDS bank conflicts on gfx950
    //  (the bank-conflict counter of a probe of each access pattern reads
    //  zero; the earlier swizzles, c ^ ((r >> 2) & 3) and c ^ (2 (r & 3)),
    //  cost one extra cycle per read).
    // Source addresses of this thread's four loads (k offset added per slice);
    // A rows past M load row M - 1 (their products are never stored).
    const uint16_t* srcA[2];
    const uint16_t* srcB[2];
#pragma unroll
    for (int j = 0; j < 2; ++j) {
        const int r = 16 * (4 * j + wave) + (lane >> 2), p = lane & 3;
        const int c = p ^ (2 * ((r >> 2) & 1));
        srcA[j] = A + static_cast<int64_t>(min(m0 + r, a.M - 1)) * a.lda + 8 * c;
        if (!B_KN) {
            srcB[j] = B + static_cast<int64_t>(n0 + r) * a.ldb + 8 * c;
        } else {
            const int kr = 4 * (4 * j + wave) + (lane >> 4), pb = lane & 15;
            srcB[j] = B + static_cast<int64_t>(kr) * a.ldb + n0 +
                      8 * (pb ^ (2 * (kr & 3)) ^ (8 * ((kr >> 3) & 1)));
        }
    }
    auto issue = [&](int kt) {
        unsigned char* st = smem + (kt % kGStages) * kGStageBytes;
        const int64_t kA = static_cast<int64_t>(kt) * kGK;
        const int64_t kB = B_KN ? kA * a.ldb : kA;
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            load_to_lds(srcA[j] + kA, st + (4 * j + wave) * 1024);
            load_to_lds(srcB[j] + kB, st + kGTileBytes + (4 * j + wave) * 1024);
        }
    };

    v4f acc[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = v4f{0.0f, 0.0f, 0.0f, 0.0f};

    // operand read offsets (bytes within a stage)
    const int swzA = 2 * ((m >> 2) & 1);
    const int offA = (64 * wm + m) * 64 + 16 * (g ^ swzA);            // + 16 i rows: + 1024 i
    const int offBnt = kGTileBytes + (64 * wn + m) * 64 + 16 * (g ^ swzA);
    // K x N: lane 4e + q of group g reads row 8g + e (and 8g + 4 + e),
    // columns 64 wn + 16 j + 4q: chunk 8 wn + 2 j + q / 2, half q % 2
    const int e = (lane >> 2) & 3, q = lane & 3;
    const int offBkn = kGTileBytes + (8 * g + e) * 256 + 8 * (q & 1);
    const int cBkn = 8 * wn + (q >> 1);

    const int nk = a.K / kGK;
#pragma unroll
    for (int s = 0; s < kGStages - 1; ++s)
        if (s < nk) issue(s);
    for (int kt = 0; kt < nk; ++kt) {
        // slice kt has landed once at most (stages - 2) later slices are in flight
        if (kt + kGStages - 2 < nk) wait_vmcnt<kGLoads * (kGStages - 2)>();
        else wait_vmcnt<0>();
        __builtin_amdgcn_s_barrier();
        if (kt + kGStages - 1 < nk) issue(kt + kGStages - 1);
        const unsigned char* st = smem + (kt % kGStages) * kGStageBytes;
        bf16x8 av[4], bv[4];
#pragma unroll
        for (int i = 0; i < 4; ++i)
            av[i] = *reinterpret_cast<const bf16x8*>(st + offA + 1024 * i);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            if (!B_KN) {
                bv[j] = *reinterpret_cast<const bf16x8*>(st + offBnt + 1024 * j);
            } else {
                const int pos = (cBkn + 2 * j) ^ (2 * e) ^ (8 * (g & 1));
                const uint16_t* p = reinterpret_cast<const uint16_t*>(st + offBkn + 16 * pos);
                const uint2 lo = __builtin_bit_cast(uint2, lds_read_tr16(p));
                const uint2 hi = __builtin_bit_cast(uint2, lds_read_tr16(p + 4 * 128));
                bv[j] = __builtin_bit_cast(bf16x8, make_uint4(lo.x, lo.y, hi.x, hi.y));
            }
        }
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int j = 0; j < 4; ++j) acc[i][j] = mfma_bf16_16x16x32(bv[j], av[i], acc[i][j]);
    }

    // Epilogue through LDS: lane holds C[64 wm + 16 i + m][64 wn + 16 j + 4 g + 0..3];
    // the bf16 tile goes to LDS ([128][128 + 8]) and leaves in 16-byte
    // pieces, 16 threads per 256-byte row (whole cache lines per store),
    // streamed past L2 (query absorption: 224 -> 130 us for its 537 MB)
    constexpr int kCS = kGN + 8;
    static_assert(sizeof(uint16_t) * kGM * kCS <= kGemmLds, "output tile fits the LDS");
    __builtin_amdgcn_s_barrier();                  // every wave done with the ring
    uint16_t* ct = reinterpret_cast<uint16_t*>(smem);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int r = 64 * wm + 16 * i + m;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const uint32_t lo = pack_bf16x2(acc[i][j][0], acc[i][j][1]);
            const uint32_t hi = pack_bf16x2(acc[i][j][2], acc[i][j][3]);
            *reinterpret_cast<uint2*>(ct + r * kCS + 64 * wn + 16 * j + 4 * g) = make_uint2(lo, hi);
        }
    }
    __syncthreads();
    const int cr = tid >> 4, cc = (tid & 15) * 8;
#pragma unroll
    for (int p = 0; p < kGM / 16; ++p) {
        const int r = 16 * p + cr;
        const int row = m0 + r;
        if (row < a.M)
            __builtin_nontemporal_store(*reinterpret_cast<const u32x4*>(ct + r * kCS + cc),
                                        reinterpret_cast<u32x4*>(C + static_cast<int64_t>(row) * a.ldc + n0 + cc));
    }
}

template <int MODE>
static hipError_t run_gemm(const GemmArgs& a, int nbatch, hipStream_t stream) {
    // more than 64 KiB of dynamic LDS (set once per device)
    const hipError_t attr = set_dynamic_lds_limit(
        reinterpret_cast<const void*>(&gemm_bf16_kernel<MODE>), static_cast<int>(kGemmLds));
    if (attr != hipSuccess) return attr;
    const int ntiles = a.N / kGN;
    hipLaunchKernelGGL(gemm_bf16_kernel<MODE>, dim3(static_cast<unsigned>(a.mtiles * ntiles),
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
        return run_gemm<0>(a, B, stream);
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
        return run_gemm<1>(a, B * Hq, stream);
    }
    a.N = 128;
    a.K = 512;
    a.B = wkv_b + 128 * 512;              // W_UV[h]: [128 (n)][512 (k)]
    return run_gemm<2>(a, B * Hq, stream);
}

}  // namespace dsa
