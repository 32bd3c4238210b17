// dsa_common.h -- device helpers shared by the gfx950 kernels of the DSA
// library (internal header; not part of the C ABI).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace dsa {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
// 16-byte staging register (a native vector: copies stay in registers)
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kWave = 64;

// Opt a kernel in to `bytes` of dynamic LDS (above the 64 KiB default) on
// the current device. The attribute is per device, so it is set once for
// each (kernel, device) pair that launches; a small table under a mutex
// remembers which pairs are done (host code only).
hipError_t set_dynamic_lds_limit(const void* kernel, int bytes);

// ---- bf16 <-> float ------------------------------------------------------
__device__ __forceinline__ float bf16_bits_to_float(uint16_t b) {
    return __uint_as_float(static_cast<uint32_t>(b) << 16);
}

// Round a finite float to the nearest bf16 (ties to even); returns the bits.
__device__ __forceinline__ uint16_t float_to_bf16_bits(float f) {
    uint32_t u = __float_as_uint(f);
    u += 0x7FFFu + ((u >> 16) & 1u);
    return static_cast<uint16_t>(u >> 16);
}

// Two floats to packed bf16 (lo in bits 0..15), rounded to nearest even by
// the hardware conversion (v_cvt_pk_bf16_f32).
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
    bf16x2 r;
    r[0] = static_cast<__bf16>(lo);
    r[1] = static_cast<__bf16>(hi);
    return __builtin_bit_cast(uint32_t, r);
}

// ---- OCP E4M3 encoding (round to nearest even, saturating at 448) --------
// The code is the hardware conversion v_cvt_pk_fp8_f32 (OCP E4M3 on gfx950,
// round to nearest even) of the input clamped to [-448, 448]. For every
// float32 of magnitude at most 464 the hardware result equals the bit-level
// definition: normal outputs round the 23-bit mantissa to 3 bits half-to-even
// (a carry bumps the exponent) and re-bias the exponent from 127 to 7,
// saturating at 0x7E (448); outputs below 2^-6 are the subnormal multiples
// of 2^-9, rint(|v| * 512); the sign is kept (checked exhaustively on the
// device). The clamp supplies the saturation above 448.
__device__ __forceinline__ float e4m3_clamp(float v) {
    return __builtin_amdgcn_fmed3f(v, -448.0f, 448.0f);
}

__device__ __forceinline__ uint8_t e4m3_encode(float v) {
    const float c = e4m3_clamp(v);
    return static_cast<uint8_t>(__builtin_amdgcn_cvt_pk_fp8_f32(c, c, 0, false) & 0xFF);
}

// Four codes packed little-endian into one word (two conversions).
__device__ __forceinline__ uint32_t e4m3_encode4(float a, float b, float c, float d) {
    int w = __builtin_amdgcn_cvt_pk_fp8_f32(e4m3_clamp(a), e4m3_clamp(b), 0, false);
    w = __builtin_amdgcn_cvt_pk_fp8_f32(e4m3_clamp(c), e4m3_clamp(d), w, true);
    return static_cast<uint32_t>(w);
}

// Quotients x / s rounded to nearest (the float32 division) for the E4M3
// codes above. With a normal, finite s, y = 1 / s (itself the rounded
// quotient) gives each one in four instructions instead of the division
// sequence: q0 = x y is within an ulp of x / s, the fma residual x - q0 s is
// exact, and q0 + (x - q0 s) y rounded once is the correctly rounded quotient
// (Markstein's division theorem); the sign is x's, which also keeps -0 / s
// at -0 (the residual step alone would give +0). Other s take the division.
__device__ __forceinline__ float quotient_rn(float x, float s, float y) {
    const float q0 = x * y;
    return copysignf(__builtin_fmaf(__builtin_fmaf(-q0, s, x), y, q0), x);
}
__device__ __forceinline__ bool quotient_fast(float s) {
    return s >= 1.17549435e-38f && s < INFINITY;       // normal, finite
}

// ---- wave reductions (wave64) ---------------------------------------------
__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) v = fmaxf(v, __shfl_xor(v, o));
    return v;
}

// DPP lane moves. `old` is what a lane keeps when its source lane is outside
// the row (row_shr) or its row is masked off (row_bcast).
constexpr int kDppRowShr1 = 0x111, kDppRowShr2 = 0x112, kDppRowShr4 = 0x114,
              kDppRowShr8 = 0x118, kDppRowBcast15 = 0x142, kDppRowBcast31 = 0x143;
template <int CTRL, int ROW_MASK>
__device__ __forceinline__ int dpp_move(int old, int v) {
    return __builtin_amdgcn_update_dpp(old, v, CTRL, ROW_MASK, 0xF, false);
}

// Inclusive prefix sum over the 64 lanes: shifts by 1, 2, 4, 8 inside each
// 16-lane row, then the last lane of row 0 (of rows 0-1) is broadcast into
// rows 1 and 3 (rows 2 and 3).
__device__ __forceinline__ int wave_incl_scan_add(int x) {
    x += dpp_move<kDppRowShr1, 0xF>(0, x);
    x += dpp_move<kDppRowShr2, 0xF>(0, x);
    x += dpp_move<kDppRowShr4, 0xF>(0, x);
    x += dpp_move<kDppRowShr8, 0xF>(0, x);
    x += dpp_move<kDppRowBcast15, 0xA>(0, x);
    x += dpp_move<kDppRowBcast31, 0xC>(0, x);
    return x;
}

// Max / min of a float over the wave, returned to every lane (the same
// prefix pattern with max/min, then lane 63 read back as a scalar).
__device__ __forceinline__ float wave_max_dpp(float v) {
    constexpr int kNegInf = static_cast<int>(0xFF800000u);
    int x = __float_as_int(v);
    x = __float_as_int(fmaxf(__int_as_float(x), __int_as_float(dpp_move<kDppRowShr1, 0xF>(kNegInf, x))));
    x = __float_as_int(fmaxf(__int_as_float(x), __int_as_float(dpp_move<kDppRowShr2, 0xF>(kNegInf, x))));
    x = __float_as_int(fmaxf(__int_as_float(x), __int_as_float(dpp_move<kDppRowShr4, 0xF>(kNegInf, x))));
    x = __float_as_int(fmaxf(__int_as_float(x), __int_as_float(dpp_move<kDppRowShr8, 0xF>(kNegInf, x))));
    x = __float_as_int(fmaxf(__int_as_float(x), __int_as_float(dpp_move<kDppRowBcast15, 0xA>(kNegInf, x))));
    x = __float_as_int(fmaxf(__int_as_float(x), __int_as_float(dpp_move<kDppRowBcast31, 0xC>(kNegInf, x))));
    return __int_as_float(__builtin_amdgcn_readlane(x, 63));
}

__device__ __forceinline__ float wave_min_dpp(float v) { return -wave_max_dpp(-v); }

// Sum of a float over the wave, returned to every lane (same lane moves).
__device__ __forceinline__ float wave_sum_dpp(float v) {
    int x = __float_as_int(v);
    x = __float_as_int(__int_as_float(x) + __int_as_float(dpp_move<kDppRowShr1, 0xF>(0, x)));
    x = __float_as_int(__int_as_float(x) + __int_as_float(dpp_move<kDppRowShr2, 0xF>(0, x)));
    x = __float_as_int(__int_as_float(x) + __int_as_float(dpp_move<kDppRowShr4, 0xF>(0, x)));
    x = __float_as_int(__int_as_float(x) + __int_as_float(dpp_move<kDppRowShr8, 0xF>(0, x)));
    x = __float_as_int(__int_as_float(x) + __int_as_float(dpp_move<kDppRowBcast15, 0xA>(0, x)));
    x = __float_as_int(__int_as_float(x) + __int_as_float(dpp_move<kDppRowBcast31, 0xC>(0, x)));
    return __int_as_float(__builtin_amdgcn_readlane(x, 63));
}

// Exact conversion of four packed E4M3 bytes to four bf16 values.
__device__ __forceinline__ void e4m3x4_to_bf16(uint32_t packed, bf16x2& lo, bf16x2& hi) {
    lo = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(packed, 1.0f, false);
    hi = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(packed, 1.0f, true);
}

__device__ __forceinline__ bf16x8 e4m3x8_to_bf16x8(uint32_t w0, uint32_t w1) {
    bf16x2 a, b, c, d;
    e4m3x4_to_bf16(w0, a, b);
    e4m3x4_to_bf16(w1, c, d);
    bf16x8 r;
    r[0] = a[0]; r[1] = a[1]; r[2] = b[0]; r[3] = b[1];
    r[4] = c[0]; r[5] = c[1]; r[6] = d[0]; r[7] = d[1];
    return r;
}

// Transposing LDS read ds_read_b64_tr_b16 (gfx950). Within each 16-lane
// group, lane 4e+q passes the address of elements 4q..4q+3 of row e of a
// 4 x 16 block of 16-bit elements; lane i receives column i of rows 0..3.
typedef short v4s __attribute__((ext_vector_type(4)));
__device__ __forceinline__ v4s lds_read_tr16(const uint16_t* p) {
    typedef __attribute__((address_space(3))) v4s lds_v4s;
    return __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        reinterpret_cast<lds_v4s*>(reinterpret_cast<__attribute__((address_space(3))) char*>(
            static_cast<uint32_t>(reinterpret_cast<uintptr_t>(p)))));
}

// 16 bytes per lane from global memory straight into LDS
// (global_load_lds_dwordx4): lane l writes bytes 16 l .. 16 l + 15 after the
// wave-uniform LDS address `dst`. Completion is counted by vmcnt.
__device__ __forceinline__ void load_to_lds(const uint16_t* src, unsigned char* dst) {
    typedef __attribute__((address_space(3))) void lds_void;
    __builtin_amdgcn_global_load_lds(
        src, reinterpret_cast<lds_void*>(reinterpret_cast<__attribute__((address_space(3))) char*>(
                 static_cast<uint32_t>(reinterpret_cast<uintptr_t>(dst)))),
        16, 0, 0);
}

// s_waitcnt with only the vector-memory counter limited to n (n < 64)
template <int n>
__device__ __forceinline__ void wait_vmcnt() {
    __builtin_amdgcn_s_waitcnt((n & 0xF) | ((n >> 4) << 14) | (0x7 << 4) | (0xF << 8));
}

__device__ __forceinline__ v4f mfma_bf16_16x16x32(bf16x8 a, bf16x8 b, v4f c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// 16x16x128 E4M3 x E4M3 -> f32 (unscaled form of the block-scaled MFMA).
__device__ __forceinline__ v4f mfma_fp8_16x16x128(v8i a, v8i b, v4f c) {
    return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c, 0, 0, 0, 0, 0, 0);
}

// Order-preserving map of a float to uint32 (larger float -> larger key);
// -0.0 is mapped like +0.0.
__device__ __forceinline__ uint32_t float_order_key(float f) {
    uint32_t u = __float_as_uint(f);
    if ((u & 0x7FFFFFFFu) == 0u) u = 0u;
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// Where position p of batch row b lives in a cache. Dense caches: row
// b * batch_rows + p. Paged caches: page table[b][p >> page_shift] of a pool
// of num_pages pages of 2^page_shift rows; row page << page_shift | offset.
// A page index outside [0, num_pages) means "not present" (row -1).
struct CacheMap {
    const int32_t* table;       // nullptr: dense
    int64_t batch_rows;         // dense: rows per batch row
    int32_t max_pages;          // table row length
    int32_t page_shift;
    int32_t num_pages;

    __device__ __forceinline__ int64_t row(int64_t b, int p) const {
        if (table == nullptr) return b * batch_rows + p;
        const int pg = table[b * max_pages + (p >> page_shift)];
        if (pg < 0 || pg >= num_pages) return -1;
        return (static_cast<int64_t>(pg) << page_shift) | (p & ((1 << page_shift) - 1));
    }
};

}  // namespace dsa
