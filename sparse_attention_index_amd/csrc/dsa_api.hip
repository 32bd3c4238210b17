// dsa_api.hip -- host side of the C ABI declared in include/dsa.h:
// argument validation, workspace sizing and kernel launches. Every check
// runs before the first launch, so an invalid call has no side effects.
#include "../../include/dsa.h"

#include <hip/hip_runtime.h>

#include "dsa_common.h"

#include <cmath>
#include <cstdint>
#include <mutex>

namespace dsa {
hipError_t launch_rope_table(int P, int npairs, double base, int yarn, double low, double high,
                             double factor, float* cos_out, float* sin_out, hipStream_t stream);
hipError_t launch_prepare(bool bf16_in, bool to_cache, int64_t nrows, int rows_per_pos, int S,
                          int Lmax, int P, const void* x, const int32_t* pos, const float* cos_t,
                          const float* sin_t, uint8_t* codes, float* scales, bool hadamard,
                          bool pow2, CacheMap cmap, hipStream_t stream);
hipError_t launch_score(int B, int S, int H, int Lmax, int P, const uint8_t* q8,
                        const float* qscale, const float* w, const int32_t* pos,
                        const uint8_t* kcache, const float* kscale, float* scores, int64_t ld,
                        CacheMap cmap, hipStream_t stream);
hipError_t launch_decode_score(bool bf16_in, int B, int H, int Lmax, int P, const void* q_raw,
                               const void* k_raw, const int32_t* pos, const float* cos_t,
                               const float* sin_t, const float* w, uint8_t* kcache,
                               float* kscale, uint8_t* q8_out, float* qs_out, float* scores,
                               int64_t ld, CacheMap cmap, bool hadamard, bool pow2,
                               hipStream_t stream);
hipError_t launch_topk(int rows, int Lmax, int K, const float* scores, int64_t ld,
                       const int32_t* pos, int32_t* idx, int32_t* count, void* workspace,
                       hipStream_t stream);
size_t topk_workspace_bytes(int rows, int Lmax, int K);
int64_t topk_max_blocks(int rows, int Lmax);
size_t mla_workspace_bytes(int rows, int Hq, int K);
hipError_t launch_sparse_mla(int B, int S, int Hq, int Lmax, int K, const uint16_t* q,
                             const uint16_t* latent, int64_t lat_rs, int64_t lat_bs,
                             const uint16_t* rope, int64_t rope_rs, int64_t rope_bs,
                             const int32_t* idx, float scale, uint16_t* out, float* lse,
                             void* workspace, CacheMap cmap, hipStream_t stream);
hipError_t launch_mla_append(int B, int S, int Hq, int Lmax, int P, const uint16_t* latent_new,
                             const uint16_t* kpe_new, const int32_t* pos, const float* cos_t,
                             const float* sin_t, uint16_t* latent, int64_t lat_rs, int64_t lat_bs,
                             uint16_t* rope, int64_t rope_rs, int64_t rope_bs, uint16_t* q,
                             CacheMap cmap, hipStream_t stream);
hipError_t launch_mla_proj(int mode, int B, int rows, int Hq, const uint16_t* wkv_b,
                           const uint16_t* x, int64_t xrs, int64_t xbs, int64_t xhs, uint16_t* y,
                           int64_t yrs, int64_t ybs, int64_t yhs, hipStream_t stream);
size_t mha_workspace_bytes(int B, int S, int Lmax);
hipError_t launch_sparse_mha(int B, int S, int Hq, int Lmax, int K, const uint16_t* q,
                             const uint16_t* kv, const uint16_t* rope, int64_t rope_rs,
                             int64_t rope_bs, const int32_t* idx, const int32_t* pos, float scale,
                             uint16_t* out, void* workspace, hipStream_t stream);
}  // namespace dsa

namespace dsa {

hipError_t set_dynamic_lds_limit(const void* kernel, int bytes) {
    constexpr int kMaxEntries = 256;
    struct Done {
        const void* kernel;
        int device;
    };
    static std::mutex mu;
    static Done done[kMaxEntries];
    static int ndone = 0;
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    std::lock_guard<std::mutex> lock(mu);
    for (int i = 0; i < ndone; ++i)
        if (done[i].kernel == kernel && done[i].device == dev) return hipSuccess;
    e = hipFuncSetAttribute(kernel, hipFuncAttributeMaxDynamicSharedMemorySize, bytes);
    if (e != hipSuccess) return e;
    if (ndone < kMaxEntries) done[ndone++] = Done{kernel, dev};
    return hipSuccess;
}

}  // namespace dsa

namespace {

constexpr int64_t kMaxGridY = 65535;

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
bool aligned4(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 3u) == 0; }
size_t round_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

// paged-cache fields (shared by every call that touches a per-position cache)
dsa_status check_paging(const int32_t* table, int32_t page_size, int32_t max_pages,
                        int32_t num_pages, int32_t Lmax) {
    if (table == nullptr) return DSA_OK;
    if (page_size < 1 || page_size > 65536 || (page_size & (page_size - 1)) != 0 ||
        num_pages < 1 || max_pages < 1)
        return DSA_ERR_SHAPE;
    if (static_cast<int64_t>(max_pages) * page_size < Lmax) return DSA_ERR_SHAPE;
    if (static_cast<int64_t>(num_pages) * page_size > (int64_t(1) << 31) - 1) return DSA_ERR_SHAPE;
    if (!aligned4(table)) return DSA_ERR_ALIGN;
    return DSA_OK;
}

dsa::CacheMap make_map(const int32_t* table, int32_t page_size, int32_t max_pages,
                       int32_t num_pages, int64_t batch_rows) {
    dsa::CacheMap m{};
    m.table = table;
    m.batch_rows = batch_rows;
    m.max_pages = max_pages;
    m.num_pages = num_pages;
    int sh = 0;
    while (table != nullptr && (1 << sh) < page_size) ++sh;
    m.page_shift = sh;
    return m;
}

// ------------------------------------------------------------- indexer ---
dsa_status check_indexer(const dsa_indexer_args* a) {
    if (a == nullptr) return DSA_ERR_NULL;
    if (a->B < 1 || a->S < 1 || a->H < 1 || a->H > DSA_MAX_INDEX_HEADS || a->Lmax < 1 || a->P < 1)
        return DSA_ERR_SHAPE;
    if (!(a->flags & DSA_INDEXER_APPEND_ONLY) && static_cast<int64_t>(a->B) * a->S > kMaxGridY)
        return DSA_ERR_SHAPE;
    if (static_cast<int64_t>(a->B) * a->S > (int64_t(1) << 31) - 1) return DSA_ERR_SHAPE;
    if (static_cast<int64_t>(a->B) * a->Lmax > (int64_t(1) << 40)) return DSA_ERR_SHAPE;
    if (a->ld_scores < a->Lmax) return DSA_ERR_SHAPE;
    if (a->act_dtype != DSA_DTYPE_F32 && a->act_dtype != DSA_DTYPE_BF16) return DSA_ERR_UNSUPPORTED;
    if ((a->flags & ~(DSA_INDEXER_APPEND_ONLY | DSA_INDEXER_HADAMARD | DSA_INDEXER_POW2_SCALE)) != 0)
        return DSA_ERR_UNSUPPORTED;
    const bool append_only = (a->flags & DSA_INDEXER_APPEND_ONLY) != 0;
    if (!a->pos || !a->rope_cos || !a->rope_sin || !a->k_cache || !a->k_scale) return DSA_ERR_NULL;
    if (append_only) {
        if (!a->k_raw) return DSA_ERR_NULL;
    } else {
        if (!a->q_raw || !a->w || !a->scores) return DSA_ERR_NULL;
        if ((a->q_fp8 == nullptr) != (a->q_scale == nullptr)) return DSA_ERR_NULL;
    }
    const uintptr_t amask = 15;                     // activation rows are read 16 bytes at a time
    if (!aligned16(a->k_cache) || (reinterpret_cast<uintptr_t>(a->k_raw) & amask) ||
        !aligned4(a->k_scale) || !aligned4(a->pos) || !aligned16(a->rope_cos) ||
        !aligned16(a->rope_sin))
        return DSA_ERR_ALIGN;
    if (!append_only &&
        ((reinterpret_cast<uintptr_t>(a->q_raw) & amask) || (a->q_fp8 && !aligned16(a->q_fp8)) ||
         !aligned4(a->scores) || !aligned4(a->w) || (a->q_scale && !aligned4(a->q_scale))))
        return DSA_ERR_ALIGN;
    return check_paging(a->block_table, a->page_size, a->max_pages, a->num_pages, a->Lmax);
}

// one query row per batch row: the fused decode launch (with or without the
// Hadamard and power-of-two options)
bool fused_decode(const dsa_indexer_args* a) {
    return a->S == 1 && !(a->flags & DSA_INDEXER_APPEND_ONLY);
}

size_t indexer_ws(const dsa_indexer_args* a) {
    if (a->q_fp8 != nullptr || (a->flags & DSA_INDEXER_APPEND_ONLY) || fused_decode(a)) return 0;
    const size_t rows = static_cast<size_t>(a->B) * a->S * a->H;
    return round_up(rows * 128, 256) + round_up(rows * sizeof(float), 256);
}

// ---------------------------------------------------------------- topk ---
dsa_status check_topk(const dsa_topk_args* a) {
    if (a == nullptr) return DSA_ERR_NULL;
    if (a->B < 1 || a->S < 1 || a->Lmax < 1 || a->K < 1 || a->K > DSA_MAX_TOPK)
        return DSA_ERR_SHAPE;
    if (static_cast<int64_t>(a->B) * a->S > (int64_t(1) << 31) - 1) return DSA_ERR_SHAPE;
    if (a->ld_scores < a->Lmax) return DSA_ERR_SHAPE;
    if (a->Lmax > (1 << 21)) return DSA_ERR_SHAPE;
    if (dsa::topk_max_blocks(a->B * a->S, a->Lmax) > (int64_t(1) << 31) - 1) return DSA_ERR_SHAPE;
    if (!a->scores || !a->pos || !a->idx) return DSA_ERR_NULL;
    if (!aligned4(a->scores) || !aligned4(a->pos) || !aligned4(a->idx) ||
        (a->count && !aligned4(a->count)))
        return DSA_ERR_ALIGN;
    return DSA_OK;
}

// ----------------------------------------------------------------- mla ---
dsa_status check_mla(const dsa_mla_args* a) {
    if (a == nullptr) return DSA_ERR_NULL;
    if (a->B < 1 || a->S < 1 || a->Hq < 1 || a->Hq > DSA_MAX_ATTN_HEADS || a->Lmax < 1 ||
        a->K < 1 || a->K > DSA_MAX_TOPK)
        return DSA_ERR_SHAPE;
    if (static_cast<int64_t>(a->B) * a->S > kMaxGridY) return DSA_ERR_SHAPE;
    if (!(a->scale > 0.0f) || !std::isfinite(a->scale)) return DSA_ERR_SHAPE;
    if (a->latent_row_stride < DSA_LATENT_DIM || a->rope_row_stride < DSA_ROPE_DIM ||
        a->latent_batch_stride < 0 || a->rope_batch_stride < 0)
        return DSA_ERR_SHAPE;
    if (!a->q || !a->latent || !a->rope || !a->idx || !a->out) return DSA_ERR_NULL;
    if (!aligned16(a->q) || !aligned16(a->latent) || !aligned16(a->rope) || !aligned16(a->out) ||
        !aligned4(a->idx) || (a->lse && !aligned4(a->lse)))
        return DSA_ERR_ALIGN;
    if ((a->latent_row_stride % 8) || (a->latent_batch_stride % 8) || (a->rope_row_stride % 8) ||
        (a->rope_batch_stride % 8))
        return DSA_ERR_ALIGN;
    return check_paging(a->block_table, a->page_size, a->max_pages, a->num_pages, a->Lmax);
}

dsa_status check_mla_append(const dsa_mla_append_args* a) {
    if (a == nullptr) return DSA_ERR_NULL;
    if (a->B < 1 || a->S < 1 || a->Lmax < 1 || a->P < 1) return DSA_ERR_SHAPE;
    if (a->q != nullptr && (a->Hq < 1 || a->Hq > DSA_MAX_ATTN_HEADS)) return DSA_ERR_SHAPE;
    if (static_cast<int64_t>(a->B) * a->S > (int64_t(1) << 31) - 1) return DSA_ERR_SHAPE;
    if (a->latent_row_stride < DSA_LATENT_DIM || a->rope_row_stride < DSA_ROPE_DIM ||
        a->latent_batch_stride < 0 || a->rope_batch_stride < 0)
        return DSA_ERR_SHAPE;
    if (!a->latent_new || !a->kpe_new || !a->pos || !a->rope_cos || !a->rope_sin || !a->latent ||
        !a->rope)
        return DSA_ERR_NULL;
    if (!aligned16(a->latent_new) || !aligned16(a->kpe_new) || !aligned16(a->latent) ||
        !aligned16(a->rope) || (a->q && !aligned16(a->q)) || !aligned4(a->pos) ||
        !aligned4(a->rope_cos) || !aligned4(a->rope_sin))
        return DSA_ERR_ALIGN;
    if ((a->latent_row_stride % 8) || (a->latent_batch_stride % 8) || (a->rope_row_stride % 8) ||
        (a->rope_batch_stride % 8))
        return DSA_ERR_ALIGN;
    return check_paging(a->block_table, a->page_size, a->max_pages, a->num_pages, a->Lmax);
}

// ----------------------------------------------------------- projections ---
// mode 0: kv_up (x rows of 512, y rows of Hq*256), 1: absorb_q (x heads of
// 128, y heads of 512), 2: absorb_o (x heads of 512, y heads of 128)
dsa_status check_mla_proj(const dsa_mla_proj_args* a, int mode) {
    if (a == nullptr) return DSA_ERR_NULL;
    if (a->B < 1 || a->rows < 1 || a->rows > (1 << 24) || a->Hq < 1 ||
        a->Hq > DSA_MAX_ATTN_HEADS)
        return DSA_ERR_SHAPE;
    const int64_t zs = mode == 0 ? a->B : static_cast<int64_t>(a->B) * a->Hq;
    if (zs > kMaxGridY) return DSA_ERR_SHAPE;
    if (!a->wkv_b || !a->x || !a->y) return DSA_ERR_NULL;
    const int64_t yw = mode == 0 ? int64_t(256) * a->Hq : (mode == 1 ? DSA_LATENT_DIM : 128);
    const int64_t xh = mode == 0 ? 0 : a->x_head_stride, yh = mode == 0 ? 0 : a->y_head_stride;
    if (a->x_row_stride < 0 || a->x_batch_stride < 0 || a->y_row_stride < 0 ||
        a->y_batch_stride < 0 || xh < 0 || yh < 0)
        return DSA_ERR_SHAPE;
    // output heads, rows and batches must not overlap
    if (mode != 0 && a->Hq > 1 && yh < yw) return DSA_ERR_SHAPE;
    const int64_t yrow = (mode == 0 ? 0 : (a->Hq - 1) * yh) + yw;
    if (a->rows > 1 && a->y_row_stride < yrow) return DSA_ERR_SHAPE;
    if (a->B > 1 && a->y_batch_stride < (a->rows - 1) * a->y_row_stride + yrow) return DSA_ERR_SHAPE;
    if (!aligned16(a->wkv_b) || !aligned16(a->x) || !aligned16(a->y)) return DSA_ERR_ALIGN;
    if ((a->x_row_stride % 8) || (a->x_batch_stride % 8) || (xh % 8) || (a->y_row_stride % 8) ||
        (a->y_batch_stride % 8) || (yh % 8))
        return DSA_ERR_ALIGN;
    return DSA_OK;
}

// ------------------------------------------------------------------- mha ---
constexpr int kMhaMaxL = 65536;

dsa_status check_mha(const dsa_mha_args* a) {
    if (a == nullptr) return DSA_ERR_NULL;
    if (a->B < 1 || a->S < 1 || a->Hq < 1 || a->Hq > DSA_MAX_ATTN_HEADS || a->Lmax < 1 ||
        a->Lmax > kMhaMaxL || a->K < 1 || a->K > DSA_MAX_TOPK)
        return DSA_ERR_SHAPE;
    const int64_t nqt = static_cast<int64_t>(a->B) * ((a->S + 127) / 128);
    if (nqt * a->Hq > (int64_t(1) << 31) - 1 || static_cast<int64_t>(a->B) * a->S > (1 << 26))
        return DSA_ERR_SHAPE;
    if (!(a->scale > 0.0f) || !std::isfinite(a->scale)) return DSA_ERR_SHAPE;
    if (a->rope_row_stride < DSA_ROPE_DIM || a->rope_batch_stride < 0) return DSA_ERR_SHAPE;
    if (!a->q || !a->kv || !a->rope || !a->idx || !a->out) return DSA_ERR_NULL;
    if (!aligned16(a->q) || !aligned16(a->kv) || !aligned16(a->rope) || !aligned16(a->out) ||
        !aligned4(a->idx) || (a->pos && !aligned4(a->pos)))
        return DSA_ERR_ALIGN;
    if ((a->rope_row_stride % 8) || (a->rope_batch_stride % 8)) return DSA_ERR_ALIGN;
    return DSA_OK;
}

dsa_status hip_status(hipError_t e) { return e == hipSuccess ? DSA_OK : DSA_ERR_HIP; }

// ------------------------------------------------- no-allocation scratch ---
// The static device array behind dsa_sparse_mla_noalloc. In host code its
// name is only a host-side stand-in: every use goes through the device
// address looked up below, once per device (each GPU holds its own copy).
static __device__ __align__(256) unsigned char scratch[DSA_MLA_NOALLOC_MAX_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// Device address of the current device's scratch (looked up on the first
// call per device, with that device current).
dsa_status scratch_of_current_device(void** out) {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess) return DSA_ERR_HIP;
    if (dev < 0 || dev >= kMaxDevices) return DSA_ERR_HIP;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (g_scratch_ptr[dev] == nullptr) {
        void* ptr = nullptr;
        if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || ptr == nullptr)
            return DSA_ERR_HIP;
        g_scratch_ptr[dev] = ptr;
    }
    *out = g_scratch_ptr[dev];
    return DSA_OK;
}

dsa_status run_mla_proj(const dsa_mla_proj_args* a, int mode, hipStream_t stream) {
    const dsa_status st = check_mla_proj(a, mode);
    if (st != DSA_OK) return st;
    return hip_status(dsa::launch_mla_proj(mode, a->B, a->rows, a->Hq, a->wkv_b, a->x,
                                           a->x_row_stride, a->x_batch_stride, a->x_head_stride,
                                           a->y, a->y_row_stride, a->y_batch_stride,
                                           a->y_head_stride, stream));
}

}  // namespace

extern "C" {

int dsa_abi_version(void) { return DSA_ABI_VERSION; }

const char* dsa_status_str(dsa_status s) {
    switch (s) {
        case DSA_OK: return "DSA_OK";
        case DSA_ERR_NULL: return "DSA_ERR_NULL: a required pointer is NULL";
        case DSA_ERR_SHAPE: return "DSA_ERR_SHAPE: a size or stride is out of range";
        case DSA_ERR_UNSUPPORTED: return "DSA_ERR_UNSUPPORTED: unknown dtype or flag";
        case DSA_ERR_WORKSPACE: return "DSA_ERR_WORKSPACE: workspace missing or too small";
        case DSA_ERR_ALIGN: return "DSA_ERR_ALIGN: pointer or stride not aligned";
        case DSA_ERR_HIP: return "DSA_ERR_HIP: a HIP launch failed";
        case DSA_ERR_SCRATCH:
            return "DSA_ERR_SCRATCH: the call needs more than the no-allocation call's static "
                   "scratch (DSA_MLA_NOALLOC_MAX_BYTES)";
    }
    return "unknown dsa_status";
}

dsa_status dsa_rope_table(const dsa_rope_table_args* a, hipStream_t stream) {
    if (a == nullptr || a->cos_out == nullptr || a->sin_out == nullptr) return DSA_ERR_NULL;
    if (a->P < 1 || !(a->theta > 1.0f) || !std::isfinite(a->theta)) return DSA_ERR_SHAPE;
    if (a->yarn != 0 && a->yarn != 1) return DSA_ERR_UNSUPPORTED;
    if (!aligned4(a->cos_out) || !aligned4(a->sin_out)) return DSA_ERR_ALIGN;
    const int npairs = DSA_INDEX_ROPE / 2;
    const int dim = DSA_INDEX_ROPE;
    double low = 0.0, high = 1.0;
    if (a->yarn) {
        if (a->orig_len < 1 || !(a->factor >= 1.0f) || !(a->beta_fast > a->beta_slow) ||
            !(a->beta_slow > 0.0f) || !std::isfinite(a->factor) || !std::isfinite(a->beta_fast))
            return DSA_ERR_SHAPE;
        // YaRN correction dims: d(r) = dim * ln(orig / (2 pi r)) / (2 ln base)
        const double pi = 3.14159265358979323846;
        auto corr = [&](double r) {
            return dim * std::log(static_cast<double>(a->orig_len) / (r * 2.0 * pi)) /
                   (2.0 * std::log(static_cast<double>(a->theta)));
        };
        low = std::floor(corr(a->beta_fast));
        high = std::ceil(corr(a->beta_slow));
        if (low < 0.0) low = 0.0;
        if (high > dim - 1) high = dim - 1;
        if (low == high) high += 0.001;
    }
    return hip_status(dsa::launch_rope_table(a->P, npairs, static_cast<double>(a->theta), a->yarn,
                                             low, high, static_cast<double>(a->factor),
                                             a->cos_out, a->sin_out, stream));
}

dsa_status dsa_indexer_workspace(const dsa_indexer_args* a, size_t* bytes) {
    if (bytes == nullptr) return DSA_ERR_NULL;
    const dsa_status st = check_indexer(a);
    if (st != DSA_OK) return st;
    *bytes = indexer_ws(a);
    return DSA_OK;
}

dsa_status dsa_indexer(const dsa_indexer_args* a, hipStream_t stream) {
    dsa_status st = check_indexer(a);
    if (st != DSA_OK) return st;
    const size_t need = indexer_ws(a);
    uint8_t* q8 = a->q_fp8;
    if (a->flags & DSA_INDEXER_APPEND_ONLY) q8 = nullptr;
    float* qs = a->q_scale;
    if (need > 0) {
        if (a->workspace == nullptr || a->workspace_bytes < need) return DSA_ERR_WORKSPACE;
        if ((reinterpret_cast<uintptr_t>(a->workspace) & 255u) != 0) return DSA_ERR_ALIGN;
        const size_t rows = static_cast<size_t>(a->B) * a->S * a->H;
        q8 = static_cast<uint8_t*>(a->workspace);
        qs = reinterpret_cast<float*>(q8 + round_up(rows * 128, 256));
    }
    const bool bf16 = a->act_dtype == DSA_DTYPE_BF16;
    const int64_t qrows = static_cast<int64_t>(a->B) * a->S * a->H;
    hipError_t e = hipSuccess;
    const bool had = (a->flags & DSA_INDEXER_HADAMARD) != 0;
    const bool pow2 = (a->flags & DSA_INDEXER_POW2_SCALE) != 0;
    const dsa::CacheMap cmap =
        make_map(a->block_table, a->page_size, a->max_pages, a->num_pages, a->Lmax);
    if (fused_decode(a)) {
        // decode: one fused launch (quantise q, append the new key, score)
        e = dsa::launch_decode_score(bf16, a->B, a->H, a->Lmax, a->P, a->q_raw, a->k_raw, a->pos,
                                     a->rope_cos, a->rope_sin, a->w, a->k_cache, a->k_scale,
                                     a->q_fp8, a->q_scale, a->scores, a->ld_scores, cmap, had,
                                     pow2, stream);
        return hip_status(e);
    }
    if (a->k_raw != nullptr) {
        e = dsa::launch_prepare(bf16, true, static_cast<int64_t>(a->B) * a->S, 1, a->S, a->Lmax,
                                a->P, a->k_raw, a->pos, a->rope_cos, a->rope_sin, a->k_cache,
                                a->k_scale, had, pow2, cmap, stream);
        if (e != hipSuccess) return DSA_ERR_HIP;
    }
    if (a->flags & DSA_INDEXER_APPEND_ONLY) return DSA_OK;
    e = dsa::launch_prepare(bf16, false, qrows, a->H, a->S, a->Lmax, a->P, a->q_raw, a->pos,
                            a->rope_cos, a->rope_sin, q8, qs, had, pow2, cmap, stream);
    if (e != hipSuccess) return DSA_ERR_HIP;
    e = dsa::launch_score(a->B, a->S, a->H, a->Lmax, a->P, q8, qs, a->w, a->pos, a->k_cache,
                          a->k_scale, a->scores, a->ld_scores, cmap, stream);
    return hip_status(e);
}

dsa_status dsa_topk_workspace(const dsa_topk_args* a, size_t* bytes) {
    if (bytes == nullptr) return DSA_ERR_NULL;
    const dsa_status st = check_topk(a);
    if (st != DSA_OK) return st;
    *bytes = dsa::topk_workspace_bytes(a->B * a->S, a->Lmax, a->K);
    return DSA_OK;
}

dsa_status dsa_topk(const dsa_topk_args* a, hipStream_t stream) {
    const dsa_status st = check_topk(a);
    if (st != DSA_OK) return st;
    const size_t need = dsa::topk_workspace_bytes(a->B * a->S, a->Lmax, a->K);
    if (need > 0) {
        if (a->workspace == nullptr || a->workspace_bytes < need) return DSA_ERR_WORKSPACE;
        if ((reinterpret_cast<uintptr_t>(a->workspace) & 255u) != 0) return DSA_ERR_ALIGN;
    }
    return hip_status(dsa::launch_topk(a->B * a->S, a->Lmax, a->K, a->scores, a->ld_scores,
                                       a->pos, a->idx, a->count, a->workspace, stream));
}

dsa_status dsa_sparse_mla_workspace(const dsa_mla_args* a, size_t* bytes) {
    if (bytes == nullptr) return DSA_ERR_NULL;
    const dsa_status st = check_mla(a);
    if (st != DSA_OK) return st;
    *bytes = dsa::mla_workspace_bytes(a->B * a->S, a->Hq, a->K);
    return DSA_OK;
}

dsa_status dsa_sparse_mla(const dsa_mla_args* a, hipStream_t stream) {
    const dsa_status st = check_mla(a);
    if (st != DSA_OK) return st;
    const size_t need = dsa::mla_workspace_bytes(a->B * a->S, a->Hq, a->K);
    if (need > 0) {
        if (a->workspace == nullptr || a->workspace_bytes < need) return DSA_ERR_WORKSPACE;
        if ((reinterpret_cast<uintptr_t>(a->workspace) & 255u) != 0) return DSA_ERR_ALIGN;
    }
    return hip_status(dsa::launch_sparse_mla(
        a->B, a->S, a->Hq, a->Lmax, a->K, a->q, a->latent, a->latent_row_stride,
        a->latent_batch_stride, a->rope, a->rope_row_stride, a->rope_batch_stride, a->idx,
        a->scale, a->out, a->lse, a->workspace,
        make_map(a->block_table, a->page_size, a->max_pages, a->num_pages, 0), stream));
}

dsa_status dsa_sparse_mla_noalloc(const dsa_mla_args* a, hipStream_t stream) {
    dsa_status st = check_mla(a);
    if (st != DSA_OK) return st;
    const size_t need = dsa::mla_workspace_bytes(a->B * a->S, a->Hq, a->K);
    if (need > DSA_MLA_NOALLOC_MAX_BYTES) return DSA_ERR_SCRATCH;
    void* ws = nullptr;
    if (need > 0) {
        st = scratch_of_current_device(&ws);
        if (st != DSA_OK) return st;
    }
    return hip_status(dsa::launch_sparse_mla(
        a->B, a->S, a->Hq, a->Lmax, a->K, a->q, a->latent, a->latent_row_stride,
        a->latent_batch_stride, a->rope, a->rope_row_stride, a->rope_batch_stride, a->idx,
        a->scale, a->out, a->lse, ws,
        make_map(a->block_table, a->page_size, a->max_pages, a->num_pages, 0), stream));
}

dsa_status dsa_mla_append(const dsa_mla_append_args* a, hipStream_t stream) {
    const dsa_status st = check_mla_append(a);
    if (st != DSA_OK) return st;
    return hip_status(dsa::launch_mla_append(
        a->B, a->S, a->q ? a->Hq : 0, a->Lmax, a->P, a->latent_new, a->kpe_new, a->pos,
        a->rope_cos, a->rope_sin, a->latent, a->latent_row_stride, a->latent_batch_stride,
        a->rope, a->rope_row_stride, a->rope_batch_stride, a->q,
        make_map(a->block_table, a->page_size, a->max_pages, a->num_pages, 0), stream));
}

dsa_status dsa_mla_kv_up(const dsa_mla_proj_args* a, hipStream_t stream) {
    return run_mla_proj(a, 0, stream);
}

dsa_status dsa_mla_absorb_q(const dsa_mla_proj_args* a, hipStream_t stream) {
    return run_mla_proj(a, 1, stream);
}

dsa_status dsa_mla_absorb_o(const dsa_mla_proj_args* a, hipStream_t stream) {
    return run_mla_proj(a, 2, stream);
}

dsa_status dsa_sparse_mha_workspace(const dsa_mha_args* a, size_t* bytes) {
    if (bytes == nullptr) return DSA_ERR_NULL;
    const dsa_status st = check_mha(a);
    if (st != DSA_OK) return st;
    *bytes = dsa::mha_workspace_bytes(a->B, a->S, a->Lmax);
    return DSA_OK;
}

dsa_status dsa_sparse_mha(const dsa_mha_args* a, hipStream_t stream) {
    const dsa_status st = check_mha(a);
    if (st != DSA_OK) return st;
    const size_t need = dsa::mha_workspace_bytes(a->B, a->S, a->Lmax);
    if (a->workspace == nullptr || a->workspace_bytes < need) return DSA_ERR_WORKSPACE;
    if ((reinterpret_cast<uintptr_t>(a->workspace) & 255u) != 0) return DSA_ERR_ALIGN;
    return hip_status(dsa::launch_sparse_mha(a->B, a->S, a->Hq, a->Lmax, a->K, a->q, a->kv,
                                             a->rope, a->rope_row_stride, a->rope_batch_stride,
                                             a->idx, a->pos, a->scale, a->out, a->workspace,
                                             stream));
}

}  // extern "C"
