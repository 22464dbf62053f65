// Host side of the C ABI declared in nabla.h: argument validation (before any HIP
// call, so it also runs on machines without a GPU) and dispatch to the launchers.
#include <math.h>
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include "nabla_internal.h"

namespace {

thread_local char g_last_error[512] = "";

nabla_status fail(nabla_status st, const char* fmt, ...) {
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_last_error, sizeof(g_last_error), fmt, ap);
    va_end(ap);
    return st;
}

nabla_status hip_status(hipError_t e, const char* where) {
    if (e == hipSuccess) return NABLA_OK;
    return fail(NABLA_E_HIP, "%s: %s", where, hipGetErrorString(e));
}

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

size_t elem_size(nabla_dtype dt) { return dt == NABLA_BF16 ? 2 : 4; }

bool valid_dtype(nabla_dtype dt) { return dt == NABLA_F32 || dt == NABLA_BF16; }

// Tokens per head times d must stay addressable with 32-bit chunk indices.
constexpr long long kMaxHeadElems = 1ll << 33;
// The attention kernels address a head's K and V through buffer resources with 32-bit
// byte offsets (signed in the tile arithmetic), so a head must stay below 2^31 bytes.
constexpr long long kMaxHeadBytes = 1ll << 31;

// Checks a raster grid of one P x P patch per N-token block; sets L = T H W.
nabla_status raster_tokens(const char* who, int T, int H, int W, int P, int N, int* L) {
    if (T <= 0 || H <= 0 || W <= 0 || P <= 0 || N <= 0) return fail(NABLA_E_INVAL, "%s: sizes must be positive", who);
    if (H % P || W % P) return fail(NABLA_E_INVAL, "%s: H=%d and W=%d must be multiples of P=%d", who, H, W, P);
    if (N != P * P)
        return fail(NABLA_E_INVAL, "%s: raster order needs one P x P patch per block (N == P*P)", who);
    const long long tokens = (long long)T * H * W;
    if (tokens >= (1ll << 31)) return fail(NABLA_E_UNSUPPORTED, "%s: tensor too large", who);
    *L = (int)tokens;
    return NABLA_OK;
}

}  // namespace

extern "C" {

const char* nabla_status_string(nabla_status st) {
    switch (st) {
        case NABLA_OK: return "NABLA_OK";
        case NABLA_E_INVAL: return "NABLA_E_INVAL";
        case NABLA_E_UNSUPPORTED: return "NABLA_E_UNSUPPORTED";
        case NABLA_E_HIP: return "NABLA_E_HIP";
        case NABLA_E_WORKSPACE: return "NABLA_E_WORKSPACE";
    }
    return "NABLA_E_UNKNOWN";
}

const char* nabla_last_error(void) { return g_last_error; }

nabla_status nabla_reorder(const void* src, void* dst, int batch, int heads, int T, int H,
                           int W, int d, int P, nabla_dtype dtype, int inverse,
                           hipStream_t stream) {
    if (!src || !dst) return fail(NABLA_E_INVAL, "nabla_reorder: null pointer");
    if (src == dst) return fail(NABLA_E_INVAL, "nabla_reorder: src and dst must differ");
    if (!aligned16(src) || !aligned16(dst))
        return fail(NABLA_E_INVAL, "nabla_reorder: pointers must be 16-byte aligned");
    if (batch <= 0 || heads <= 0 || T <= 0 || H <= 0 || W <= 0 || d <= 0 || P <= 0)
        return fail(NABLA_E_INVAL, "nabla_reorder: sizes must be positive");
    if (H % P || W % P)
        return fail(NABLA_E_INVAL, "nabla_reorder: H=%d and W=%d must be multiples of P=%d", H, W, P);
    if (inverse != 0 && inverse != 1) return fail(NABLA_E_INVAL, "nabla_reorder: inverse must be 0 or 1");
    if (!valid_dtype(dtype)) return fail(NABLA_E_INVAL, "nabla_reorder: unknown dtype %d", (int)dtype);
    const long long L = (long long)T * H * W;
    const size_t row_bytes = (size_t)d * elem_size(dtype);
    if (row_bytes % 16)
        return fail(NABLA_E_UNSUPPORTED, "nabla_reorder: d*sizeof(dtype) = %zu is not a multiple of 16", row_bytes);
    const long long chunks = L * (long long)(row_bytes / 16);
    if (chunks >= (1ll << 31) || (long long)batch * heads > 65535)
        return fail(NABLA_E_UNSUPPORTED, "nabla_reorder: tensor too large");
    int chunk_shift = 0;
    while ((size_t(16) << chunk_shift) < row_bytes) ++chunk_shift;
    if ((size_t(16) << chunk_shift) != row_bytes)
        return fail(NABLA_E_UNSUPPORTED, "nabla_reorder: d*sizeof(dtype) must be 16 bytes times a power of two");
    nabla::ReorderArgs a{src, dst, batch * heads, T, H, W, P, (int)L, chunk_shift, inverse};
    return hip_status(nabla::launch_reorder(a, stream), "nabla_reorder");
}

namespace {

size_t up256(size_t n) { return (n + 255) & ~(size_t)255; }

// The NABLA workspace: the pooled K (the map kernel pools Q itself).
struct NablaSections {
    size_t kp, kexp;
    size_t total() const { return kp + kexp; }
};

NablaSections nabla_sections(long long BH, long long nb, int d) {
    // split Kp in tiles of 16 blocks (the last one padded), then one exponent per block
    const long long nb16 = (nb + 15) / 16 * 16;
    return {up256((size_t)BH * nb16 * d * sizeof(float)), up256((size_t)BH * nb * sizeof(int32_t))};
}

}  // namespace

size_t nabla_build_mask_workspace_size(int batch, int heads, int L, int d, int N) {
    if (batch <= 0 || heads <= 0 || L <= 0 || d <= 0 || N <= 0 || L % N) return 0;
    return nabla_sections((long long)batch * heads, L / N, d).total();
}

namespace {

// Sections of the IBCS workspace, each a multiple of 256 bytes: pooled K, centroids,
// weights, score rows.
struct IbcsSections {
    size_t kp, cent, cw, scores;
    size_t total() const { return kp + cent + cw + scores; }
};

IbcsSections ibcs_sections(long long BH, long long nb, long long groups, int d) {
    // float32 pooled K in tiles of 16 blocks (the last one padded), then centroids, weights, scores
    const long long nb16 = (nb + 15) / 16 * 16;
    return {up256((size_t)BH * nb16 * d * sizeof(float)),
            up256((size_t)BH * groups * nabla::kIbcsClusters * d * sizeof(float)),
            up256((size_t)BH * groups * nabla::kIbcsClusters * sizeof(float)),
            up256((size_t)BH * groups * nb * sizeof(float))};
}

}  // namespace

size_t nabla_build_mask_ibcs_workspace_size(int batch, int heads, int L, int d, int N, int q_group) {
    if (batch <= 0 || heads <= 0 || L <= 0 || d <= 0 || N <= 0 || q_group <= 0 || L % N || q_group % N ||
        L % q_group)
        return 0;
    return ibcs_sections((long long)batch * heads, L / N, L / q_group, d).total();
}

namespace {

nabla_status build_mask_impl(const char* who, int raster, const void* q, const void* k, int batch,
                             int heads, int T, int H, int W, int d, int P, int N, float thr,
                             const nabla_sta_window* sta, float scale, nabla_dtype dtype,
                             int32_t* kv_count, int32_t* kv_index, uint32_t* bitmap,
                             int32_t* schedule, void* workspace, size_t workspace_bytes,
                             hipStream_t stream, int sip_budget = 0, const float* uniforms = nullptr,
                             float* kv_logw = nullptr, int ibcs_q_group = 0, int use_scratch = 0);

}  // namespace

nabla_status nabla_build_mask(const void* q, const void* k, int batch, int heads, int T, int H,
                              int W, int d, int P, int N, float thr,
                              const nabla_sta_window* sta, float scale, nabla_dtype dtype,
                              int32_t* kv_count, int32_t* kv_index, uint32_t* bitmap,
                              int32_t* schedule, void* workspace, size_t workspace_bytes,
                              hipStream_t stream) {
    return build_mask_impl("nabla_build_mask", 0, q, k, batch, heads, T, H, W, d, P, N, thr, sta, scale,
                           dtype, kv_count, kv_index, bitmap, schedule, workspace, workspace_bytes, stream);
}

nabla_status nabla_build_mask_sip(const void* q, const void* k, int batch, int heads, int T, int H,
                                  int W, int d, int P, int N, int budget, const float* uniforms,
                                  float scale, nabla_dtype dtype, int32_t* kv_count, int32_t* kv_index,
                                  float* kv_logw, uint32_t* bitmap, int32_t* schedule, void* workspace,
                                  size_t workspace_bytes, hipStream_t stream) {
    const char* who = "nabla_build_mask_sip";
    if (!uniforms || !kv_logw) return fail(NABLA_E_INVAL, "%s: null pointer", who);
    if (((uintptr_t)uniforms & 3) || ((uintptr_t)kv_logw & 3))
        return fail(NABLA_E_INVAL, "%s: misaligned pointer", who);
    if (budget < 1) return fail(NABLA_E_INVAL, "%s: budget must be at least 1", who);
    return build_mask_impl(who, 0, q, k, batch, heads, T, H, W, d, P, N, 0.0f, nullptr, scale, dtype,
                           kv_count, kv_index, bitmap, schedule, workspace, workspace_bytes, stream, budget,
                           uniforms, kv_logw);
}

nabla_status nabla_build_mask_ibcs(const void* q, const void* k, int batch, int heads, int T, int H,
                                   int W, int d, int P, int N, int q_group, float thr,
                                   const nabla_sta_window* sta, float scale, nabla_dtype dtype,
                                   int32_t* kv_count, int32_t* kv_index, uint32_t* bitmap,
                                   int32_t* schedule, void* workspace, size_t workspace_bytes,
                                   hipStream_t stream) {
    const char* who = "nabla_build_mask_ibcs";
    if (q_group <= 0 || N <= 0 || q_group % N)
        return fail(NABLA_E_INVAL, "%s: q_group=%d must be a positive multiple of N=%d", who, q_group, N);
    return build_mask_impl(who, 0, q, k, batch, heads, T, H, W, d, P, N, thr, sta, scale, dtype, kv_count, kv_index,
                           bitmap, schedule, workspace, workspace_bytes, stream, 0, nullptr, nullptr, q_group);
}

nabla_status nabla_build_mask_ibcs_raster(const void* q, const void* k, int batch, int heads, int T, int H,
                                          int W, int d, int P, int N, int q_group, float thr,
                                          const nabla_sta_window* sta, float scale, nabla_dtype dtype,
                                          int32_t* kv_count, int32_t* kv_index, uint32_t* bitmap,
                                          int32_t* schedule, void* workspace, size_t workspace_bytes,
                                          hipStream_t stream) {
    const char* who = "nabla_build_mask_ibcs_raster";
    if (q_group <= 0 || N <= 0 || q_group % N)
        return fail(NABLA_E_INVAL, "%s: q_group=%d must be a positive multiple of N=%d", who, q_group, N);
    return build_mask_impl(who, 1, q, k, batch, heads, T, H, W, d, P, N, thr, sta, scale, dtype, kv_count, kv_index,
                           bitmap, schedule, workspace, workspace_bytes, stream, 0, nullptr, nullptr, q_group);
}

nabla_status nabla_build_mask_ibcs_sip(const void* q, const void* k, int batch, int heads, int T, int H, int W,
                                       int d, int P, int N, int q_group, int budget, const float* uniforms,
                                       float scale, nabla_dtype dtype, int32_t* kv_count, int32_t* kv_index,
                                       float* kv_logw, uint32_t* bitmap, int32_t* schedule, void* workspace,
                                       size_t workspace_bytes, hipStream_t stream) {
    const char* who = "nabla_build_mask_ibcs_sip";
    if (!uniforms || !kv_logw) return fail(NABLA_E_INVAL, "%s: null pointer", who);
    if (((uintptr_t)uniforms & 3) || ((uintptr_t)kv_logw & 3))
        return fail(NABLA_E_INVAL, "%s: misaligned pointer", who);
    if (budget < 1) return fail(NABLA_E_INVAL, "%s: budget must be at least 1", who);
    if (q_group <= 0 || N <= 0 || q_group % N)
        return fail(NABLA_E_INVAL, "%s: q_group=%d must be a positive multiple of N=%d", who, q_group, N);
    return build_mask_impl(who, 0, q, k, batch, heads, T, H, W, d, P, N, 0.0f, nullptr, scale, dtype, kv_count,
                           kv_index, bitmap, schedule, workspace, workspace_bytes, stream, budget, uniforms, kv_logw,
                           q_group);
}

nabla_status nabla_build_mask_raster(const void* q, const void* k, int batch, int heads, int T, int H,
                                     int W, int d, int P, int N, float thr,
                                     const nabla_sta_window* sta, float scale, nabla_dtype dtype,
                                     int32_t* kv_count, int32_t* kv_index, uint32_t* bitmap,
                                     int32_t* schedule, void* workspace, size_t workspace_bytes,
                                     hipStream_t stream) {
    return build_mask_impl("nabla_build_mask_raster", 1, q, k, batch, heads, T, H, W, d, P, N, thr, sta,
                           scale, dtype, kv_count, kv_index, bitmap, schedule, workspace, workspace_bytes,
                           stream);
}

nabla_status nabla_build_mask_raster_noalloc(const void* q, const void* k, int batch, int heads, int T, int H,
                                             int W, int d, int P, int N, float thr, const nabla_sta_window* sta,
                                             float scale, nabla_dtype dtype, int32_t* kv_count, int32_t* kv_index,
                                             uint32_t* bitmap, int32_t* schedule, hipStream_t stream) {
    return build_mask_impl("nabla_build_mask_raster_noalloc", 1, q, k, batch, heads, T, H, W, d, P, N, thr, sta,
                           scale, dtype, kv_count, kv_index, bitmap, schedule, nullptr, 0, stream, 0, nullptr,
                           nullptr, 0, 1);
}

namespace {

nabla_status build_mask_impl(const char* who, int raster, const void* q, const void* k, int batch,
                             int heads, int T, int H, int W, int d, int P, int N, float thr,
                             const nabla_sta_window* sta, float scale, nabla_dtype dtype,
                             int32_t* kv_count, int32_t* kv_index, uint32_t* bitmap,
                             int32_t* schedule, void* workspace, size_t workspace_bytes,
                             hipStream_t stream, int sip_budget, const float* uniforms,
                             float* kv_logw, int ibcs_q_group, int use_scratch) {
    if (!q || !k || !kv_count || !kv_index) return fail(NABLA_E_INVAL, "%s: null pointer", who);
    if (!aligned16(q) || !aligned16(k) || ((uintptr_t)kv_count & 3) || ((uintptr_t)kv_index & 3) ||
        ((uintptr_t)bitmap & 3) || ((uintptr_t)schedule & 3))
        return fail(NABLA_E_INVAL, "%s: misaligned pointer", who);
    if (batch <= 0 || heads <= 0 || T <= 0 || H <= 0 || W <= 0 || d <= 0 || P <= 0 || N <= 0)
        return fail(NABLA_E_INVAL, "%s: sizes must be positive", who);
    if (H % P || W % P)
        return fail(NABLA_E_INVAL, "%s: H=%d and W=%d must be multiples of P=%d", who, H, W, P);
    const long long L = (long long)T * H * W;
    if (L % N) return fail(NABLA_E_INVAL, "%s: L=%lld is not a multiple of N=%d", who, L, N);
    if (!(thr >= 0.f && thr < 1.f)) return fail(NABLA_E_INVAL, "%s: thr must lie in [0, 1)", who);
    if (isnan(scale) || isinf(scale)) return fail(NABLA_E_INVAL, "%s: scale must be finite", who);
    if (!valid_dtype(dtype)) return fail(NABLA_E_INVAL, "%s: unknown dtype %d", who, (int)dtype);
    if (sta) {
        if (sta->wt < 1 || sta->wh < 1 || sta->ww < 1 || !(sta->wt & 1) || !(sta->wh & 1) || !(sta->ww & 1))
            return fail(NABLA_E_INVAL, "%s: STA window sizes must be odd and >= 1", who);
        if (N != P * P)
            return fail(NABLA_E_INVAL, "%s: an STA tile is one P x P patch, so N must equal P*P", who);
    }
    if (raster && N != P * P)
        return fail(NABLA_E_INVAL, "%s: raster order needs one P x P patch per block (N == P*P)", who);
    if (N != 64) return fail(NABLA_E_UNSUPPORTED, "%s: only N = 64 is implemented", who);
    if (d != 64 && d != 128) return fail(NABLA_E_UNSUPPORTED, "%s: d must be 64 or 128", who);
    if (ibcs_q_group && L % ibcs_q_group)
        return fail(NABLA_E_INVAL, "%s: L=%lld is not a multiple of q_group=%d", who, L, ibcs_q_group);
    if (ibcs_q_group && ibcs_q_group != 64 && ibcs_q_group != 128)
        return fail(NABLA_E_UNSUPPORTED, "%s: q_group must be 64 or 128", who);
    const long long nb = L / N;
    if (nb > NABLA_MAX_BLOCKS)
        return fail(NABLA_E_UNSUPPORTED, "%s: %lld blocks per head exceed %d", who, nb, NABLA_MAX_BLOCKS);
    if (ibcs_q_group && nb > NABLA_IBCS_MAX_BLOCKS)
        return fail(NABLA_E_UNSUPPORTED, "%s: %lld blocks per head exceed %d (IBCS score rows are held in LDS)",
                    who, nb, NABLA_IBCS_MAX_BLOCKS);
    // the launches cover up to 256 threads per block of every head with 32-bit thread ids
    if ((long long)batch * heads > 65535 || L * d >= kMaxHeadElems || (long long)batch * heads * nb >= (1ll << 24))
        return fail(NABLA_E_UNSUPPORTED, "%s: tensor too large", who);
    // pooled K of one head in the split half form, and its exponents (the first part a
    // multiple of 256 bytes for d = 64, 128)
    const size_t head_kp_bytes = (size_t)((nb + 15) / 16 * 16) * d * sizeof(float);
    const size_t head_pool_bytes = head_kp_bytes + (size_t)nb * sizeof(int32_t);
    if (use_scratch && head_pool_bytes > nabla::kScratchBytes)
        return fail(NABLA_E_UNSUPPORTED, "%s: one head's pooled K needs %zu bytes, the scratch holds %zu", who,
                    head_pool_bytes, nabla::kScratchBytes);
    const size_t need = ibcs_q_group ? nabla_build_mask_ibcs_workspace_size(batch, heads, (int)L, d, N, ibcs_q_group)
                                     : nabla_build_mask_workspace_size(batch, heads, (int)L, d, N);
    if (use_scratch) {
        // the library's own device array stands in for the workspace
        size_t bytes = 0;
        nabla_status st = hip_status(nabla::device_scratch(&workspace, &bytes), who);
        if (st != NABLA_OK) return st;
        workspace_bytes = bytes;
    } else if (!workspace || workspace_bytes < need)
        return fail(NABLA_E_WORKSPACE, "%s: workspace of %zu bytes needed, %zu given", who, need,
                    workspace ? workspace_bytes : (size_t)0);
    if (((uintptr_t)workspace & 15)) return fail(NABLA_E_INVAL, "%s: misaligned workspace", who);

    nabla::MaskArgs a{};
    a.q = q;
    a.k = k;
    a.BH = batch * heads;
    a.nb = (int)nb;
    a.d = d;
    a.N = N;
    a.T = T;
    a.nH = H / P;
    a.nW = W / P;
    a.thr = thr;
    a.scale = scale > 0.f ? scale : 1.0f / sqrtf((float)d);
    a.sta = sta ? 1 : 0;
    a.rt = sta ? (sta->wt - 1) / 2 : 0;
    a.rh = sta ? (sta->wh - 1) / 2 : 0;
    a.rw = sta ? (sta->ww - 1) / 2 : 0;
    a.kv_count = kv_count;
    a.kv_index = kv_index;
    a.bitmap = bitmap;
    a.schedule = schedule;
    if (ibcs_q_group) {
        // [Kp | centroids | weights | score rows], sections 256-byte aligned
        const IbcsSections sec = ibcs_sections(a.BH, nb, L / ibcs_q_group, d);
        char* base = (char*)workspace;
        a.qp = nullptr;
        a.kp = (float*)base;
        a.cent = (float*)(base + sec.kp);
        a.cent_w = (float*)(base + sec.kp + sec.cent);
        a.scores = (float*)(base + sec.kp + sec.cent + sec.cw);
        a.ibcs = 1;
        a.ibcs_group = ibcs_q_group / N;
    } else {
        // [split Kp | exponents]
        const NablaSections sec = nabla_sections(a.BH, nb, d);
        a.qp = nullptr;
        a.kp = (float*)workspace;
        a.kexp = (int32_t*)((char*)workspace + sec.kp);
    }
    a.bf16 = dtype == NABLA_BF16;
    a.raster = raster;
    a.H = H;
    a.W = W;
    a.sip_budget = sip_budget;
    a.uniforms = uniforms;
    a.kv_logw = kv_logw;
    if (!use_scratch) return hip_status(nabla::launch_build_mask(a, stream), who);

    // Heads in chunks whose pooled K fits the scratch, each chunk's launches reusing
    // it in stream order; the start order, which reads only the counts, runs once at the end.
    const int per_chunk = (int)(workspace_bytes / head_pool_bytes);
    const size_t head_bytes = (size_t)L * d * elem_size(dtype);
    const size_t words = (size_t)(nb + 31) / 32;
    for (int h0 = 0; h0 < a.BH; h0 += per_chunk) {
        nabla::MaskArgs c = a;
        c.BH = a.BH - h0 < per_chunk ? a.BH - h0 : per_chunk;
        c.q = (const char*)q + (size_t)h0 * head_bytes;
        c.k = (const char*)k + (size_t)h0 * head_bytes;
        c.kv_count = kv_count + (size_t)h0 * nb;
        c.kv_index = kv_index + (size_t)h0 * nb * nb;
        c.bitmap = bitmap ? bitmap + (size_t)h0 * nb * words : nullptr;
        c.schedule = nullptr;
        c.kp = (float*)workspace;
        c.kexp = (int32_t*)((char*)workspace + (size_t)per_chunk * head_kp_bytes);
        nabla_status st = hip_status(nabla::launch_build_mask(c, stream), who);
        if (st != NABLA_OK) return st;
    }
    if (!schedule) return NABLA_OK;
    return hip_status(nabla::launch_pair_schedule(a, kv_count, schedule, stream), who);
}

}  // namespace

namespace {

nabla_status attn_fwd_impl(const char* who, const void* q, const void* k, const void* v, void* o,
                           int batch, int heads, int L, int d, int N, const int32_t* kv_count,
                           const int32_t* kv_index, const int32_t* schedule, float scale,
                           nabla_dtype dtype, float* lse, int raster, int H, int W, hipStream_t stream,
                           const float* kv_logw = nullptr);

}  // namespace

nabla_status block_sparse_attn_fwd(const void* q, const void* k, const void* v, void* o,
                                   int batch, int heads, int L, int d, int N,
                                   const int32_t* kv_count, const int32_t* kv_index,
                                   const int32_t* schedule, float scale, nabla_dtype dtype,
                                   hipStream_t stream) {
    return attn_fwd_impl("block_sparse_attn_fwd", q, k, v, o, batch, heads, L, d, N, kv_count, kv_index,
                         schedule, scale, dtype, nullptr, 0, 0, 0, stream);
}

nabla_status block_sparse_attn_fwd_weighted(const void* q, const void* k, const void* v, void* o,
                                            int batch, int heads, int L, int d, int N,
                                            const int32_t* kv_count, const int32_t* kv_index,
                                            const float* kv_logw, const int32_t* schedule, float scale,
                                            nabla_dtype dtype, hipStream_t stream) {
    const char* who = "block_sparse_attn_fwd_weighted";
    if (!kv_logw) return fail(NABLA_E_INVAL, "%s: null kv_logw", who);
    if ((uintptr_t)kv_logw & 3) return fail(NABLA_E_INVAL, "%s: misaligned kv_logw", who);
    return attn_fwd_impl(who, q, k, v, o, batch, heads, L, d, N, kv_count, kv_index, schedule, scale, dtype,
                         nullptr, 0, 0, 0, stream, kv_logw);
}

nabla_status block_sparse_attn_fwd_raster(const void* q, const void* k, const void* v, void* o,
                                          int batch, int heads, int T, int H, int W, int d, int P, int N,
                                          const int32_t* kv_count, const int32_t* kv_index,
                                          const int32_t* schedule, float scale, nabla_dtype dtype,
                                          hipStream_t stream) {
    const char* who = "block_sparse_attn_fwd_raster";
    int L = 0;
    const nabla_status st = raster_tokens(who, T, H, W, P, N, &L);
    if (st != NABLA_OK) return st;
    return attn_fwd_impl(who, q, k, v, o, batch, heads, L, d, N, kv_count, kv_index, schedule, scale, dtype,
                         nullptr, 1, H, W, stream);
}

nabla_status block_sparse_attn_fwd_lse(const void* q, const void* k, const void* v, void* o,
                                       int batch, int heads, int L, int d, int N,
                                       const int32_t* kv_count, const int32_t* kv_index,
                                       const int32_t* schedule, float scale, nabla_dtype dtype,
                                       float* lse, hipStream_t stream) {
    if (!lse) return fail(NABLA_E_INVAL, "block_sparse_attn_fwd_lse: null lse");
    if (!aligned16(lse)) return fail(NABLA_E_INVAL, "block_sparse_attn_fwd_lse: misaligned lse");
    return attn_fwd_impl("block_sparse_attn_fwd_lse", q, k, v, o, batch, heads, L, d, N, kv_count,
                         kv_index, schedule, scale, dtype, lse, 0, 0, 0, stream);
}

nabla_status block_sparse_attn_fwd_lse_raster(const void* q, const void* k, const void* v, void* o,
                                              int batch, int heads, int T, int H, int W, int d, int P, int N,
                                              const int32_t* kv_count, const int32_t* kv_index,
                                              const int32_t* schedule, float scale, nabla_dtype dtype,
                                              float* lse, hipStream_t stream) {
    const char* who = "block_sparse_attn_fwd_lse_raster";
    if (!lse) return fail(NABLA_E_INVAL, "%s: null lse", who);
    if (!aligned16(lse)) return fail(NABLA_E_INVAL, "%s: misaligned lse", who);
    int L = 0;
    const nabla_status st = raster_tokens(who, T, H, W, P, N, &L);
    if (st != NABLA_OK) return st;
    return attn_fwd_impl(who, q, k, v, o, batch, heads, L, d, N, kv_count, kv_index, schedule, scale, dtype,
                         lse, 1, H, W, stream);
}

size_t nabla_attn_bwd_workspace_size(int batch, int heads, int L, int N) {
    if (batch <= 0 || heads <= 0 || L <= 0 || N <= 0 || L % N) return 0;
    const size_t BH = (size_t)batch * heads, nb = (size_t)(L / N), words = (nb + 31) / 32;
    auto up = [](size_t b) { return (b + 255) & ~(size_t)255; };
    return up(BH * L * 4) + up(BH * nb * words * 4) + up(BH * nb * 4) + up(BH * nb * nb * 4) +
           2 * up(BH * nb * 4);
}

namespace {

nabla_status attn_bwd_impl(const char* who, const void* q, const void* k, const void* v, const void* o,
                           const void* dout, const float* lse, void* dq, void* dk, void* dv, int batch,
                           int heads, int L, int d, int N, const int32_t* kv_count, const int32_t* kv_index,
                           float scale, nabla_dtype dtype, void* workspace, size_t workspace_bytes, int raster,
                           int H, int W, hipStream_t stream) {
    if (!q || !k || !v || !o || !dout || !lse || !dq || !dk || !dv || !kv_count || !kv_index)
        return fail(NABLA_E_INVAL, "%s: null pointer", who);
    if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o) || !aligned16(dout) ||
        !aligned16(lse) || !aligned16(dq) || !aligned16(dk) || !aligned16(dv) || ((uintptr_t)kv_count & 3) ||
        ((uintptr_t)kv_index & 3))
        return fail(NABLA_E_INVAL, "%s: misaligned pointer", who);
    const void* ins[] = {q, k, v, o, dout, lse};
    for (const void* out : {(const void*)dq, (const void*)dk, (const void*)dv}) {
        for (const void* in : ins)
            if (out == in) return fail(NABLA_E_INVAL, "%s: an output aliases an input", who);
    }
    if (dq == dk || dq == dv || dk == dv) return fail(NABLA_E_INVAL, "%s: outputs must differ", who);
    if (batch <= 0 || heads <= 0 || L <= 0 || d <= 0 || N <= 0)
        return fail(NABLA_E_INVAL, "%s: sizes must be positive", who);
    if (L % N) return fail(NABLA_E_INVAL, "%s: L=%d is not a multiple of N=%d", who, L, N);
    if (isnan(scale) || isinf(scale)) return fail(NABLA_E_INVAL, "%s: scale must be finite", who);
    if (!valid_dtype(dtype)) return fail(NABLA_E_INVAL, "%s: unknown dtype %d", who, (int)dtype);
    if (N != 64) return fail(NABLA_E_UNSUPPORTED, "%s: only N = 64 is implemented", who);
    if (d != 64 && d != 128) return fail(NABLA_E_UNSUPPORTED, "%s: d must be 64 or 128", who);
    if (L / N > NABLA_MAX_BLOCKS)
        return fail(NABLA_E_UNSUPPORTED, "%s: %d blocks per head exceed %d", who, L / N, NABLA_MAX_BLOCKS);
    if ((long long)L * d * (long long)elem_size(dtype) >= kMaxHeadBytes ||
        (long long)batch * heads * (L / N) >= (1ll << 31))
        return fail(NABLA_E_UNSUPPORTED, "%s: tensor too large (a head must stay below 2^31 bytes)", who);
    const size_t need = nabla_attn_bwd_workspace_size(batch, heads, L, N);
    if (!workspace || workspace_bytes < need)
        return fail(NABLA_E_WORKSPACE, "%s: workspace of %zu bytes needed, %zu given", who, need,
                    workspace ? workspace_bytes : (size_t)0);
    if ((uintptr_t)workspace & 255) return fail(NABLA_E_INVAL, "%s: workspace must be 256-byte aligned", who);

    nabla::AttnBwdArgs a{};
    a.q = q;
    a.k = k;
    a.v = v;
    a.o = o;
    a.dout = dout;
    a.lse = lse;
    a.dq = dq;
    a.dk = dk;
    a.dv = dv;
    a.BH = batch * heads;
    a.L = L;
    a.nb = L / N;
    a.d = d;
    a.kv_count = kv_count;
    a.kv_index = kv_index;
    a.scale = scale > 0.f ? scale : 1.0f / sqrtf((float)d);
    a.bf16 = dtype == NABLA_BF16;
    a.raster = raster;
    a.H = H;
    a.W = W;
    const size_t BH = (size_t)a.BH, nb = (size_t)a.nb, words = (nb + 31) / 32;
    auto up = [](size_t b) { return (b + 255) & ~(size_t)255; };
    char* w = (char*)workspace;
    a.drow = (float*)w;
    w += up(BH * L * 4);
    a.bits = (uint32_t*)w;
    w += up(BH * nb * words * 4);
    a.q_count = (int32_t*)w;
    w += up(BH * nb * 4);
    a.q_index = (int32_t*)w;
    w += up(BH * nb * nb * 4);
    a.sched_q = (int32_t*)w;
    w += up(BH * nb * 4);
    a.sched_k = (int32_t*)w;
    return hip_status(nabla::launch_attn_bwd(a, stream), who);
}

}  // namespace

nabla_status block_sparse_attn_bwd(const void* q, const void* k, const void* v, const void* o,
                                   const void* dout, const float* lse, void* dq, void* dk, void* dv,
                                   int batch, int heads, int L, int d, int N,
                                   const int32_t* kv_count, const int32_t* kv_index, float scale,
                                   nabla_dtype dtype, void* workspace, size_t workspace_bytes,
                                   hipStream_t stream) {
    return attn_bwd_impl("block_sparse_attn_bwd", q, k, v, o, dout, lse, dq, dk, dv, batch, heads, L, d, N,
                         kv_count, kv_index, scale, dtype, workspace, workspace_bytes, 0, 0, 0, stream);
}

nabla_status block_sparse_attn_bwd_raster(const void* q, const void* k, const void* v, const void* o,
                                          const void* dout, const float* lse, void* dq, void* dk, void* dv,
                                          int batch, int heads, int T, int H, int W, int d, int P, int N,
                                          const int32_t* kv_count, const int32_t* kv_index, float scale,
                                          nabla_dtype dtype, void* workspace, size_t workspace_bytes,
                                          hipStream_t stream) {
    const char* who = "block_sparse_attn_bwd_raster";
    int L = 0;
    const nabla_status st = raster_tokens(who, T, H, W, P, N, &L);
    if (st != NABLA_OK) return st;
    return attn_bwd_impl(who, q, k, v, o, dout, lse, dq, dk, dv, batch, heads, L, d, N, kv_count, kv_index, scale,
                         dtype, workspace, workspace_bytes, 1, H, W, stream);
}

namespace {

nabla_status attn_fwd_impl(const char* who, const void* q, const void* k, const void* v, void* o,
                           int batch, int heads, int L, int d, int N, const int32_t* kv_count,
                           const int32_t* kv_index, const int32_t* schedule, float scale,
                           nabla_dtype dtype, float* lse, int raster, int H, int W, hipStream_t stream,
                           const float* kv_logw) {
    if (!q || !k || !v || !o || !kv_count || !kv_index)
        return fail(NABLA_E_INVAL, "%s: null pointer", who);
    if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o) ||
        ((uintptr_t)kv_count & 3) || ((uintptr_t)kv_index & 3) || ((uintptr_t)schedule & 3))
        return fail(NABLA_E_INVAL, "%s: misaligned pointer", who);
    if (batch <= 0 || heads <= 0 || L <= 0 || d <= 0 || N <= 0)
        return fail(NABLA_E_INVAL, "%s: sizes must be positive", who);
    if (L % N) return fail(NABLA_E_INVAL, "%s: L=%d is not a multiple of N=%d", who, L, N);
    if (isnan(scale) || isinf(scale)) return fail(NABLA_E_INVAL, "%s: scale must be finite", who);
    if (!valid_dtype(dtype)) return fail(NABLA_E_INVAL, "%s: unknown dtype %d", who, (int)dtype);
    if (N != 64) return fail(NABLA_E_UNSUPPORTED, "%s: only N = 64 is implemented", who);
    if (d != 64 && d != 128) return fail(NABLA_E_UNSUPPORTED, "%s: d must be 64 or 128", who);
    if ((long long)L * d * (long long)elem_size(dtype) >= kMaxHeadBytes ||
        (long long)batch * heads * (L / N) >= (1ll << 31))
        return fail(NABLA_E_UNSUPPORTED, "%s: tensor too large (a head must stay below 2^31 bytes)", who);
    nabla::AttnArgs a{};
    a.q = q;
    a.k = k;
    a.v = v;
    a.o = o;
    a.BH = batch * heads;
    a.L = L;
    a.nb = L / N;
    a.d = d;
    a.kv_count = kv_count;
    a.kv_index = kv_index;
    a.schedule = schedule;
    a.scale = scale > 0.f ? scale : 1.0f / sqrtf((float)d);
    a.lse = lse;
    a.raster = raster;
    a.H = H;
    a.W = W;
    a.kv_logw = kv_logw;
    hipError_t e = dtype == NABLA_BF16 ? nabla::launch_attn_bf16(a, stream)
                                       : nabla::launch_attn_f32(a, stream);
    return hip_status(e, who);
}

}  // namespace

}  // extern "C"
