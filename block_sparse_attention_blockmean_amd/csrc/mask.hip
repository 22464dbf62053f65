// Adaptive block mask (NABLA technical summary, "Metodologia: NABLA", item 2, with the
// STA union of item 3):
//   pool_kernel        block means of Q and K (one HBM pass over both, float32 sums)
//   map_select_kernel  reduced map S = Qp Kp^T * scale on float32 MFMA, row softmax,
//                      then per row (select_row) the CDF cutoff found by bisection on
//                      float32 bit patterns (or SIP sampling), the STA OR, and
//                      compaction into an ascending kept list
// With IBCS block scores the rows of the map are the 8 cluster centroids of each query
// group (ibcs.hip) instead of its mean: ibcs_score_kernel writes each group's score row,
// the weighted sum of its centroids' softmax rows, and select_kernel applies select_row
// to those rows; the cut and the lists are the same.
#include <math.h>

#include "attn_tile.h"
#include "nabla_internal.h"

namespace nabla {
namespace {

typedef float f32x4 __attribute__((ext_vector_type(4)));

// ---------------------------------------------------------------------------
// Block-mean pooling.  One wave per (tensor, head, block): lane l reads 16-byte
// chunk (l % CHUNKS) of tokens (l / CHUNKS), (l / CHUNKS) + G, ... so each load
// instruction covers G whole token rows; per-lane sums run in token order and the
// G partial sums are combined by a fixed butterfly, so the result is deterministic.
// ---------------------------------------------------------------------------
template <typename T>
struct Elem;
template <>
struct Elem<__bf16> {
    static constexpr int kPerChunk = 8;
    __device__ static inline void unpack(const u32x4& v, float* out) {
        const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            out[2 * i] = __uint_as_float(w[i] << 16);
            out[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
        }
    }
};
template <>
struct Elem<float> {
    static constexpr int kPerChunk = 4;
    __device__ static inline void unpack(const u32x4& v, float* out) {
        out[0] = __uint_as_float(v.x);
        out[1] = __uint_as_float(v.y);
        out[2] = __uint_as_float(v.z);
        out[3] = __uint_as_float(v.w);
    }
};

template <typename T, int D, int N, bool RASTER>
__global__ __launch_bounds__(256) void pool_kernel(const T* __restrict__ q,
                                                    const T* __restrict__ k,
                                                    float* __restrict__ qp,
                                                    float* __restrict__ kp, int total_blocks, int nb,
                                                    int L, attn::RasterGrid grid, int first_wave) {
    constexpr int EPC = Elem<T>::kPerChunk;
    constexpr int CHUNKS = D / EPC;          // 16-byte chunks per token
    constexpr int G = 64 / CHUNKS;           // tokens per load instruction
    constexpr int ITERS = N / G;
    const int wave = first_wave + ((blockIdx.x * 256 + threadIdx.x) >> 6);
    const int lane = threadIdx.x & 63;
    if (wave >= 2 * total_blocks) return;
    const bool is_k = wave >= total_blocks;
    const int blk = is_k ? wave - total_blocks : wave;
    // the block's first row: fractal order, runs of N rows; raster order, one 8 x 8 patch
    const T* src;
    if (RASTER) {
        const int bh = blk / nb;
        src = (is_k ? k : q) + ((size_t)bh * L + attn::block_row<true>(grid, blk - bh * nb)) * D;
    } else {
        src = (is_k ? k : q) + (size_t)blk * N * D;
    }
    float* dst = (is_k ? kp : qp) + (size_t)blk * D;
    const int c = lane % CHUNKS;
    const int g = lane / CHUNKS;

    u32x4 raw[ITERS];
#pragma unroll
    for (int r = 0; r < ITERS; ++r) {
        raw[r] = __builtin_nontemporal_load(
            reinterpret_cast<const u32x4*>(src + (size_t)attn::row_in_block<RASTER>(grid, r * G + g) * D) + c);
    }
    float acc[EPC];
#pragma unroll
    for (int e = 0; e < EPC; ++e) acc[e] = 0.f;
#pragma unroll
    for (int r = 0; r < ITERS; ++r) {
        float v[EPC];
        Elem<T>::unpack(raw[r], v);
#pragma unroll
        for (int e = 0; e < EPC; ++e) acc[e] += v[e];
    }
#pragma unroll
    for (int off = CHUNKS; off < 64; off <<= 1) {
#pragma unroll
        for (int e = 0; e < EPC; ++e) acc[e] += __shfl_xor(acc[e], off);
    }
    if (g == 0) {
        constexpr float inv = 1.0f / N;      // N is a power of two: exact
        float* o = dst + c * EPC;
#pragma unroll
        for (int e = 0; e < EPC; e += 4) {
            *reinterpret_cast<f32x4*>(o + e) =
                f32x4{acc[e] * inv, acc[e + 1] * inv, acc[e + 2] * inv, acc[e + 3] * inv};
        }
    }
}

// ---------------------------------------------------------------------------
// Reduced map, then the cut.
// The map kernels hold kRows = 16 rows of S per workgroup (the M of the 16x16 float32
//   MFMA).
// The cut (select_row) takes one row in one wave.  Keeping block j iff F_j > thr is the
//   same as keeping every block whose probability is at least v*, the smallest row
//   value with g(v*) > thr, where g(u) = sum of the row values <= u.  g only grows with
//   u, and non-negative floats order like their bit patterns, so v* is found by
//   bisection over bit patterns.  The search starts at u0 = thr / nb (g(u0) <= nb u0 =
//   thr) and keeps only the values still inside the bracket (compacted into a per-wave
//   LDS buffer), so each step touches fewer values and the search stops once a single
//   candidate is left.  All sums run in a fixed order, so the result is deterministic.
// ---------------------------------------------------------------------------
constexpr int kRows = 16;
constexpr int kCap = 256;   // candidates per wave held in LDS

// Wave-wide reductions on DPP: shifts of 1, 2, 4, 8 lanes inside each 16-lane row, then
// the row broadcasts of lanes 15 and 31 (a fixed order, so the result is deterministic);
// lane 63 ends with the total, which every lane then reads.  VALU latency only, no LDS.
template <int CTRL, int ROWS>
__device__ inline int dpp_i(int identity, int x) {
    return __builtin_amdgcn_update_dpp(identity, x, CTRL, ROWS, 0xf, false);
}
template <typename Op>
__device__ inline int wave_reduce_bits(int x, int identity, Op op) {
    x = op(x, dpp_i<0x111, 0xf>(identity, x));   // row_shr:1
    x = op(x, dpp_i<0x112, 0xf>(identity, x));   // row_shr:2
    x = op(x, dpp_i<0x114, 0xf>(identity, x));   // row_shr:4
    x = op(x, dpp_i<0x118, 0xf>(identity, x));   // row_shr:8
    x = op(x, dpp_i<0x142, 0xa>(identity, x));   // row_bcast:15 into rows 1, 3
    x = op(x, dpp_i<0x143, 0xc>(identity, x));   // row_bcast:31 into rows 2, 3
    return __builtin_amdgcn_readlane(x, 63);
}
__device__ inline float wave_sum(float x) {
    return __int_as_float(wave_reduce_bits(__float_as_int(x), 0, [](int a, int b) {
        return __float_as_int(__int_as_float(a) + __int_as_float(b));
    }));
}
__device__ inline float wave_max(float x) {
    return __int_as_float(wave_reduce_bits(__float_as_int(x), __float_as_int(-INFINITY), [](int a, int b) {
        return __float_as_int(fmaxf(__int_as_float(a), __int_as_float(b)));
    }));
}
__device__ inline uint32_t wave_max_u(uint32_t x) {
    return (uint32_t)wave_reduce_bits((int)x, 0, [](int a, int b) { return (int)max((uint32_t)a, (uint32_t)b); });
}

// Writes the values of src[0..len) whose bit pattern lies in (lo, hi] to dst, in
// order; src may equal dst (each write lands at or before its source).
__device__ inline int compact(const float* src, int len, uint32_t lo, uint32_t hi, float* dst,
                              int lane) {
    int n = 0;
    for (int j0 = 0; j0 < len; j0 += 64) {
        const int j = j0 + lane;
        const float x = (j < len) ? src[j] : 0.f;
        const uint32_t b = __float_as_uint(x);
        const bool in = (j < len) && b > lo && b <= hi;
        const uint64_t ballot = __ballot(in);
        if (in) dst[n + __popcll(ballot & ((1ull << lane) - 1ull))] = x;
        n += __popcll(ballot);
    }
    return n;
}

// ---------------------------------------------------------------------------
// SIP (AB-Attention page, "Os três recursos do AB-Attention", second feature) on one
// row of block scores A (the pooled softmax), in one wave: block j is kept with
// probability pi_j proportional to A_j and capped at 1, and carries the logit shift
// log(1 / pi_j), the Horvitz-Thompson weight.  The row's top block (smallest index
// among equal maxima) is certain; the others share budget - 1 through
// pi_j = min(1, c A_j), the water level c found by growing the set of certain blocks
// (c only increases as blocks become certain, so the set only grows).  Kept iff the
// given uniform draw u_j < pi_j.
// ---------------------------------------------------------------------------
__device__ void sip_row(float* arow, int nb, float inv_sum, int budget, const float* u, int32_t* out_idx,
                        float* out_logw, uint32_t* out_bits, int nwords, int32_t* out_count, int lane) {
    float best = -1.f;
    int bj = nb;
    for (int j = lane; j < nb; j += 64) {
        const float p = arow[j] * inv_sum;
        arow[j] = p;
        if (p > best) {
            best = p;
            bj = j;
        }
    }
    const float amax = wave_max(best);
    const int top = (int)~wave_max_u(~(uint32_t)(best == amax ? bj : nb));
    const int kp = budget - 1;
    const bool all = budget >= nb;
    // water level over the blocks other than the top one
    float c = 0.f, c_cert = 0.f;
    if (!all && kp > 0) {
        float rest = 0.f;
        for (int j = lane; j < nb; j += 64)
            if (j != top) rest += arow[j];
        rest = wave_sum(rest);
        c = rest > 0.f ? (float)kp / rest : 0.f;
        c_cert = c;
        int m = 0;
        for (int it = 0; it < 64; ++it) {
            float unc = 0.f;   // mass of the blocks still below 1
            int cnt = 0;
            for (int j0 = 0; j0 < nb; j0 += 64) {
                const int j = j0 + lane;
                const bool other = j < nb && j != top;
                const bool cert = other && c * arow[j] >= 1.f;
                if (other && !cert) unc += arow[j];
                cnt += __popcll(__ballot(cert));
            }
            unc = wave_sum(unc);
            if (cnt == m) {
                c_cert = c;
                break;
            }
            m = cnt;
            c_cert = c;
            if (m >= kp || !(unc > 0.f)) {
                c = 0.f;
                break;
            }
            c = (float)(kp - m) / unc;
        }
    }
    int base = 0;
    for (int j0 = 0; j0 < nb; j0 += 64) {
        const int j = j0 + lane;
        bool keep = false;
        float pi = 0.f;
        if (j < nb) {
            const float a = arow[j];
            pi = (all || j == top || c_cert * a >= 1.f) ? 1.f : c * a;
            keep = u[j] < pi;
        }
        const uint64_t ballot = __ballot(keep);
        if (keep) {
            const int pos = base + __popcll(ballot & ((1ull << lane) - 1ull));
            out_idx[pos] = j;
            out_logw[pos] = -logf(pi);
        }
        base += __popcll(ballot);
        if (out_bits) {
            const int w = j0 >> 5;
            if (lane == 0 && w < nwords) out_bits[w] = (uint32_t)ballot;
            if (lane == 1 && w + 1 < nwords) out_bits[w + 1] = (uint32_t)(ballot >> 32);
        }
    }
    if (lane == 0) *out_count = base;
}

// ---------------------------------------------------------------------------
// Rows of the reduced map: S[r][j] = scale * X[r] . Kp_j for the workgroup's kRows rows
// r, parked in LDS rows of ld_s floats.  The kRows X rows sit in LDS (x_lds, rows of
// d + 4 floats: row r starts 4 r banks on, so the 16 rows of one 16-byte read fall in
// distinct banks), staged once by the whole workgroup (rows past the last are zeros).
// The NW waves take column tiles of 16 blocks in turn with v_mfma_f32_16x16x4_f32
// (float32 operands and accumulation).  Lane (row l % 16, group g = l / 16) supplies
// coordinate 16 v + 4 g + i of its row at MFMA step 4 v + i, in both operands: each
// 16-byte load instruction then reads 64 contiguous bytes of each of 16 rows (16 cache
// lines), where a contiguous quarter of d per lane would touch 64 lines per instruction
// and leave the loads bound by the texture unit's per-line rate.  A wave holds half a
// column tile's Kp operand at a time: about 35 VGPRs, so 16-wave workgroups run two to
// a CU, and one's loads and barrier waits overlap the other's work.
// ---------------------------------------------------------------------------
template <int D>
constexpr int kXld = D + 4;

// Stages rows row0 .. row0 + kRows - 1 of X [n_rows, D] (zeros past the last) into x_lds.
template <int D, int NT>
__device__ inline void stage_rows(const float* __restrict__ xh, int n_rows, int row0, float* x_lds) {
    for (int e = threadIdx.x; e < kRows * D / 4; e += NT) {
        const int r = e / (D / 4), c4 = e % (D / 4);
        f32x4 v = {0.f, 0.f, 0.f, 0.f};
        if (row0 + r < n_rows) v = reinterpret_cast<const f32x4*>(xh + (size_t)(row0 + r) * D)[c4];
        *reinterpret_cast<f32x4*>(x_lds + r * kXld<D> + 4 * c4) = v;
    }
}

template <int D, int NW>
__device__ inline void map_rows(const float* __restrict__ x_lds, const float* __restrict__ kh, int nb, int ld_s,
                                   float scale, float* s_lds, int wave, int lane) {
    constexpr int KC = D / 4;
    const int li = lane & 15;
    const int kq = lane >> 4;
    const f32x4* xa = reinterpret_cast<const f32x4*>(x_lds + li * kXld<D>) + kq;
    const int n_ct = (nb + 15) / 16;
    for (int ct = wave; ct < n_ct; ct += NW) {
        const int j = ct * 16 + li;
        const f32x4* src = reinterpret_cast<const f32x4*>(kh + (size_t)min(j, nb - 1) * D) + kq;
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
        // the K operand in two halves of d (16 values per lane each)
#pragma unroll 1
        for (int h = 0; h < 2; ++h) {
            f32x4 b[KC / 8];
#pragma unroll
            for (int v = 0; v < KC / 8; ++v) {
                b[v] = src[4 * (h * (KC / 8) + v)];
                if (j >= nb) b[v] = f32x4{0.f, 0.f, 0.f, 0.f};
            }
#pragma unroll
            for (int v = 0; v < KC / 8; ++v) {
                const f32x4 a = xa[4 * (h * (KC / 8) + v)];
#pragma unroll
                for (int i = 0; i < 4; ++i) acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a[i], b[v][i], acc, 0, 0, 0);
            }
        }
        if (j < nb) {
#pragma unroll
            for (int r = 0; r < 4; ++r) s_lds[(4 * kq + r) * ld_s + j] = acc[r] * scale;
        }
    }
}

constexpr float kLog2e = 1.4426950408889634f;

// ---------------------------------------------------------------------------
// IBCS scores.  A workgroup owns kRows centroid rows (kRows / 8 query groups) of one
// head: the centroid rows staged in LDS and the map by map_rows; per row the maximum
// and the softmax normaliser (one wave per row); then each group's row A = sum of its 8
// rows' w_c softmax in cluster order, the exponentials recomputed there rather than
// stored, written to A_out [BH, groups, nb] for the select kernel.  Rows sum to one.
// Sixteen waves and the LDS-staged operand (35 VGPRs) let two workgroups share a CU.
// ---------------------------------------------------------------------------
static_assert(kRows % kIbcsClusters == 0, "a workgroup holds whole query blocks' centroids");
constexpr int kScoreWaves = 16;

template <int D>
__global__ __launch_bounds__(kScoreWaves * 64) __attribute__((amdgpu_waves_per_eu(8, 8))) void ibcs_score_kernel(
    const float* __restrict__ cent, const float* __restrict__ cw, const float* __restrict__ kp, int nb, int groups,
    int ld_s, float scale, float* __restrict__ A_out) {
    // [kRows][ld_s] rows, then [kRows][kXld] centroid rows
    extern __shared__ __align__(16) float s_lds[];
    const int wave = threadIdx.x >> 6;
    const int lane = threadIdx.x & 63;
    const int bh = blockIdx.y;
    const int row0 = blockIdx.x * kRows;
    const int n_rows = groups * kIbcsClusters;
    float* x_lds = s_lds + kRows * ld_s;
    stage_rows<D, kScoreWaves * 64>(cent + (size_t)bh * n_rows * D, n_rows, row0, x_lds);
    __syncthreads();
    map_rows<D, kScoreWaves>(x_lds, kp + (size_t)bh * nb * D, nb, ld_s, scale, s_lds, wave, lane);
    __syncthreads();
    // per centroid row: the maximum m_c and the factor w_c / sum_j exp(S_cj - m_c)
    __shared__ float fac[kRows], mx2[kRows];
    for (int r = wave; r < kRows; r += kScoreWaves) {
        const int crow = row0 + r;
        float f = 0.f, m2 = 0.f;
        if (crow < n_rows) {
            const float* srow = s_lds + r * ld_s;
            float mx = -INFINITY;
            for (int j = lane; j < nb; j += 64) mx = fmaxf(mx, srow[j]);
            m2 = wave_max(mx) * kLog2e;
            float sum = 0.f;
            for (int j = lane; j < nb; j += 64) sum += __builtin_amdgcn_exp2f(fmaf(srow[j], kLog2e, -m2));
            f = cw[(size_t)bh * n_rows + crow] / wave_sum(sum);
        }
        if (lane == 0) {
            fac[r] = f;
            mx2[r] = m2;
        }
    }
    __syncthreads();
    // A_gj = sum over the group's clusters, in cluster order, of w_c softmax_j(S_c)
    for (int r = 0; r < kRows / kIbcsClusters; ++r) {
        const int row = row0 / kIbcsClusters + r;
        if (row >= groups) break;
        const float* grp = s_lds + r * kIbcsClusters * ld_s;
        float* out = A_out + ((size_t)bh * groups + row) * nb;
        for (int j = threadIdx.x; j < nb; j += kScoreWaves * 64) {
            float a = 0.f;
#pragma unroll
            for (int c = 0; c < kIbcsClusters; ++c) {
                const int rc = r * kIbcsClusters + c;
                a = fmaf(fac[rc], __builtin_amdgcn_exp2f(fmaf(grp[c * ld_s + j], kLog2e, -mx2[rc])), a);
            }
            out[j] = a;
        }
    }
}

// ---------------------------------------------------------------------------
// The cut of one row, in one wave: `arow` (LDS) holds the row's values, inv_sum times
// which are its probabilities A (summing to one; the product is written back on the
// first pass), `cand` is the wave's candidate buffer.  SIP sampling when
// sip_budget > 0, else the CDF cut; then the STA OR and the ascending list, count and
// bitmap of query block `row` of head bh.
// ---------------------------------------------------------------------------
__device__ void select_row(float* arow, float inv_sum, float* cand, int nb, int bh, int row, float thr, int sta,
                           int nH, int nW, int rt, int rh, int rw, int32_t* __restrict__ kv_count,
                           int32_t* __restrict__ kv_index, uint32_t* __restrict__ bitmap, int sip_budget,
                           const float* __restrict__ uniforms, float* __restrict__ kv_logw, int lane) {
    const int nwords = (nb + 31) >> 5;
    if (sip_budget > 0) {
        sip_row(arow, nb, inv_sum, sip_budget, uniforms + ((size_t)bh * nb + row) * nb,
                kv_index + ((size_t)bh * nb + row) * nb, kv_logw + ((size_t)bh * nb + row) * nb,
                bitmap ? bitmap + ((size_t)bh * nb + row) * nwords : nullptr, nwords,
                kv_count + (size_t)bh * nb + row, lane);
        return;
    }
    // start of the bracket: u0 = thr / nb, nudged down so rounding cannot push
    // g(u0) above thr; it is verified below and dropped to 0 if it fails
    uint32_t lo = __float_as_uint(thr / ((float)nb * 1.0001f));
    float g_lo = 0.f;
    int n_in = 0;
    uint32_t maxb = 0;
    for (int j0 = 0; j0 < nb; j0 += 64) {
        const int j = j0 + lane;
        bool in = false;
        if (j < nb) {
            const float p = arow[j] * inv_sum;
            arow[j] = p;
            const uint32_t b = __float_as_uint(p);
            maxb = max(maxb, b);
            if (b <= lo) g_lo += p; else in = true;
        }
        n_in += __popcll(__ballot(in));
    }
    g_lo = wave_sum(g_lo);
    maxb = wave_max_u(maxb);
    if (g_lo > thr) {   // cannot happen in exact arithmetic; fall back to g(0) = 0
        lo = 0;
        g_lo = 0.f;
        n_in = 0;
        for (int j0 = 0; j0 < nb; j0 += 64) {
            const int j = j0 + lane;
            n_in += __popcll(__ballot(j < nb && __float_as_uint(arow[j]) > 0u));
        }
    }
    uint32_t hi = maxb;
    // bracket (lo, hi]: g(lo) = g_lo <= thr and, unless the whole row sums to at
    // most thr, g(hi) > thr; n_in values lie inside it (always >= 1: the maximum)
    const float* src = arow;
    int len = nb;
    if (n_in <= kCap) {
        len = compact(arow, nb, lo, hi, cand, lane);
        src = cand;
    }
    // bisection until at most 64 values are left in the bracket
    while (hi - lo > 1 && n_in > 64) {
        const uint32_t mid = lo + ((hi - lo) >> 1);
        float s_ = 0.f;
        int c = 0;
        for (int j0 = 0; j0 < len; j0 += 64) {
            const int j = j0 + lane;
            const float x = (j < len) ? src[j] : 0.f;
            const uint32_t b = __float_as_uint(x);
            const bool in = (j < len) && b > lo && b <= mid;
            if (in) s_ += x;
            c += __popcll(__ballot(in));
        }
        s_ = wave_sum(s_);
        if (g_lo + s_ > thr) {
            hi = mid;
            n_in = c;
        } else {
            lo = mid;
            g_lo += s_;
            n_in -= c;
        }
        if (n_in <= kCap && 2 * n_in <= len) {
            len = compact(src, len, lo, hi, cand, lane);
            src = cand;
        }
    }
    uint32_t cut = hi;
    if (n_in <= 64) {
        // one candidate per lane: F(x) = g_lo + (sum of the candidates <= x), tied
        // values together; the cut is the smallest candidate with F(x) > thr
        len = compact(src, len, lo, hi, cand, lane);
        const float x = lane < len ? cand[lane] : 0.f;
        const uint32_t bx = __float_as_uint(x);
        float below = 0.f;
        for (int m = 0; m < len; ++m) {
            const float y = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), m));
            if (__float_as_uint(y) <= bx) below += y;
        }
        const bool crosses = lane < len && g_lo + below > thr;
        const uint32_t pick = crosses ? bx : 0xffffffffu;
        const uint32_t best = ~wave_max_u(~pick);   // smallest pattern among the crossing ones
        if (best != 0xffffffffu) cut = best;
    }

    int qt = 0, qh_ = 0, qw = 0;
    const int pf = nH * nW;
    if (sta) {
        qt = row / pf;
        const int rem = row - qt * pf;
        qh_ = rem / nW;
        qw = rem - qh_ * nW;
    }
    int32_t* out_idx = kv_index + ((size_t)bh * nb + row) * nb;
    uint32_t* out_bits = bitmap ? bitmap + ((size_t)bh * nb + row) * nwords : nullptr;
    int base = 0;
    for (int j0 = 0; j0 < nb; j0 += 64) {
        const int j = j0 + lane;
        bool keep = false;
        if (j < nb) {
            keep = __float_as_uint(arow[j]) >= cut;
            if (sta && !keep) {
                const int kt = j / pf;
                const int rem = j - kt * pf;
                const int kh_ = rem / nW;
                const int kw = rem - kh_ * nW;
                keep = abs(kt - qt) <= rt && abs(kh_ - qh_) <= rh && abs(kw - qw) <= rw;
            }
        }
        const uint64_t ballot = __ballot(keep);
        if (keep) out_idx[base + __popcll(ballot & ((1ull << lane) - 1ull))] = j;
        base += __popcll(ballot);
        if (out_bits) {
            const int w = j0 >> 5;
            if (lane == 0 && w < nwords) out_bits[w] = (uint32_t)ballot;
            if (lane == 1 && w + 1 < nwords) out_bits[w + 1] = (uint32_t)(ballot >> 32);
        }
    }
    if (lane == 0) kv_count[(size_t)bh * nb + row] = base;
}

// ---------------------------------------------------------------------------
// NABLA's reduced map and cut in one kernel.  A workgroup (16 waves) owns kRows pooled
// query rows of one head: the map by map_rows, then per row (one wave) the softmax
// A = exp(S - max) / sum in place and select_row.  The rows never leave LDS, which at
// large nb (nb^2 floats per head) saves an HBM round trip.
// ---------------------------------------------------------------------------
constexpr int kWaves = 16;

template <int D>
__global__ __launch_bounds__(kWaves * 64) __attribute__((amdgpu_waves_per_eu(8, 8))) void map_select_kernel(
    const float* __restrict__ qp, const float* __restrict__ kp, int nb, int ld_s, float scale, float thr, int sta,
    int nH, int nW, int rt, int rh, int rw, int32_t* __restrict__ kv_count, int32_t* __restrict__ kv_index,
    uint32_t* __restrict__ bitmap, int sip_budget, const float* __restrict__ uniforms,
    float* __restrict__ kv_logw) {
    // [kRows][ld_s] rows, then [kWaves][kCap] candidates, then [kRows][kXld] pooled queries
    extern __shared__ __align__(16) float s_lds[];
    const int wave = threadIdx.x >> 6;
    const int lane = threadIdx.x & 63;
    const int bh = blockIdx.y;
    const int row0 = blockIdx.x * kRows;
    float* x_lds = s_lds + kRows * ld_s + kWaves * kCap;
    stage_rows<D, kWaves * 64>(qp + (size_t)bh * nb * D, nb, row0, x_lds);
    __syncthreads();
    map_rows<D, kWaves>(x_lds, kp + (size_t)bh * nb * D, nb, ld_s, scale, s_lds, wave, lane);
    __syncthreads();
    float* cand = s_lds + kRows * ld_s + wave * kCap;
    for (int r = wave; r < kRows; r += kWaves) {
        const int row = row0 + r;
        if (row >= nb) break;
        float* arow = s_lds + r * ld_s;
        float mx = -INFINITY;
        for (int j = lane; j < nb; j += 64) mx = fmaxf(mx, arow[j]);
        const float mx2 = wave_max(mx) * kLog2e;
        float sum = 0.f;
        for (int j = lane; j < nb; j += 64) {
            const float e = __builtin_amdgcn_exp2f(fmaf(arow[j], kLog2e, -mx2));
            arow[j] = e;
            sum += e;
        }
        const float inv_sum = 1.0f / wave_sum(sum);
        select_row(arow, inv_sum, cand, nb, bh, row, thr, sta, nH, nW, rt, rh, rw, kv_count, kv_index, bitmap,
                   sip_budget, uniforms, kv_logw, lane);
    }
}

// ---------------------------------------------------------------------------
// Cut of score rows computed elsewhere (IBCS): one wave per query block, its row
// (row i / a_group of A [BH, nb / a_group, nb], summing to one) copied into the wave's
// LDS row, then select_row.  Waves share nothing, so the workgroup never synchronises.
// ---------------------------------------------------------------------------
constexpr int kSelWaves = 4;

__global__ __launch_bounds__(kSelWaves * 64) void select_kernel(
    const float* __restrict__ A, int a_group, int nb, int ld_s, float thr, int sta, int nH, int nW, int rt, int rh,
    int rw, int32_t* __restrict__ kv_count, int32_t* __restrict__ kv_index, uint32_t* __restrict__ bitmap,
    int sip_budget, const float* __restrict__ uniforms, float* __restrict__ kv_logw) {
    extern __shared__ float s_lds[];   // [kSelWaves][ld_s] rows, then [kSelWaves][kCap] candidates
    const int wave = threadIdx.x >> 6;
    const int lane = threadIdx.x & 63;
    const int bh = blockIdx.y;
    const int row = blockIdx.x * kSelWaves + wave;
    if (row >= nb) return;
    float* arow = s_lds + wave * ld_s;
    const float* src = A + ((size_t)bh * (nb / a_group) + row / a_group) * nb;
    for (int j = lane; j < nb; j += 64) arow[j] = src[j];
    select_row(arow, 1.0f, s_lds + kSelWaves * ld_s + wave * kCap, nb, bh, row, thr, sta, nH, nW, rt, rh, rw,
               kv_count, kv_index, bitmap, sip_budget, uniforms, kv_logw, lane);
}

// ---------------------------------------------------------------------------
// Work order for the attention launch: heads one after another, and inside a head its
// query blocks by decreasing kept count.  Consecutive workgroups are dealt round-robin
// to the 8 XCDs, so all of them work on the same one or two heads at any time: the
// K/V tiles in flight are those of one or two heads (tens of MB at the 720p shapes),
// which the last-level cache holds, and each head's short lists run last, which keeps
// the tail of the launch short.  One wave per head (counting sort on nb + 1 bins).
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(64) void schedule_kernel(const int32_t* __restrict__ kv_count, int nb,
                                                      int32_t* __restrict__ schedule) {
    extern __shared__ int bins[];   // nb + 1 counters
    const int h = blockIdx.x;
    const int lane = threadIdx.x;
    const int32_t* cnt = kv_count + (size_t)h * nb;
    for (int b = lane; b <= nb; b += 64) bins[b] = 0;
    __syncthreads();
    for (int i = lane; i < nb; i += 64) atomicAdd(&bins[nb - min(max(cnt[i], 0), nb)], 1);
    __syncthreads();
    // exclusive prefix sum over the nb + 1 bins: one contiguous chunk per lane
    const int per = (nb + 1 + 63) / 64;
    const int b0 = lane * per, b1 = min(b0 + per, nb + 1);
    int local = 0;
    for (int b = b0; b < b1; ++b) local += bins[b];
    int incl = local;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
        const int y = __shfl_up(incl, off);
        if (lane >= off) incl += y;
    }
    int run = incl - local;
    for (int b = b0; b < b1; ++b) {
        const int n = bins[b];
        bins[b] = run;
        run += n;
    }
    __syncthreads();
    for (int i = lane; i < nb; i += 64) {
        const int pos = atomicAdd(&bins[nb - min(max(cnt[i], 0), nb)], 1);
        schedule[(size_t)h * nb + pos] = h * nb + i;
    }
}

template <typename T, int D>
hipError_t launch_pool(const MaskArgs& a, hipStream_t s) {
    const int total = a.BH * a.nb;
    const int waves = 2 * total;
    const int first = a.ibcs ? total : 0;   // IBCS clusters Q instead of pooling it
    attn::RasterGrid grid{};
    if (a.raster) {
        grid.W = (uint32_t)a.W;
        grid.HW = (uint32_t)(a.H * a.W);
        grid.nHW = FastDiv((uint32_t)(a.nH * a.nW));
        grid.nW = FastDiv((uint32_t)a.nW);
        hipLaunchKernelGGL((pool_kernel<T, D, 64, true>), dim3((waves - first + 3) / 4), dim3(256), 0, s,
                           (const T*)a.q, (const T*)a.k, a.qp, a.kp, total, a.nb, a.nb * 64, grid, first);
    } else {
        hipLaunchKernelGGL((pool_kernel<T, D, 64, false>), dim3((waves - first + 3) / 4), dim3(256), 0, s,
                           (const T*)a.q, (const T*)a.k, a.qp, a.kp, total, a.nb, a.nb * 64, grid, first);
    }
    return hipGetLastError();
}

template <int D>
hipError_t launch_map_select(const MaskArgs& a, hipStream_t s) {
    const int ld_s = ((a.nb + 63) / 64) * 64 + 16;
    const size_t lds = ((size_t)kRows * ld_s + (size_t)kWaves * kCap + (size_t)kRows * kXld<D>) * sizeof(float);
    static std::atomic<uint64_t> lds_set{0};
    const int max_lds =
        (kRows * (((NABLA_MAX_BLOCKS + 63) / 64) * 64 + 16) + kWaves * kCap + kRows * kXld<D>) * (int)sizeof(float);
    static_assert((kRows * (((NABLA_MAX_BLOCKS + 63) / 64) * 64 + 16) + kWaves * kCap + kRows * kXld<128>) *
                          sizeof(float) <= 160 * 1024,
                  "map/select LDS at the largest nb");
    hipError_t e = set_max_dynamic_lds((const void*)map_select_kernel<D>, max_lds, lds_set);
    if (e != hipSuccess) return e;
    dim3 grid((a.nb + kRows - 1) / kRows, a.BH);
    hipLaunchKernelGGL((map_select_kernel<D>), grid, dim3(kWaves * 64), lds, s, a.qp, a.kp, a.nb, ld_s, a.scale,
                       a.thr, a.sta, a.nH, a.nW, a.rt, a.rh, a.rw, a.kv_count, a.kv_index, a.bitmap, a.sip_budget,
                       a.uniforms, a.kv_logw);
    return hipGetLastError();
}

hipError_t launch_select(const MaskArgs& a, hipStream_t s) {
    const int ld_s = ((a.nb + 63) / 64) * 64 + 16;
    const size_t lds = ((size_t)kSelWaves * ld_s + (size_t)kSelWaves * kCap) * sizeof(float);
    static std::atomic<uint64_t> lds_set{0};
    const int max_lds = (kSelWaves * (((NABLA_MAX_BLOCKS + 63) / 64) * 64 + 16) + kSelWaves * kCap) * (int)sizeof(float);
    hipError_t e = set_max_dynamic_lds((const void*)select_kernel, max_lds, lds_set);
    if (e != hipSuccess) return e;
    dim3 grid((a.nb + kSelWaves - 1) / kSelWaves, a.BH);
    hipLaunchKernelGGL(select_kernel, grid, dim3(kSelWaves * 64), lds, s, a.scores, a.ibcs_group, a.nb,
                       ld_s, a.thr, a.sta, a.nH, a.nW, a.rt, a.rh, a.rw, a.kv_count, a.kv_index, a.bitmap,
                       a.sip_budget, a.uniforms, a.kv_logw);
    return hipGetLastError();
}

template <int D>
hipError_t launch_ibcs_score(const MaskArgs& a, hipStream_t s) {
    const int ld_s = ((a.nb + 63) / 64) * 64 + 16;
    const size_t lds = ((size_t)kRows * ld_s + (size_t)kRows * kXld<D>) * sizeof(float);
    static std::atomic<uint64_t> lds_set{0};
    const int max_lds = (kRows * (((NABLA_MAX_BLOCKS + 63) / 64) * 64 + 16) + kRows * kXld<D>) * (int)sizeof(float);
    hipError_t e = set_max_dynamic_lds((const void*)ibcs_score_kernel<D>, max_lds, lds_set);
    if (e != hipSuccess) return e;
    const int groups = a.nb / a.ibcs_group;
    dim3 grid((groups * kIbcsClusters + kRows - 1) / kRows, a.BH);
    hipLaunchKernelGGL((ibcs_score_kernel<D>), grid, dim3(kScoreWaves * 64), lds, s, a.cent, a.cent_w, a.kp, a.nb,
                       groups, ld_s, a.scale, a.scores);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_build_mask(const MaskArgs& a, hipStream_t s) {
    hipError_t e;
    if (a.bf16) {
        e = (a.d == 128) ? launch_pool<__bf16, 128>(a, s) : launch_pool<__bf16, 64>(a, s);
    } else {
        e = (a.d == 128) ? launch_pool<float, 128>(a, s) : launch_pool<float, 64>(a, s);
    }
    if (e != hipSuccess) return e;
    if (a.ibcs) {
        if ((e = launch_ibcs_cluster(a, s)) != hipSuccess) return e;
        e = (a.d == 128) ? launch_ibcs_score<128>(a, s) : launch_ibcs_score<64>(a, s);
        if (e == hipSuccess) e = launch_select(a, s);
    } else {
        e = (a.d == 128) ? launch_map_select<128>(a, s) : launch_map_select<64>(a, s);
    }
    if (e != hipSuccess || !a.schedule) return e;
    // one wave per head; its bins fit the default LDS limit (NABLA_MAX_BLOCKS + 1 ints)
    return launch_schedule(a.kv_count, a.BH, a.nb, a.schedule, s);
}

hipError_t launch_schedule(const int32_t* counts, int BH, int nb, int32_t* schedule, hipStream_t s) {
    hipLaunchKernelGGL(schedule_kernel, dim3(BH), dim3(64), (size_t)(nb + 1) * sizeof(int), s, counts, nb,
                       schedule);
    return hipGetLastError();
}

}  // namespace nabla
