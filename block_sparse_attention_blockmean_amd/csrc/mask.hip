// Adaptive block mask (NABLA technical summary, "Metodologia: NABLA", item 2, with the
// STA union of item 3):
//   pool_kernel           block means of K (one HBM pass, float32 sums), stored in a
//                         two-term half-precision form in the map's operand order
//   map_select_kernel     per workgroup 16 query blocks: their means pooled from Q, the
//                         reduced map S = Qp Kp^T * scale on the fp16 MFMA (three
//                         products of the split terms, float32 accumulation) into the
//                         waves' registers, row softmax, then per row (select_row_regs)
//                         the CDF cutoff found by bisection on float32 bit patterns (or
//                         SIP sampling), the STA OR, and compaction into an ascending list
//   pair_schedule_kernel  the attention's start order: pairs of blocks of neighbouring
//                         frames, each head's pairs by decreasing combined count
// With IBCS block scores the rows of the map are the 8 cluster centroids of each query
// group (ibcs.hip) instead of its mean: ibcs_score_kernel (float32 MFMA on float32 means)
// writes each group's score row, the weighted sum of its centroids' softmax rows, and
// select_kernel applies select_row (the same cut on an LDS row) to those rows; the cut
// and the lists are the same.
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

// Sum of one N-token block in one wave: lane l reads 16-byte chunk c = l % CHUNKS of
// tokens g = l / CHUNKS, g + G, ... (`row(r)` gives the head row of the block's r-th
// token), sums them in token order, and a fixed butterfly adds the G partial sums.  The
// lanes with l < CHUNKS end with the block's sums of elements c*EPC .. c*EPC + EPC - 1.
// BATCH loads are in flight at a time (all of them, ITERS, in the HBM-bound pool kernel;
// fewer where registers are scarce); the sums run in token order either way.
template <typename T, int D, int N, int BATCH, typename RowOf>
__device__ inline void block_sum_wave(const T* __restrict__ head, RowOf row, int lane, float (&acc)[Elem<T>::kPerChunk]) {
    constexpr int EPC = Elem<T>::kPerChunk;
    constexpr int CHUNKS = D / EPC;          // 16-byte chunks per token
    constexpr int G = 64 / CHUNKS;           // tokens per load instruction
    constexpr int ITERS = N / G;
    constexpr int NB = BATCH < ITERS ? BATCH : ITERS;
    static_assert(ITERS % NB == 0, "whole batches");
    const int c = lane % CHUNKS;
    const int g = lane / CHUNKS;
#pragma unroll
    for (int e = 0; e < EPC; ++e) acc[e] = 0.f;
#pragma unroll
    for (int r0 = 0; r0 < ITERS; r0 += NB) {
        u32x4 raw[NB];
#pragma unroll
        for (int r = 0; r < NB; ++r)
            raw[r] = __builtin_nontemporal_load(
                reinterpret_cast<const u32x4*>(head + (size_t)row((r0 + r) * G + g) * D) + c);
#pragma unroll
        for (int r = 0; r < NB; ++r) {
            float v[EPC];
            Elem<T>::unpack(raw[r], v);
#pragma unroll
            for (int e = 0; e < EPC; ++e) acc[e] += v[e];
        }
    }
#pragma unroll
    for (int off = CHUNKS; off < 64; off <<= 1) {
#pragma unroll
        for (int e = 0; e < EPC; ++e) acc[e] += __shfl_xor(acc[e], off);
    }
}

// The head row of token r of block b: fractal order, runs of N rows; raster order, one
// 8 x 8 patch (attn::block_row / row_in_block).
template <bool RASTER, int N>
struct BlockRows {
    uint32_t base;
    attn::RasterGrid grid;
    __device__ BlockRows(const attn::RasterGrid& g, uint32_t b)
        : base(RASTER ? attn::block_row<true>(g, b) : b * N), grid(g) {}
    __device__ uint32_t operator()(int r) const { return base + attn::row_in_block<RASTER>(grid, r); }
};

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

// ---------------------------------------------------------------------------
// Two-term half-precision form of a pooled row, for the map on the fp16 MFMA (the split
// of Ootomo & Yokota, "Recovering single precision accuracy from Tensor Cores while
// surpassing the FP32 theoretical peak performance", IJHPCA 2022, with the low term
// scaled by 2^11).  The row is scaled by 2^-e, e = floor(log2 of its largest magnitude),
// which is exact and brings every element into the half range; then x = hi + lo 2^-11
// with hi = fp16(x) and lo = fp16((x - hi) 2^11), the subtraction and the scaling being
// exact.  That keeps x to about 2^-22 of itself (2^-35 of the row's largest element where
// x is tiny).  A dot product of two split rows is hi.hi + (hi.lo + lo.hi) 2^-11 with the
// lo.lo term dropped: three fp16 products accumulated in float32, as close to the float64
// value as one float32 product pass.
// ---------------------------------------------------------------------------
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));

// e for a row whose elements c * EPC .. c * EPC + EPC - 1 every lane holds (for some c):
// the exponent of the largest magnitude, -126 for a zero or subnormal row
template <int EPC>
__device__ inline int split_exponent(const float (&m)[EPC]) {
    uint32_t mx = 0;
#pragma unroll
    for (int i = 0; i < EPC; ++i) mx = max(mx, __float_as_uint(m[i]) & 0x7fffffffu);
    mx = wave_max_u(mx);
    return max((int)(mx >> 23), 1) - 127;
}

// hi and lo halves of m * 2^-e, EPC consecutive elements each
template <int EPC>
__device__ inline void split_store(const float (&m)[EPC], int e, _Float16* __restrict__ hi, _Float16* __restrict__ lo) {
    static_assert(EPC == 4 || EPC == 8, "one 8- or 16-byte store per term");
    _Float16 h[EPC], l[EPC];
#pragma unroll
    for (int i = 0; i < EPC; ++i) {
        const float x = ldexpf(m[i], -e);
        h[i] = (_Float16)x;
        l[i] = (_Float16)((x - (float)h[i]) * 2048.0f);
    }
    if constexpr (EPC == 8) {
        *reinterpret_cast<f16x8*>(hi) = f16x8{h[0], h[1], h[2], h[3], h[4], h[5], h[6], h[7]};
        *reinterpret_cast<f16x8*>(lo) = f16x8{l[0], l[1], l[2], l[3], l[4], l[5], l[6], l[7]};
    } else {
        *reinterpret_cast<f16x4*>(hi) = f16x4{h[0], h[1], h[2], h[3]};
        *reinterpret_cast<f16x4*>(lo) = f16x4{l[0], l[1], l[2], l[3]};
    }
}

// Layout of the split Kp in the workspace, in the order the map's MFMA operands are read:
// per head, tiles of 16 blocks (the last one padded; its extra columns are never read
// back); inside a tile, for each step s of 32 coordinates and each term (hi, lo), the
// 16-byte pieces of the 64 lanes: lane l = 16 g + (j % 16) holds coordinates
// 32 s + 8 g .. + 7 of block j.  One load instruction of a wave then reads 1 KiB of
// consecutive memory.  kKpTileHalves halves per tile.
template <int D>
constexpr int kKpTileHalves = 16 * D * 2;

template <int D>
__device__ inline size_t kp_piece(int bh, int ntiles, int j, int e, int term) {
    const int st = e >> 5, g = (e >> 3) & 3;
    return ((size_t)bh * ntiles + (j >> 4)) * kKpTileHalves<D> + (size_t)((st * 2 + term) * 64 + 16 * g + (j & 15)) * 8 +
           (e & 7);
}

// The float32 means for the IBCS scores in the same spirit, for the float32 MFMA's
// operand order (map_rows): per head, tiles of 16 blocks; inside a tile, for each group m
// of 16 coordinates, the 16-byte pieces of the 64 lanes (lane 16g + (j mod 16) holds
// coordinates 16m + 4g .. + 3 of block j).  kKpF32TileFloats floats per tile.
template <int D>
constexpr int kKpF32TileFloats = 16 * D;

template <int D>
__device__ inline size_t kpf_piece(int bh, int ntiles, int j, int e) {
    return ((size_t)bh * ntiles + (j >> 4)) * kKpF32TileFloats<D> +
           (size_t)((e >> 4) * 64 + 16 * ((e >> 2) & 3) + (j & 15)) * 4 + (e & 3);
}

// Mean of query block b of one head (one wave), with pool_kernel's arithmetic, in the
// two-term half form (split_store) into the LDS rows hi, lo, its exponent in *e_out.
template <typename T, int D, int BATCH>
__device__ inline void pool_row_split(const T* __restrict__ head, const attn::RasterGrid& grid, bool raster,
                                      uint32_t b, int lane, _Float16* hi, _Float16* lo, int* e_out) {
    constexpr int EPC = Elem<T>::kPerChunk;
    constexpr int CHUNKS = D / EPC;
    float acc[EPC];
    if (raster) block_sum_wave<T, D, 64, BATCH>(head, BlockRows<true, 64>(grid, b), lane, acc);
    else block_sum_wave<T, D, 64, BATCH>(head, BlockRows<false, 64>(grid, b), lane, acc);
    constexpr float inv = 1.0f / 64;
#pragma unroll
    for (int e = 0; e < EPC; ++e) acc[e] *= inv;
    const int ex = split_exponent(acc);
    if (lane < CHUNKS) split_store(acc, ex, hi + lane * EPC, lo + lane * EPC);
    if (lane == 0) *e_out = ex;
}

// Block means of K: one wave per (head, block).  SPLIT = false: float32 means in the
// tiled layout of kpf_piece (the IBCS scores read them).  SPLIT = true: the two-term half
// form in the tiled layout of kp_piece, with the block's exponent in kexp[block] (NABLA's
// map).  (The query blocks are pooled where they are used: in the map kernel for NABLA,
// by the clustering for IBCS.)
template <typename T, int D, int N, bool RASTER, bool SPLIT>
__global__ __launch_bounds__(256) void pool_kernel(const T* __restrict__ k, float* __restrict__ kp,
                                                    int32_t* __restrict__ kexp, int total_blocks, int nb, int L,
                                                    attn::RasterGrid grid) {
    constexpr int EPC = Elem<T>::kPerChunk;
    constexpr int CHUNKS = D / EPC;
    const int blk = (blockIdx.x * 256 + threadIdx.x) >> 6;
    const int lane = threadIdx.x & 63;
    if (blk >= total_blocks) return;
    const int bh = blk / nb;
    const int j = blk - bh * nb, ntiles = (nb + 15) >> 4;
    float acc[EPC];
    block_sum_wave<T, D, N, 64>(k + (size_t)bh * L * D, BlockRows<RASTER, N>(grid, j), lane, acc);
    constexpr float inv = 1.0f / N;      // N is a power of two: exact
#pragma unroll
    for (int e = 0; e < EPC; ++e) acc[e] *= inv;
    if constexpr (SPLIT) {
        const int ex = split_exponent(acc);
        _Float16* base = reinterpret_cast<_Float16*>(kp);
        if (lane < CHUNKS)
            split_store(acc, ex, base + kp_piece<D>(bh, ntiles, j, lane * EPC, 0),
                        base + kp_piece<D>(bh, ntiles, j, lane * EPC, 1));
        if (lane == 0) kexp[blk] = ex;
    } else if (lane < CHUNKS) {
#pragma unroll
        for (int e = 0; e < EPC; e += 4)
            *reinterpret_cast<f32x4*>(kp + kpf_piece<D>(bh, ntiles, j, lane * EPC + e)) =
                f32x4{acc[e], acc[e + 1], acc[e + 2], acc[e + 3]};
    }
}

// ---------------------------------------------------------------------------
// Reduced map, then the cut.
// The map kernels hold kRows = 16 rows of S per workgroup (the M of the 16 x 16 MFMA).
// The cut (select_row on an LDS row, select_row_regs on a row in registers) takes one row
//   in one wave.  Keeping block j iff F_j > thr is the
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
        // the tile's operand pieces, one 1 KiB read per 16 coordinates (the padding columns
        // past nb are read but never stored)
        const float* src = kh + (size_t)ct * kKpF32TileFloats<D> + lane * 4;
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
        // the K operand in two halves of d (16 values per lane each)
#pragma unroll 1
        for (int h = 0; h < 2; ++h) {
            f32x4 b[KC / 8];
#pragma unroll
            for (int v = 0; v < KC / 8; ++v) b[v] = *reinterpret_cast<const f32x4*>(src + (h * (KC / 8) + v) * 256);
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
    map_rows<D, kScoreWaves>(x_lds, kp + (size_t)bh * ((nb + 15) >> 4) * kKpF32TileFloats<D>, nb, ld_s, scale,
                             s_lds, wave, lane);
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
// SIP on one row held in registers (v[i] = A_j of block j = lane + 64 i, probabilities):
// the same rule and order of arithmetic as sip_row.
// ---------------------------------------------------------------------------
template <int NREG>
__device__ void sip_row_regs(const float (&v)[NREG], int nb, int budget, const float* u, int32_t* out_idx,
                             float* out_logw, uint32_t* out_bits, int nwords, int32_t* out_count, int lane) {
    float best = -1.f;
    int bj = nb;
#pragma unroll
    for (int i = 0; i < NREG; ++i) {
        const int j = lane + 64 * i;
        if (j < nb && v[i] > best) {
            best = v[i];
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
#pragma unroll
        for (int i = 0; i < NREG; ++i) {
            const int j = lane + 64 * i;
            if (j < nb && j != top) rest += v[i];
        }
        rest = wave_sum(rest);
        c = rest > 0.f ? (float)kp / rest : 0.f;
        c_cert = c;
        int m = 0;
        for (int it = 0; it < 64; ++it) {
            float unc = 0.f;   // mass of the blocks still below 1
            int cnt = 0;
#pragma unroll
            for (int i = 0; i < NREG; ++i) {
                const int j = lane + 64 * i;
                const bool other = j < nb && j != top;
                const bool cert = other && c * v[i] >= 1.f;
                if (other && !cert) unc += v[i];
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
#pragma unroll
    for (int i = 0; i < NREG; ++i) {
        const int j = lane + 64 * i;
        bool keep = false;
        float pi = 0.f;
        if (j < nb) {
            pi = (all || j == top || c_cert * v[i] >= 1.f) ? 1.f : c * v[i];
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
            const int w = 2 * i;
            if (lane == 0 && w < nwords) out_bits[w] = (uint32_t)ballot;
            if (lane == 1 && w + 1 < nwords) out_bits[w + 1] = (uint32_t)(ballot >> 32);
        }
    }
    if (lane == 0) *out_count = base;
}

// ---------------------------------------------------------------------------
// The CDF cut of one row held in registers, in one wave: v[i] = A_j of block
// j = lane + 64 i (probabilities summing to one; entries past nb must be +0, which no
// bracket (lo, hi] holds and no sum notices).  The same cut as select_row: bisection over
// bit patterns from u0 = thr / nb.  The first steps pass over the whole row in
// registers; once at most kCap values are left in the bracket they are compacted, in
// block order, through the wave's LDS buffer `cand` into four registers per lane, where
// the steps continue until at most kFinish remain; those take the exact finish, one per
// lane.  Then the STA OR (tile coordinates by multiply-high division), the ascending
// list, the count and the bitmap.
// ---------------------------------------------------------------------------
constexpr int kFinish = 16;

// Writes the values of v (NV registers per lane, lane-major) whose bit pattern lies in
// (lo, hi] to cand in order and returns their number.
template <int NV>
__device__ inline int compact_regs(const float (&v)[NV], uint32_t lo, uint32_t hi, float* cand, int lane) {
    int len = 0;
#pragma unroll
    for (int i = 0; i < NV; ++i) {
        const uint32_t b = __float_as_uint(v[i]);
        const bool in = b > lo && b <= hi;
        const uint64_t ballot = __ballot(in);
        if (in) cand[len + __popcll(ballot & ((1ull << lane) - 1ull))] = v[i];
        len += __popcll(ballot);
    }
    return len;
}

// One bisection step over the compacted candidates (the values in (lo, hi]): narrows
// the bracket to the half that holds the cut, keeping g_lo (mass of the row's values
// <= lo) and n_in (values in the bracket).
template <int NV>
__device__ inline void bisect_step(const float (&v)[NV], uint32_t& lo, uint32_t& hi, float& g_lo, int& n_in,
                                   float thr) {
    const uint32_t mid = lo + ((hi - lo) >> 1);
    float s_ = 0.f;
    int c = 0;
#pragma unroll
    for (int i = 0; i < NV; ++i) {
        const uint32_t b = __float_as_uint(v[i]);
        const bool in = b > lo && b <= mid;
        if (in) s_ += v[i];
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
}

// The same step over the whole row: g(mid) is summed afresh over every value <= mid (one
// compare, one select and one add per value, no lower bound to test), and the counts of
// values <= lo and <= hi give the bracket's population.
template <int NV>
__device__ inline void bisect_step_row(const float (&v)[NV], uint32_t& lo, uint32_t& hi, float& g_lo, int& c_lo,
                                       int& c_hi, float thr) {
    const uint32_t mid = lo + ((hi - lo) >> 1);
    float s_ = 0.f;
    int c = 0;
#pragma unroll
    for (int i = 0; i < NV; ++i) {
        const bool le = __float_as_uint(v[i]) <= mid;
        s_ += le ? v[i] : 0.f;
        c += __popcll(__ballot(le));
    }
    s_ = wave_sum(s_);
    if (s_ > thr) {
        hi = mid;
        c_hi = c;
    } else {
        lo = mid;
        g_lo = s_;
        c_lo = c;
    }
}

template <int NREG>
__device__ void select_row_regs(const float (&v)[NREG], float* cand, int nb, int bh, int row, float thr, int sta,
                                FastDiv fd_pf, FastDiv fd_nw, int rt, int rh, int rw,
                                int32_t* __restrict__ kv_count, int32_t* __restrict__ kv_index,
                                uint32_t* __restrict__ bitmap, int lane) {
    const int nwords = (nb + 31) >> 5;
    // start of the bracket: u0 = thr / nb, nudged down so rounding cannot push g(u0)
    // above thr; verified below and dropped to 0 if it fails
    uint32_t lo = __float_as_uint(thr / ((float)nb * 1.0001f));
    float g_lo = 0.f;
    int n_in = 0;
    uint32_t maxb = 0;
#pragma unroll
    for (int i = 0; i < NREG; ++i) {
        const uint32_t b = __float_as_uint(v[i]);
        maxb = max(maxb, b);
        const bool in = b > lo;
        if (!in) g_lo += v[i];
        n_in += __popcll(__ballot(in));
    }
    g_lo = wave_sum(g_lo);
    maxb = wave_max_u(maxb);
    if (g_lo > thr) {   // cannot happen in exact arithmetic; fall back to g(0) = 0
        lo = 0;
        g_lo = 0.f;
        n_in = 0;
#pragma unroll
        for (int i = 0; i < NREG; ++i) n_in += __popcll(__ballot(__float_as_uint(v[i]) > 0u));
    }
    uint32_t hi = maxb;
    // bracket (lo, hi]: g(lo) = g_lo <= thr and, unless the whole row sums to at most
    // thr, g(hi) > thr; n_in values lie inside it (always >= 1: the maximum)
    {
        int c_lo = NREG * 64 - n_in, c_hi = NREG * 64;   // values <= lo, <= hi (padding included)
        while (hi - lo > 1 && c_hi - c_lo > kCap) bisect_step_row(v, lo, hi, g_lo, c_lo, c_hi, thr);
        n_in = c_hi - c_lo;
    }
    uint32_t cut = hi;
    if (n_in <= kCap) {
        float c4[kCap / 64];
        const int len = compact_regs(v, lo, hi, cand, lane);
#pragma unroll
        for (int k = 0; k < kCap / 64; ++k) c4[k] = lane + 64 * k < len ? cand[lane + 64 * k] : 0.f;
        while (hi - lo > 1 && n_in > kFinish) bisect_step(c4, lo, hi, g_lo, n_in, thr);
        if (n_in <= kFinish) {
            // one candidate per lane: F(x) = g_lo + (sum of the candidates <= x), tied
            // values together; the cut is the smallest candidate with F(x) > thr
            const int m_len = compact_regs(c4, lo, hi, cand, lane);
            const float x = lane < m_len ? cand[lane] : 0.f;
            const uint32_t bx = __float_as_uint(x);
            float below = 0.f;
            for (int m = 0; m < m_len; ++m) {
                const float y = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), m));
                if (__float_as_uint(y) <= bx) below += y;
            }
            const bool crosses = lane < m_len && g_lo + below > thr;
            const uint32_t pick = crosses ? bx : 0xffffffffu;
            const uint32_t best = ~wave_max_u(~pick);   // smallest pattern among the crossing ones
            if (best != 0xffffffffu) cut = best;
        }
    }

    int qt = 0, qh_ = 0, qw = 0;
    int jlo = 0, jhi = 0;   // the blocks of the frames the window reaches
    if (sta) {
        uint32_t t_, rem_, h_, w_;
        fd_pf.divmod((uint32_t)row, t_, rem_);
        fd_nw.divmod(rem_, h_, w_);
        qt = (int)t_;
        qh_ = (int)h_;
        qw = (int)w_;
        jlo = max(qt - rt, 0) * (int)fd_pf.d;
        jhi = (qt + rt + 1) * (int)fd_pf.d;
    }
    int32_t* out_idx = kv_index + ((size_t)bh * nb + row) * nb;
    uint32_t* out_bits = bitmap ? bitmap + ((size_t)bh * nb + row) * nwords : nullptr;
    int base = 0;
#pragma unroll
    for (int i = 0; i < NREG; ++i) {
        const int j = lane + 64 * i;
        bool keep = j < nb && __float_as_uint(v[i]) >= cut;
        // the window test only where this register's 64 blocks meet the window's frames
        // (a uniform branch)
        if (sta && 64 * i < jhi && 64 * i + 64 > jlo) {
            if (!keep && j < nb && j >= jlo && j < jhi) {
                uint32_t kt, rem, kh_, kw;
                fd_pf.divmod((uint32_t)j, kt, rem);
                fd_nw.divmod(rem, kh_, kw);
                keep = abs((int)kt - qt) <= rt && abs((int)kh_ - qh_) <= rh && abs((int)kw - qw) <= rw;
            }
        }
        const uint64_t ballot = __ballot(keep);
        if (keep) out_idx[base + __popcll(ballot & ((1ull << lane) - 1ull))] = j;
        base += __popcll(ballot);
        if (out_bits) {
            const int w = 2 * i;
            if (lane == 0 && w < nwords) out_bits[w] = (uint32_t)ballot;
            if (lane == 1 && w + 1 < nwords) out_bits[w + 1] = (uint32_t)(ballot >> 32);
        }
    }
    if (lane == 0) kv_count[(size_t)bh * nb + row] = base;
}

// ---------------------------------------------------------------------------
// NABLA's reduced map and cut in one kernel.  A workgroup owns kRows = 16 query blocks of
// one head (16 waves, one row each; for rows of 24 and 32 registers 8 waves, two rows
// each).  A wave pools its blocks from Q (block_sum_wave, as pool_kernel does for K) and
// owns their rows of the map: a row ends up in the wave's registers (v[i] = S_j of block
// j = lane + 64 i), so the softmax and the cut run without touching LDS.  The map runs in
// chunks of 256 columns: each wave computes its 16 x 16 tile(s) of the chunk on the fp16
// MFMA (map_tile / tile_products) into an LDS chunk buffer, and after one barrier every
// wave copies its rows' 256 values into registers.  Two chunk buffers alternate, so one
// barrier per chunk suffices (a wave writes chunk c + 2 only after the barrier of chunk
// c + 1, which every wave reaches after reading chunk c).  LDS per workgroup is 58 KiB
// whatever nb, and two workgroups share a CU: one's loads and barriers overlap the
// other's cut.
// ---------------------------------------------------------------------------
constexpr int kWaves = 16;
constexpr int kChunkCols = 16 * kWaves;     // one 16-column tile per wave
constexpr int kChunkLd = kChunkCols + 4;    // padded row: the 16 x 16 tile stores hit distinct banks
constexpr int kRowCand = kCap;              // a wave's compacted candidates

// LDS row of a split pooled query: D halves and a 16-byte pad, so the 16-byte reads of
// 8 consecutive lanes (8 rows) fall on distinct banks
template <int D>
constexpr int kQld = D + 8;

// One 16 x 16 tile of S = scale * Qp Kp^T: rows row0 .. row0 + 15 of the workgroup (split
// halves q_hi, q_lo in LDS, exponents eq), columns j0 .. j0 + 15 (j0 a multiple of 16,
// below nb) of the head's split Kp (tiled layout of kp_piece, exponents kexp; columns
// past nb hold padding, and their S values are never read).  Three
// v_mfma_f32_16x16x32_f16 per 32 coordinates: hi.hi into one accumulator, hi.lo and lo.hi
// into another, combined as hh + x 2^-11 and scaled back by 2^(eq + ek).  Lane (row/col
// l % 16, group g = l / 16) supplies coordinates 32 s + 8 g .. + 7 at step s in both
// operands (one 16-byte load per term, 1 KiB per wave).  The Kp operand comes in two
// rounds of half the steps (16 VGPRs at d = 128), leaving the registers to the wave's row.
template <int D>
__device__ inline f32x4 map_tile(const _Float16* __restrict__ q_hi, const _Float16* __restrict__ q_lo,
                                 const int* __restrict__ eq, const _Float16* __restrict__ kh,
                                 const int32_t* __restrict__ kexp, int nb, int j0, float scale, int lane) {
    constexpr int KS = D / 32;           // MFMA steps
    constexpr int H = KS / 2;            // steps per load round
    const int li = lane & 15;
    const int kq = lane >> 4;
    const int j = j0 + li;
    const _Float16* src = kh + (size_t)(j0 >> 4) * kKpTileHalves<D> + lane * 8;
    const _Float16* qa = q_hi + li * kQld<D> + 8 * kq;
    const _Float16* qb = q_lo + li * kQld<D> + 8 * kq;
    f32x4 hh = {0.f, 0.f, 0.f, 0.f};
    f32x4 x = {0.f, 0.f, 0.f, 0.f};
#pragma unroll 1
    for (int h = 0; h < 2; ++h) {
        f16x8 bh[H], bl[H];
#pragma unroll
        for (int m = 0; m < H; ++m) {
            const int st = h * H + m;
            bh[m] = *reinterpret_cast<const f16x8*>(src + (st * 2) * 512);
            bl[m] = *reinterpret_cast<const f16x8*>(src + (st * 2 + 1) * 512);
        }
#pragma unroll
        for (int m = 0; m < H; ++m) {
            const int st = h * H + m;
            const f16x8 ah = *reinterpret_cast<const f16x8*>(qa + 32 * st);
            const f16x8 al = *reinterpret_cast<const f16x8*>(qb + 32 * st);
            hh = __builtin_amdgcn_mfma_f32_16x16x32_f16(ah, bh[m], hh, 0, 0, 0);
            x = __builtin_amdgcn_mfma_f32_16x16x32_f16(ah, bl[m], x, 0, 0, 0);
            x = __builtin_amdgcn_mfma_f32_16x16x32_f16(al, bh[m], x, 0, 0, 0);
        }
    }
    const int ek = kexp[min(j, nb - 1)];
    f32x4 out;
#pragma unroll
    for (int r = 0; r < 4; ++r) out[r] = ldexpf(fmaf(x[r], 1.0f / 2048.0f, hh[r]) * scale, eq[4 * kq + r] + ek);
    return out;
}

// The Kp operand of one tile, whole: columns j0 + l % 16, coordinates 32 s + 8 (l / 16)
// .. + 7 of both terms for every step s (eight 1 KiB reads of the tiled layout), and the
// column's exponent.  Columns past nb hold padding: their S values are never read (the
// rows take -inf there), and not zeroing the loaded registers keeps the loads in flight
// until they are used.
template <int D>
struct KpTile {
    f16x8 hi[D / 32], lo[D / 32];
    int ek;
};

template <int D>
__device__ inline void load_kp_tile(const _Float16* __restrict__ kh, const int32_t* __restrict__ kexp, int nb,
                                    int j0, int lane, KpTile<D>& t) {
    // j0 is a multiple of 16; past the last tile the last one is read again
    const int tile = min(j0, nb - 1) >> 4;
    const _Float16* src = kh + (size_t)tile * kKpTileHalves<D> + lane * 8;
#pragma unroll
    for (int st = 0; st < D / 32; ++st) {
        t.hi[st] = *reinterpret_cast<const f16x8*>(src + (st * 2) * 512);
        t.lo[st] = *reinterpret_cast<const f16x8*>(src + (st * 2 + 1) * 512);
    }
    t.ek = kexp[min(j0 + (lane & 15), nb - 1)];
}

// hi.hi + (hi.lo + lo.hi) 2^-11 for the workgroup's 16 split query rows against a
// loaded Kp tile, scaled to S (see map_tile)
template <int D>
__device__ inline f32x4 tile_products(const _Float16* __restrict__ q_hi, const _Float16* __restrict__ q_lo,
                                      const int* __restrict__ eq, const KpTile<D>& t, float scale, int lane) {
    const int li = lane & 15;
    const int kq = lane >> 4;
    const _Float16* qa = q_hi + li * kQld<D> + 8 * kq;
    const _Float16* qb = q_lo + li * kQld<D> + 8 * kq;
    f32x4 hh = {0.f, 0.f, 0.f, 0.f};
    f32x4 x = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int st = 0; st < D / 32; ++st) {
        const f16x8 ah = *reinterpret_cast<const f16x8*>(qa + 32 * st);
        const f16x8 al = *reinterpret_cast<const f16x8*>(qb + 32 * st);
        hh = __builtin_amdgcn_mfma_f32_16x16x32_f16(ah, t.hi[st], hh, 0, 0, 0);
        x = __builtin_amdgcn_mfma_f32_16x16x32_f16(ah, t.lo[st], x, 0, 0, 0);
        x = __builtin_amdgcn_mfma_f32_16x16x32_f16(al, t.hi[st], x, 0, 0, 0);
    }
    f32x4 out;
#pragma unroll
    for (int r = 0; r < 4; ++r) out[r] = ldexpf(fmaf(x[r], 1.0f / 2048.0f, hh[r]) * scale, eq[4 * kq + r] + t.ek);
    return out;
}

// Rows of up to 20 register blocks (1280 KV blocks) run eight waves per SIMD (two
// workgroups per CU) within 64 VGPRs; longer rows four waves per SIMD with 128, and so
// does the SIP form from rows of 12 registers on (it keeps more values live across its
// water-level loop).
template <int NREG, bool SIP>
constexpr int kMapSelectWaves = (NREG > 20 || (SIP && NREG >= 12)) ? 4 : 8;
// Where the registers allow (four waves per SIMD, rows of at most 32 registers), a wave
// loads the next chunk's Kp tile whole while the current chunk is exchanged and read, so
// the load's latency is hidden behind the barrier; otherwise the tile comes in two rounds
// per chunk (map_tile).  There the query block's mean also keeps all sixteen loads in
// flight instead of two.  Rows of 48 and 64 registers (up to 4096 blocks) fit in 128
// VGPRs only without both.
template <int NREG, bool SIP>
constexpr bool kMapPrefetch = kMapSelectWaves<NREG, SIP> == 4 && NREG <= 32 && !(!SIP && NREG > 20);
template <int NREG, bool SIP>
constexpr int kPoolBatch = kMapSelectWaves<NREG, SIP> == 4 && NREG <= 32 ? 16 : 2;
// Rows of 24 and 32 registers (NABLA's cut, not SIP) take two rows per wave in eight-wave
// workgroups, so two workgroups share a CU at four waves per SIMD: one's pooling and map
// overlap the other's cut, where one sixteen-wave workgroup per CU would leave the
// SIMDs idle through its own pooling.
template <int NREG, bool SIP>
constexpr int kRowsPerWave = (!SIP && NREG > 20 && NREG <= 32) ? 2 : 1;
template <int NREG, bool SIP>
constexpr int kMapThreads = 64 * kRows / kRowsPerWave<NREG, SIP>;

// The softmax of one row held in registers and its cut (or SIP sampling).
template <int NREG, bool SIP>
__device__ __attribute__((always_inline)) inline void cut_row(float (&v)[NREG], float* cand, int nb, int bh, int row, float thr,
                               int sta, FastDiv fd_pf, FastDiv fd_nw, int rt, int rh, int rw,
                               int32_t* __restrict__ kv_count, int32_t* __restrict__ kv_index,
                               uint32_t* __restrict__ bitmap, int sip_budget, const float* __restrict__ uniforms,
                               float* __restrict__ kv_logw, int lane) {
    // softmax in place: A = exp2((S - max) log2 e) / sum, the sum in block order per lane
    float mx = -INFINITY;
#pragma unroll
    for (int i = 0; i < NREG; ++i) mx = fmaxf(mx, v[i]);
    const float mx2 = wave_max(mx) * kLog2e;
    float sum = 0.f;
#pragma unroll
    for (int i = 0; i < NREG; ++i) {
        const float e = __builtin_amdgcn_exp2f(fmaf(v[i], kLog2e, -mx2));   // -inf past nb: +0
        v[i] = e;
        sum += e;
    }
    const float inv_sum = 1.0f / wave_sum(sum);
#pragma unroll
    for (int i = 0; i < NREG; ++i) v[i] *= inv_sum;
    if constexpr (SIP) {
        const int nwords = (nb + 31) >> 5;
        sip_row_regs<NREG>(v, nb, sip_budget, uniforms + ((size_t)bh * nb + row) * nb,
                           kv_index + ((size_t)bh * nb + row) * nb, kv_logw + ((size_t)bh * nb + row) * nb,
                           bitmap ? bitmap + ((size_t)bh * nb + row) * nwords : nullptr, nwords,
                           kv_count + (size_t)bh * nb + row, lane);
    } else {
        select_row_regs<NREG>(v, cand, nb, bh, row, thr, sta, fd_pf, fd_nw, rt, rh, rw, kv_count, kv_index, bitmap,
                              lane);
    }
}

template <int D, int NREG, bool SIP>
__global__ __launch_bounds__((kMapThreads<NREG, SIP>)) __attribute__((amdgpu_waves_per_eu(kMapSelectWaves<NREG, SIP>,
                                                                                       kMapSelectWaves<NREG, SIP>))) void
map_select_kernel(const void* __restrict__ q, int bf16, int raster, attn::RasterGrid grid, int L,
                  const _Float16* __restrict__ kp, const int32_t* __restrict__ kexp, int nb, float scale,
                  float thr, int sta,
                  FastDiv fd_pf, FastDiv fd_nw, int rt, int rh, int rw, int32_t* __restrict__ kv_count,
                  int32_t* __restrict__ kv_index, uint32_t* __restrict__ bitmap, int sip_budget,
                  const float* __restrict__ uniforms, float* __restrict__ kv_logw) {
    constexpr int RPW = kRowsPerWave<NREG, SIP>;   // rows (and map tiles per chunk) per wave
    // [2][kRows][kChunkLd] chunk buffers, [waves][kRowCand] candidates, then the split
    // pooled queries: [kRows][kQld] hi halves, [kRows][kQld] lo halves, [kRows] exponents
    extern __shared__ __align__(16) float s_lds[];
    const int wave = threadIdx.x >> 6;
    const int lane = threadIdx.x & 63;
    // Workgroups are dealt round-robin to the 8 XCDs; XCD x takes the x-th eighth of the
    // (head, row group) items in order, so the workgroups on one XCD's L2 read the pooled
    // K of one or two heads at a time instead of all the heads in flight on the GPU.
    const int groups = (nb + kRows - 1) / kRows;
    const int nwg = gridDim.x;
    const int full = (nwg / 8) * 8;
    const int w = blockIdx.x;
    const int item = w < full ? (w % 8) * (nwg / 8) + w / 8 : w;
    const int bh = item / groups;
    const int row0 = (item - bh * groups) * kRows;
    float* cand = s_lds + 2 * kRows * kChunkLd + wave * kRowCand;
    _Float16* q_hi = reinterpret_cast<_Float16*>(s_lds + 2 * kRows * kChunkLd + kWaves * kRowCand);
    _Float16* q_lo = q_hi + kRows * kQld<D>;
    int* eq = reinterpret_cast<int*>(q_lo + kRows * kQld<D>);
    const _Float16* kh = kp + (size_t)bh * ((nb + 15) >> 4) * kKpTileHalves<D>;
    const int32_t* kexp_h = kexp + (size_t)bh * nb;
    // the first chunk's Kp tile, in flight while the query block is pooled
    constexpr bool kPf = kMapPrefetch<NREG, SIP>;
    KpTile<D> kt;
    if constexpr (kPf) load_kp_tile<D>(kh, kexp_h, nb, 16 * wave, lane, kt);
    // the workgroup's pooled query rows: wave w forms the mean of query block row0 + w
    // from Q itself (zeros past nb), so Q is read once, here, beside other workgroups' work
    if constexpr (RPW == 1) {
        const int row = row0 + wave;
        _Float16* hr = q_hi + wave * kQld<D>;
        _Float16* lr = q_lo + wave * kQld<D>;
        if (row < nb) {
            constexpr int kB = kPoolBatch<NREG, SIP>;
            if (bf16)
                pool_row_split<__bf16, D, kB>((const __bf16*)q + (size_t)bh * L * D, grid, raster, (uint32_t)row,
                                              lane, hr, lr, eq + wave);
            else
                pool_row_split<float, D, kB>((const float*)q + (size_t)bh * L * D, grid, raster, (uint32_t)row,
                                             lane, hr, lr, eq + wave);
        } else {
            for (int e = lane; e < D; e += 64) hr[e] = lr[e] = (_Float16)0.f;
            if (lane == 0) eq[wave] = 0;
        }
    } else {
        // the same for local rows RPW wave + u
#pragma unroll
        for (int u = 0; u < RPW; ++u) {
            const int r = RPW * wave + u;
            const int row = row0 + r;
            _Float16* hr = q_hi + r * kQld<D>;
            _Float16* lr = q_lo + r * kQld<D>;
            if (row < nb) {
                constexpr int kB = kPoolBatch<NREG, SIP>;
                if (bf16)
                    pool_row_split<__bf16, D, kB>((const __bf16*)q + (size_t)bh * L * D, grid, raster,
                                                  (uint32_t)row, lane, hr, lr, eq + r);
                else
                    pool_row_split<float, D, kB>((const float*)q + (size_t)bh * L * D, grid, raster,
                                                 (uint32_t)row, lane, hr, lr, eq + r);
            } else {
                for (int e = lane; e < D; e += 64) hr[e] = lr[e] = (_Float16)0.f;
                if (lane == 0) eq[r] = 0;
            }
        }
    }
    attn::lds_barrier();   // LDS only: prefetched tiles stay in flight

    // the rows in registers: va for local row RPW wave, vb for RPW wave + 1 (two rows per
    // wave only)
    float va[NREG];
    float vb[RPW == 2 ? NREG : 1];
    const int li = lane & 15;
    const int kq = lane >> 4;
#pragma unroll
    for (int c = 0; c < NREG / 4; ++c) {
        if (c * kChunkCols < nb) {              // uniform over the workgroup
            float* buf = s_lds + (c & 1) * kRows * kChunkLd;
#pragma unroll
            for (int u = 0; u < RPW; ++u) {
                const int t = RPW * wave + u;      // the chunk's 16-column tile this wave computes
                const int j0 = c * kChunkCols + 16 * t;
                if (j0 < nb) {
                    f32x4 sv;
                    if constexpr (kPf) {
                        sv = tile_products<D>(q_hi, q_lo, eq, kt, scale, lane);
                        // the next chunk's tile, in flight across this chunk's exchange (past the
                        // last chunk a clamped, unused one: an unconditional load is not copied
                        // between registers, which would wait for it here)
                        load_kp_tile<D>(kh, kexp_h, nb, j0 + kChunkCols, lane, kt);
                    } else {
                        sv = map_tile<D>(q_hi, q_lo, eq, kh, kexp_h, nb, j0, scale, lane);
                    }
#pragma unroll
                    for (int r = 0; r < 4; ++r) buf[(4 * kq + r) * kChunkLd + 16 * t + li] = sv[r];
                }
            }
            attn::lds_barrier();   // LDS only: prefetched tiles stay in flight
#pragma unroll
            for (int m = 0; m < 4; ++m) {
                const int j = c * kChunkCols + lane + 64 * m;
                va[4 * c + m] = j < nb ? buf[(RPW * wave) * kChunkLd + lane + 64 * m] : -INFINITY;
                if constexpr (RPW == 2)
                    vb[4 * c + m] = j < nb ? buf[(RPW * wave + 1) * kChunkLd + lane + 64 * m] : -INFINITY;
            }
        } else {
#pragma unroll
            for (int m = 0; m < 4; ++m) {
                va[4 * c + m] = -INFINITY;
                if constexpr (RPW == 2) vb[4 * c + m] = -INFINITY;
            }
        }
    }
    const int row_a = row0 + RPW * wave;
    if (row_a < nb)
        cut_row<NREG, SIP>(va, cand, nb, bh, row_a, thr, sta, fd_pf, fd_nw, rt, rh, rw, kv_count, kv_index, bitmap,
                           sip_budget, uniforms, kv_logw, lane);
    if constexpr (RPW == 2) {
        if (row_a + 1 < nb)
            cut_row<NREG, SIP>(vb, cand, nb, bh, row_a + 1, thr, sta, fd_pf, fd_nw, rt, rh, rw, kv_count, kv_index,
                               bitmap, sip_budget, uniforms, kv_logw, lane);
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
// the tail of the launch short.  One wave per head (counting sort on nb + 1 bins); the
// blocks' bins are read from the counts once, with the loads batched, and kept in LDS.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(64) void schedule_kernel(const int32_t* __restrict__ kv_count, int nb,
                                                      int32_t* __restrict__ schedule) {
    extern __shared__ int bins[];   // nb + 1 counters, then the nb blocks' bins
    int* keyl = bins + nb + 1;
    const int h = blockIdx.x;
    const int lane = threadIdx.x;
    const int32_t* cnt = kv_count + (size_t)h * nb;
    for (int b = lane; b <= nb; b += 64) bins[b] = 0;
    // eight blocks per lane per round: eight count loads in flight
    for (int i0 = lane; i0 < nb; i0 += 512) {
        int c[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) c[u] = cnt[min(i0 + 64 * u, nb - 1)];
#pragma unroll
        for (int u = 0; u < 8; ++u)
            if (i0 + 64 * u < nb) keyl[i0 + 64 * u] = nb - min(max(c[u], 0), nb);
    }
    __syncthreads();
    for (int i = lane; i < nb; i += 64) atomicAdd(&bins[keyl[i]], 1);
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
        const int pos = atomicAdd(&bins[keyl[i]], 1);
        schedule[(size_t)h * nb + pos] = h * nb + i;
    }
}

// ---------------------------------------------------------------------------
// Start order for the attention launch, which computes two query blocks per workgroup
// (schedule entries 2j and 2j+1) and copies each KV tile the two keep once.  Blocks of
// neighbouring frames at the same patch position keep largely the same KV blocks, so
// block i of frame t is paired with block i of frame t + 1 (t even); with an odd number
// of frames the last frame's blocks pair side by side, and with an odd number of blocks
// per frame as well one block per head is left single.  Inside a head the pairs run by
// decreasing combined kept count (counting sort, one wave per head), heads in order, so
// consecutive workgroups - dealt round-robin to the 8 XCDs - keep the whole GPU on one
// or two heads at a time and each head's short lists run last.  The single blocks of all
// heads go at the very end, so that every head's pairs stay aligned to even positions.
// `fpf` is the number of blocks per frame (1 when frames do not hold whole blocks, which
// pairs blocks 2j and 2j + 1).  The pairs' bins are computed once, with the count loads
// batched, and kept in LDS.
// ---------------------------------------------------------------------------
__device__ inline void pair_members(int j, int fpf, int tpairs, int& a, int& b) {
    if (j < tpairs * fpf) {
        const int t = 2 * (j / fpf), p = j - (j / fpf) * fpf;
        a = t * fpf + p;
        b = a + fpf;
    } else {
        a = 2 * tpairs * fpf + 2 * (j - tpairs * fpf);
        b = a + 1;
    }
}

__global__ __launch_bounds__(64) void pair_schedule_kernel(const int32_t* __restrict__ kv_count, int nb, int fpf,
                                                           int BH, int32_t* __restrict__ schedule) {
    extern __shared__ int bins[];   // 2 nb + 1 counters, then the nb / 2 pairs' bins
    const int h = blockIdx.x;
    const int lane = threadIdx.x;
    const int32_t* cnt = kv_count + (size_t)h * nb;
    const int frames = nb / fpf;
    const int tpairs = frames / 2;                    // frame pairs (t, t + 1), t even
    const int single = (frames & 1) & (fpf & 1);      // a block left without a partner
    const int npairs = (nb - single) / 2;
    const int nbins = 2 * nb + 1;
    int* keyl = bins + nbins;
    for (int b = lane; b < nbins; b += 64) bins[b] = 0;
    // four pairs per lane per round: eight count loads in flight (indices past the pairs
    // clamped to a valid block, their bins unused)
    for (int j0 = lane; j0 < npairs; j0 += 256) {
        int ca[4], cb[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            int a, b;
            pair_members(min(j0 + 64 * u, npairs - 1), fpf, tpairs, a, b);
            ca[u] = cnt[a];
            cb[u] = cnt[b];
        }
#pragma unroll
        for (int u = 0; u < 4; ++u)
            if (j0 + 64 * u < npairs) keyl[j0 + 64 * u] = 2 * nb - (min(max(ca[u], 0), nb) + min(max(cb[u], 0), nb));
    }
    __syncthreads();
    for (int j = lane; j < npairs; j += 64) atomicAdd(&bins[keyl[j]], 1);
    __syncthreads();
    // exclusive prefix sum over the bins: one contiguous chunk per lane
    const int per = (nbins + 63) / 64;
    const int b0 = lane * per, b1 = min(b0 + per, nbins);
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
    int32_t* out = schedule + (size_t)h * (nb - single);
    for (int j = lane; j < npairs; j += 64) {
        int a, b;
        pair_members(j, fpf, tpairs, a, b);
        const int pos = atomicAdd(&bins[keyl[j]], 1);
        out[2 * pos] = h * nb + a;
        out[2 * pos + 1] = h * nb + b;
    }
    if (single && lane == 0) schedule[(size_t)BH * (nb - 1) + h] = h * nb + nb - 1;
}

template <typename T, int D, bool RASTER, bool SPLIT>
void launch_pool_form(const MaskArgs& a, const attn::RasterGrid& grid, hipStream_t s) {
    const int total = a.BH * a.nb;
    hipLaunchKernelGGL((pool_kernel<T, D, 64, RASTER, SPLIT>), dim3((total + 3) / 4), dim3(256), 0, s, (const T*)a.k,
                       a.kp, a.kexp, total, a.nb, a.nb * 64, grid);
}

template <typename T, int D>
hipError_t launch_pool(const MaskArgs& a, hipStream_t s) {
    attn::RasterGrid grid{};
    if (a.raster) {
        grid.W = (uint32_t)a.W;
        grid.HW = (uint32_t)(a.H * a.W);
        grid.nHW = FastDiv((uint32_t)(a.nH * a.nW));
        grid.nW = FastDiv((uint32_t)a.nW);
    }
    // the IBCS scores read float32 means, NABLA's map the half form
    if (a.raster) {
        if (a.ibcs) launch_pool_form<T, D, true, false>(a, grid, s);
        else launch_pool_form<T, D, true, true>(a, grid, s);
    } else {
        if (a.ibcs) launch_pool_form<T, D, false, false>(a, grid, s);
        else launch_pool_form<T, D, false, true>(a, grid, s);
    }
    return hipGetLastError();
}

template <int D>
constexpr size_t map_select_lds_bytes() {
    return ((size_t)2 * kRows * kChunkLd + (size_t)kWaves * kRowCand) * sizeof(float) +
           (size_t)2 * kRows * kQld<D> * sizeof(_Float16) + (size_t)kRows * sizeof(int);
}
static_assert(map_select_lds_bytes<128>() <= 64 * 1024, "map/select LDS within the default dynamic limit");

template <int D, int NREG>
hipError_t launch_map_select(const MaskArgs& a, hipStream_t s) {
    const size_t lds = map_select_lds_bytes<D>();
    dim3 grid(((a.nb + kRows - 1) / kRows) * a.BH);   // (head, row group) items, see the kernel
    const FastDiv fd_pf((uint32_t)(a.nH * a.nW)), fd_nw((uint32_t)a.nW);   // block -> (frame, patch row, column)
    attn::RasterGrid rg{};
    if (a.raster) {
        rg.W = (uint32_t)a.W;
        rg.HW = (uint32_t)(a.H * a.W);
        rg.nHW = FastDiv((uint32_t)(a.nH * a.nW));
        rg.nW = FastDiv((uint32_t)a.nW);
    }
    const _Float16* kp = reinterpret_cast<const _Float16*>(a.kp);
    if (a.sip_budget > 0) {
        hipLaunchKernelGGL((map_select_kernel<D, NREG, true>), grid, dim3((kMapThreads<NREG, true>)), lds, s, a.q, a.bf16, a.raster,
                           rg, a.nb * 64, kp, a.kexp, a.nb, a.scale, a.thr, a.sta, fd_pf, fd_nw, a.rt, a.rh, a.rw,
                           a.kv_count, a.kv_index, a.bitmap, a.sip_budget, a.uniforms, a.kv_logw);
    } else {
        hipLaunchKernelGGL((map_select_kernel<D, NREG, false>), grid, dim3((kMapThreads<NREG, false>)), lds, s, a.q, a.bf16,
                           a.raster, rg, a.nb * 64, kp, a.kexp, a.nb, a.scale, a.thr, a.sta, fd_pf, fd_nw, a.rt,
                           a.rh, a.rw, a.kv_count, a.kv_index, a.bitmap, a.sip_budget, a.uniforms, a.kv_logw);
    }
    return hipGetLastError();
}

// registers per lane for a row of nb values: a multiple of 4 (one 256-column chunk)
// covering nb / 64
template <int D>
hipError_t launch_map_select_nreg(const MaskArgs& a, hipStream_t s) {
    static_assert(NABLA_MAX_BLOCKS <= 64 * 64, "rows of at most 64 registers per lane");
    if (a.nb <= 4 * 64) return launch_map_select<D, 4>(a, s);
    if (a.nb <= 8 * 64) return launch_map_select<D, 8>(a, s);
    if (a.nb <= 12 * 64) return launch_map_select<D, 12>(a, s);
    if (a.nb <= 16 * 64) return launch_map_select<D, 16>(a, s);
    if (a.nb <= 20 * 64) return launch_map_select<D, 20>(a, s);
    if (a.nb <= 24 * 64) return launch_map_select<D, 24>(a, s);
    if (a.nb <= 32 * 64) return launch_map_select<D, 32>(a, s);
    if (a.nb <= 48 * 64) return launch_map_select<D, 48>(a, s);
    return launch_map_select<D, 64>(a, s);
}

hipError_t launch_map_select_for(const MaskArgs& a, hipStream_t s) {
    return a.d == 128 ? launch_map_select_nreg<128>(a, s) : launch_map_select_nreg<64>(a, s);
}

hipError_t launch_select(const MaskArgs& a, hipStream_t s) {
    const int ld_s = ((a.nb + 63) / 64) * 64 + 16;
    const size_t lds = ((size_t)kSelWaves * ld_s + (size_t)kSelWaves * kCap) * sizeof(float);
    static std::atomic<uint64_t> lds_set{0};
    const int max_lds = (kSelWaves * (((NABLA_IBCS_MAX_BLOCKS + 63) / 64) * 64 + 16) + kSelWaves * kCap) * (int)sizeof(float);
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
    const int max_lds = (kRows * (((NABLA_IBCS_MAX_BLOCKS + 63) / 64) * 64 + 16) + kRows * kXld<D>) * (int)sizeof(float);
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
        e = launch_map_select_for(a, s);
    }
    if (e != hipSuccess || !a.schedule) return e;
    return launch_pair_schedule(a, a.kv_count, a.schedule, s);
}

hipError_t launch_pair_schedule(const MaskArgs& a, const int32_t* counts, int32_t* schedule, hipStream_t s) {
    // blocks per frame when frames hold whole N-token blocks, else 1 (blocks 2j, 2j + 1)
    const long long hw = (long long)a.H * a.W;
    const int fpf = (hw % a.N == 0 && a.nb % (int)(hw / a.N) == 0) ? (int)(hw / a.N) : 1;
    // one wave per head; its 2 nb + 1 bins and nb / 2 pair bins fit the default LDS limit
    static_assert((2 * NABLA_MAX_BLOCKS + 1 + NABLA_MAX_BLOCKS / 2) * 4 <= 64 * 1024, "schedule LDS");
    hipLaunchKernelGGL(pair_schedule_kernel, dim3(a.BH), dim3(64), (size_t)(2 * a.nb + 1 + a.nb / 2) * sizeof(int), s,
                       counts, a.nb, fpf, a.BH, schedule);
    return hipGetLastError();
}

hipError_t launch_schedule(const int32_t* counts, int BH, int nb, int32_t* schedule, hipStream_t s) {
    static_assert((2 * NABLA_MAX_BLOCKS + 1) * 4 <= 64 * 1024, "schedule LDS");
    hipLaunchKernelGGL(schedule_kernel, dim3(BH), dim3(64), (size_t)(2 * nb + 1) * sizeof(int), s, counts, nb,
                       schedule);
    return hipGetLastError();
}

}  // namespace nabla
