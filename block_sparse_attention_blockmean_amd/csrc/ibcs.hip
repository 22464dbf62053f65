// IBCS query clustering (AB-Attention page, "Os três recursos do AB-Attention", first
// feature): the queries of each group of QN consecutive tokens (one 64-token block, or
// the page's 128-token blocks) are grouped into 8 clusters, each with a centroid and a
// weight equal to the fraction of the group's queries it holds.  The block scores
// A_ij = sum_c w_c softmax_j(scale * mu_c . Kp_j) are then formed in mask.hip, with the
// centroids as the rows of the reduced map.
//
// Clustering is Lloyd's k-means: initial centroids the queries at rows 0, QN/8, ...,
// four rounds of assign-then-update, nearest centroid by squared Euclidean distance
// with ties to the lowest index, a centroid the mean of its queries (an empty cluster
// keeps its centroid).  Distances and means use float32 operations in a fixed order -
// per coordinate in index order the rounded difference, then its square added to the
// running sum by one fused multiply-add; a running sum over the cluster's queries in row
// order, then one division - so the assignment is a function of the inputs alone, the
// same on any machine that performs those operations in that order.
#include <math.h>

#include "attn_tile.h"
#include "nabla_internal.h"

namespace nabla {
namespace {

// Four threads per query: 256 for a 64-query group, 512 for 128.
template <int QN>
constexpr int cluster_threads() {
    return 4 * QN;
}

typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

__device__ inline void unpack16(const u32x4_t& v, __bf16, float* out) {
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        out[2 * i] = __uint_as_float(w[i] << 16);
        out[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
    }
}
__device__ inline void unpack16(const u32x4_t& v, float, float* out) {
    out[0] = __uint_as_float(v.x);
    out[1] = __uint_as_float(v.y);
    out[2] = __uint_as_float(v.z);
    out[3] = __uint_as_float(v.w);
}

// Dynamic LDS of one workgroup: queries, centroids, per-thread best distance and
// cluster, member lists and counts.
template <int D, int QN>
constexpr size_t cluster_lds_bytes() {
    constexpr int NT = cluster_threads<QN>();
    return ((size_t)QN * (D + 4) + (size_t)kIbcsClusters * (D + 4) + NT) * sizeof(float) +
           ((size_t)NT + (size_t)kIbcsClusters * QN + kIbcsClusters) * sizeof(int);
}

// One workgroup per query group (bh * groups + g).  In fractal order the group is QN
// consecutive rows; in raster order (RASTER) its 64-token blocks are the 8 x 8 patches
// that fractal order numbers g * QN / 64, ..., read through the patch addressing.  LDS rows are padded by 16 bytes
// (d + 4 floats): row t starts 4 t banks further on, so the 16 queries a wave reads with
// one 16-byte load fall in distinct bank groups.  Float contraction is off in the whole
// kernel, so the only fused operations are the explicit fmaf of the distances; every
// other +, - and * rounds on its own, and the division is the correctly rounded one
// (hipcc's default for float32 division).
template <typename T, int D, int QN, bool RASTER>
__global__ __launch_bounds__(cluster_threads<QN>()) void ibcs_cluster_kernel(const T* __restrict__ q,
                                                                             float* __restrict__ cent,
                                                                             float* __restrict__ weight, int groups,
                                                                             int L, attn::RasterGrid grid) {
#pragma clang fp contract(off)
    constexpr int kThreads = cluster_threads<QN>();
    constexpr int kPerCluster = kThreads / kIbcsClusters;     // threads per centroid in the update step
    constexpr int LD = D + 4;
    constexpr int EPC = 16 / sizeof(T);                       // elements per 16-byte chunk
    constexpr int PQ = kThreads / QN;                         // threads per query in the assign step
    constexpr int PT = kIbcsClusters / PQ;                    // centroids each of them measures
    static_assert(QN % 64 == 0 && kThreads % QN == 0 && kIbcsClusters % PQ == 0, "thread split");
    static_assert(kThreads % kIbcsClusters == 0 && D % kPerCluster == 0, "update split");
    static_assert(QN % kIbcsClusters == 0, "initial centroids are every (QN / k)-th query");
    extern __shared__ __align__(16) float lds[];
    float* xq = lds;                                          // [QN][LD]
    float* cen = xq + QN * LD;                                // [k][LD]
    float* dist = cen + kIbcsClusters * LD;                   // [kThreads]
    int* best = reinterpret_cast<int*>(dist + kThreads);      // [kThreads]
    int* members = best + kThreads;                           // [k][QN] each cluster's queries in row order
    int* counts = members + kIbcsClusters * QN;               // [k]

    const size_t grp = blockIdx.x;
    const int tid = threadIdx.x;
    for (int ch = tid; ch < QN * D / EPC; ch += kThreads) {
        float v[EPC];
        const int row = ch / (D / EPC), col = (ch % (D / EPC)) * EPC;
        size_t token;
        if (RASTER) {
            const size_t bh = grp / groups;
            const uint32_t blk = (uint32_t)(grp - bh * groups) * (QN / 64) + row / 64;
            token = bh * L + attn::block_row<true>(grid, blk) + attn::row_in_block<true>(grid, row % 64);
        } else {
            token = grp * QN + row;
        }
        unpack16(__builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(q + token * D + col)), T{}, v);
#pragma unroll
        for (int e = 0; e < EPC; e += 4)
            *reinterpret_cast<float4*>(xq + row * LD + col + e) = make_float4(v[e], v[e + 1], v[e + 2], v[e + 3]);
    }
    __syncthreads();
    for (int e = tid; e < kIbcsClusters * D; e += kThreads) {
        const int c = e / D, col = e % D;
        cen[c * LD + col] = xq[c * (QN / kIbcsClusters) * LD + col];
    }
    __syncthreads();

    for (int it = 0; it < kIbcsIters; ++it) {
        // assign, part 1: thread (query t, slot p) measures centroids PT p + m,
        // coordinates in index order
        {
            const int t = tid / PQ, p = tid % PQ;
            const float4* x4 = reinterpret_cast<const float4*>(xq + t * LD);
            const float4* c4 = reinterpret_cast<const float4*>(cen + p * PT * LD);
            float acc[PT];
#pragma unroll
            for (int m = 0; m < PT; ++m) acc[m] = 0.f;
#pragma unroll 4
            for (int e4 = 0; e4 < D / 4; ++e4) {
                const float4 xv = x4[e4];
#pragma unroll
                for (int m = 0; m < PT; ++m) {
                    const float4 cv = c4[m * (LD / 4) + e4];
                    float df = xv.x - cv.x;
                    acc[m] = fmaf(df, df, acc[m]);
                    df = xv.y - cv.y;
                    acc[m] = fmaf(df, df, acc[m]);
                    df = xv.z - cv.z;
                    acc[m] = fmaf(df, df, acc[m]);
                    df = xv.w - cv.w;
                    acc[m] = fmaf(df, df, acc[m]);
                }
            }
            float bd = acc[0];
            int bc = p * PT;
#pragma unroll
            for (int m = 1; m < PT; ++m) {
                if (acc[m] < bd) {     // strict: a tie keeps the lower index
                    bd = acc[m];
                    bc = p * PT + m;
                }
            }
            dist[tid] = bd;
            best[tid] = bc;
        }
        __syncthreads();
        // assign, part 2 (wave 0, 64 queries at a time): the slots hold increasing
        // cluster ranges, so a strict compare in slot order keeps the lowest index among
        // equal distances.  Each cluster's member list is filled in row order by ballot
        // ranks; base[c] is the same in every lane.
        if (tid < 64) {
            const uint64_t below = (1ull << tid) - 1ull;
            int base[kIbcsClusters];
#pragma unroll
            for (int c = 0; c < kIbcsClusters; ++c) base[c] = 0;
            for (int ch = 0; ch < QN / 64; ++ch) {
                const int t = ch * 64 + tid;
                float bd = dist[t * PQ];
                int bc = best[t * PQ];
#pragma unroll
                for (int p = 1; p < PQ; ++p) {
                    const float dd = dist[t * PQ + p];
                    if (dd < bd) {
                        bd = dd;
                        bc = best[t * PQ + p];
                    }
                }
#pragma unroll
                for (int c = 0; c < kIbcsClusters; ++c) {
                    const uint64_t in = __ballot(bc == c);
                    if (bc == c) members[c * QN + base[c] + __popcll(in & below)] = t;
                    base[c] += __popcll(in);
                }
            }
            if (tid == 0) {
#pragma unroll
                for (int c = 0; c < kIbcsClusters; ++c) counts[c] = base[c];
            }
        }
        __syncthreads();
        // update: thread (cluster c, part) owns coordinates part, part + kPerCluster, ...
        // and sums them over the cluster's queries in row order
        {
            const int c = tid / kPerCluster, part = tid % kPerCluster;
            constexpr int NC = D / kPerCluster;
            const int cnt = counts[c];
            float acc[NC];
#pragma unroll
            for (int m = 0; m < NC; ++m) acc[m] = 0.f;
            for (int n = 0; n < cnt; ++n) {
                const float* x = xq + members[c * QN + n] * LD + part;
#pragma unroll
                for (int m = 0; m < NC; ++m) acc[m] = acc[m] + x[m * kPerCluster];
            }
            if (cnt > 0) {
                const float fc = (float)cnt;
#pragma unroll
                for (int m = 0; m < NC; ++m) cen[c * LD + part + m * kPerCluster] = acc[m] / fc;
            }
        }
        __syncthreads();
    }

    float* out = cent + grp * kIbcsClusters * D;
    for (int e = tid; e < kIbcsClusters * D; e += kThreads) out[e] = cen[(e / D) * LD + e % D];
    if (tid < kIbcsClusters) weight[grp * kIbcsClusters + tid] = (float)counts[tid] / (float)QN;
}

template <typename T, int D, int QN, bool RASTER>
hipError_t launch(const MaskArgs& a, hipStream_t s) {
    constexpr size_t lds = cluster_lds_bytes<D, QN>();
    static std::atomic<uint64_t> lds_set{0};
    hipError_t e = set_max_dynamic_lds((const void*)ibcs_cluster_kernel<T, D, QN, RASTER>, (int)lds, lds_set);
    if (e != hipSuccess) return e;
    const int groups = a.nb / a.ibcs_group;
    attn::RasterGrid grid{};
    if (RASTER) {
        grid.W = (uint32_t)a.W;
        grid.HW = (uint32_t)(a.H * a.W);
        grid.nHW = FastDiv((uint32_t)(a.nH * a.nW));
        grid.nW = FastDiv((uint32_t)a.nW);
    }
    hipLaunchKernelGGL((ibcs_cluster_kernel<T, D, QN, RASTER>), dim3(a.BH * groups), dim3(cluster_threads<QN>()), lds,
                       s, (const T*)a.q, a.cent, a.cent_w, groups, a.nb * 64, grid);
    return hipGetLastError();
}

template <typename T, int D, int QN>
hipError_t launch_r(const MaskArgs& a, hipStream_t s) {
    return a.raster ? launch<T, D, QN, true>(a, s) : launch<T, D, QN, false>(a, s);
}

template <typename T>
hipError_t launch_t(const MaskArgs& a, hipStream_t s) {
    if (a.ibcs_group == 2) return a.d == 128 ? launch_r<T, 128, 128>(a, s) : launch_r<T, 64, 128>(a, s);
    return a.d == 128 ? launch_r<T, 128, 64>(a, s) : launch_r<T, 64, 64>(a, s);
}

}  // namespace

hipError_t launch_ibcs_cluster(const MaskArgs& a, hipStream_t s) {
    return a.bf16 ? launch_t<__bf16>(a, s) : launch_t<float>(a, s);
}

}  // namespace nabla
