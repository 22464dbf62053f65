// IBCS query clustering (AB-Attention page, "Os três recursos do AB-Attention", first
// feature): the 64 queries of each query block are grouped into 8 clusters, each with
// a centroid and a weight equal to the fraction of the block's queries it holds.  The
// block scores A_ij = sum_c w_c softmax_j(scale * mu_c . Kp_j) are then formed by the
// map/select kernel, with the centroids as the rows of its reduced map.
//
// Clustering is Lloyd's k-means: initial centroids the queries at rows 0, 8, ..., 56,
// four rounds of assign-then-update, nearest centroid by squared Euclidean distance
// with ties to the lowest index, a centroid the mean of its queries (an empty cluster
// keeps its centroid).  Distances and means use individually rounded float32 operations
// in a fixed order - per coordinate the difference, its square, a running sum over d in
// index order; a running sum over the cluster's queries in row order, then one division
// - so the assignment is a function of the inputs alone, the same on any machine that
// performs those operations in that order.
#include <math.h>

#include "nabla_internal.h"

namespace nabla {
namespace {

constexpr int kBlkQ = 64;       // queries per block
constexpr int kThreads = 256;
constexpr int kPerQuery = kThreads / kBlkQ;                 // threads per query in the assign step
constexpr int kPerThread = kIbcsClusters / kPerQuery;       // centroids each of them measures
constexpr int kPerCluster = kThreads / kIbcsClusters;       // threads per centroid in the update step
static_assert(kIbcsClusters % kPerQuery == 0 && kThreads % kIbcsClusters == 0, "thread split");
static_assert(kBlkQ % kIbcsClusters == 0, "initial centroids are every (64 / k)-th query");

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

// One workgroup per query block (bh * nb + i).  LDS rows are padded by 16 bytes (d + 4
// floats): row t starts 4 t banks further on, so the 16 queries a wave reads with one
// 16-byte load fall in distinct bank groups.  Float contraction is off in the whole
// kernel: each +, - and * rounds on its own, and the division is the correctly rounded
// one (hipcc's default for float32 division).
template <typename T, int D>
__global__ __launch_bounds__(kThreads) void ibcs_cluster_kernel(const T* __restrict__ q, float* __restrict__ cent,
                                                                float* __restrict__ weight) {
#pragma clang fp contract(off)
    constexpr int LD = D + 4;
    constexpr int EPC = 16 / sizeof(T);                       // elements per 16-byte chunk
    __shared__ __align__(16) float xq[kBlkQ * LD];
    __shared__ __align__(16) float cen[kIbcsClusters * LD];
    __shared__ float dist[kThreads];
    __shared__ int best[kThreads];
    __shared__ int members[kIbcsClusters * kBlkQ];           // each cluster's queries in row order
    __shared__ int counts[kIbcsClusters];

    const size_t blk = blockIdx.x;
    const int tid = threadIdx.x;
    const u32x4_t* src = reinterpret_cast<const u32x4_t*>(q + blk * kBlkQ * D);
    for (int ch = tid; ch < kBlkQ * D / EPC; ch += kThreads) {
        float v[EPC];
        unpack16(__builtin_nontemporal_load(src + ch), T{}, v);
        const int row = ch / (D / EPC), col = (ch % (D / EPC)) * EPC;
#pragma unroll
        for (int e = 0; e < EPC; e += 4)
            *reinterpret_cast<float4*>(xq + row * LD + col + e) = make_float4(v[e], v[e + 1], v[e + 2], v[e + 3]);
    }
    __syncthreads();
    for (int e = tid; e < kIbcsClusters * D; e += kThreads) {
        const int c = e / D, col = e % D;
        cen[c * LD + col] = xq[c * (kBlkQ / kIbcsClusters) * LD + col];
    }
    __syncthreads();

    for (int it = 0; it < kIbcsIters; ++it) {
        // assign, part 1: thread (query t, slot p) measures centroids kPerThread p + m,
        // coordinates in index order
        {
            const int t = tid / kPerQuery, p = tid % kPerQuery;
            const float4* x4 = reinterpret_cast<const float4*>(xq + t * LD);
            const float4* c4 = reinterpret_cast<const float4*>(cen + p * kPerThread * LD);
            float acc[kPerThread];
#pragma unroll
            for (int m = 0; m < kPerThread; ++m) acc[m] = 0.f;
#pragma unroll 4
            for (int e4 = 0; e4 < D / 4; ++e4) {
                const float4 xv = x4[e4];
#pragma unroll
                for (int m = 0; m < kPerThread; ++m) {
                    const float4 cv = c4[m * (LD / 4) + e4];
                    float df = xv.x - cv.x;
                    float sq = df * df;
                    acc[m] = acc[m] + sq;
                    df = xv.y - cv.y;
                    sq = df * df;
                    acc[m] = acc[m] + sq;
                    df = xv.z - cv.z;
                    sq = df * df;
                    acc[m] = acc[m] + sq;
                    df = xv.w - cv.w;
                    sq = df * df;
                    acc[m] = acc[m] + sq;
                }
            }
            float bd = acc[0];
            int bc = p * kPerThread;
#pragma unroll
            for (int m = 1; m < kPerThread; ++m) {
                if (acc[m] < bd) {     // strict: a tie keeps the lower index
                    bd = acc[m];
                    bc = p * kPerThread + m;
                }
            }
            dist[tid] = bd;
            best[tid] = bc;
        }
        __syncthreads();
        // assign, part 2 (wave 0, lane = query): the slots hold increasing cluster
        // ranges, so a strict compare in slot order keeps the lowest index among equal
        // distances.  Each cluster's member list is then filled in row order by ballot
        // ranks.
        if (tid < kBlkQ) {
            float bd = dist[tid * kPerQuery];
            int bc = best[tid * kPerQuery];
#pragma unroll
            for (int p = 1; p < kPerQuery; ++p) {
                const float dd = dist[tid * kPerQuery + p];
                if (dd < bd) {
                    bd = dd;
                    bc = best[tid * kPerQuery + p];
                }
            }
            const uint64_t below = (1ull << tid) - 1ull;
#pragma unroll
            for (int c = 0; c < kIbcsClusters; ++c) {
                const uint64_t in = __ballot(bc == c);
                if (bc == c) members[c * kBlkQ + __popcll(in & below)] = tid;
                if (tid == 0) counts[c] = __popcll(in);
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
                const float* x = xq + members[c * kBlkQ + n] * LD + part;
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

    float* out = cent + blk * kIbcsClusters * D;
    for (int e = tid; e < kIbcsClusters * D; e += kThreads) out[e] = cen[(e / D) * LD + e % D];
    if (tid < kIbcsClusters) weight[blk * kIbcsClusters + tid] = (float)counts[tid] / (float)kBlkQ;
}

template <typename T, int D>
hipError_t launch(const MaskArgs& a, hipStream_t s) {
    hipLaunchKernelGGL((ibcs_cluster_kernel<T, D>), dim3(a.BH * a.nb), dim3(kThreads), 0, s, (const T*)a.q,
                       a.cent, a.cent_w);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_ibcs_cluster(const MaskArgs& a, hipStream_t s) {
    if (a.bf16) return a.d == 128 ? launch<__bf16, 128>(a, s) : launch<__bf16, 64>(a, s);
    return a.d == 128 ? launch<float, 128>(a, s) : launch<float, 64>(a, s);
}

}  // namespace nabla
