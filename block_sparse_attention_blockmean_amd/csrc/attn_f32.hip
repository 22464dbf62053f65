// Block-sparse attention in float32 for 64-token blocks: the same tiles as the bf16
// kernel (NABLA technical summary, "Metodologia: NABLA", item 2, "Expansão"), on plain
// float32 FMAs.  Serves float32 workloads such as small test grids; accuracy first.
//
// One workgroup = one 64-row query block, 256 threads: four threads per query row,
// each scoring 16 of the 64 keys of a tile and accumulating d/4 output columns.
#include <math.h>

#include "attn_tile.h"
#include "nabla_internal.h"

namespace nabla {
namespace {

constexpr int kBlk = 64;
constexpr int kThreads = 256;

using attn::RasterGrid;
using attn::block_row;
using attn::row_in_block;

template <int D, bool RASTER, bool WEIGHTED>
__global__ __launch_bounds__(kThreads) void attn_fwd_f32_kernel(
    const float* __restrict__ q, const float* __restrict__ k, const float* __restrict__ v,
    float* __restrict__ o, int L, int nb, const int32_t* __restrict__ kv_count,
    const int32_t* __restrict__ kv_index, const int32_t* __restrict__ schedule,
    RasterGrid grid, float scale, float* __restrict__ lse, const float* __restrict__ kv_logw) {
    constexpr int LD = D + 1;
    extern __shared__ float lds[];
    float* q_s = lds;                   // [64][LD]
    float* k_s = q_s + kBlk * LD;       // [64][LD]
    float* v_s = k_s + kBlk * LD;       // [64][LD]
    float* p_s = v_s + kBlk * LD;       // [64][65]

    const int blk = schedule ? schedule[blockIdx.x] : (int)blockIdx.x;
    const int bh = blk / nb;
    const int qb = blk - bh * nb;
    const int tid = threadIdx.x;
    const int row = tid >> 2;
    const int part = tid & 3;
    const size_t head_off = (size_t)bh * L * D;

    const uint32_t qbase = block_row<RASTER>(grid, qb);
    for (int i = tid; i < kBlk * D; i += kThreads)
        q_s[(i / D) * LD + i % D] = q[head_off + (size_t)(qbase + row_in_block<RASTER>(grid, i / D)) * D + i % D];

    float m_run = -INFINITY, l_run = 0.f;
    float acc[D / 4];
#pragma unroll
    for (int c = 0; c < D / 4; ++c) acc[c] = 0.f;

    const int count = kv_count[(size_t)bh * nb + qb];
    const int32_t* list = kv_index + ((size_t)bh * nb + qb) * nb;
    for (int it = 0; it < count; ++it) {
        const uint32_t jbase = block_row<RASTER>(grid, list[it]);
        const float wl = WEIGHTED ? kv_logw[((size_t)bh * nb + qb) * nb + it] : 0.f;
        __syncthreads();
        for (int i = tid; i < kBlk * D; i += kThreads) {
            const size_t src = head_off + (size_t)(jbase + row_in_block<RASTER>(grid, i / D)) * D + i % D;
            k_s[(i / D) * LD + i % D] = k[src];
            v_s[(i / D) * LD + i % D] = v[src];
        }
        __syncthreads();
        float s[16];
        float mx = -INFINITY;
#pragma unroll
        for (int c = 0; c < 16; ++c) {
            const int kv = part + 4 * c;
            float dot = 0.f;
            for (int e = 0; e < D; ++e) dot = fmaf(q_s[row * LD + e], k_s[kv * LD + e], dot);
            s[c] = dot * scale + wl;   // a sampled tile's log(1 / pi) shift
            mx = fmaxf(mx, s[c]);
        }
        mx = fmaxf(mx, __shfl_xor(mx, 1));
        mx = fmaxf(mx, __shfl_xor(mx, 2));
        const float m_new = fmaxf(m_run, mx);
        const float alpha = expf(m_run - m_new);
        float ps = 0.f;
#pragma unroll
        for (int c = 0; c < 16; ++c) {
            const float p = expf(s[c] - m_new);
            ps += p;
            p_s[row * 65 + part + 4 * c] = p;
        }
        l_run = l_run * alpha + ps;
        m_run = m_new;
        __syncthreads();
#pragma unroll
        for (int c = 0; c < D / 4; ++c) {
            const int col = part + 4 * c;
            float a = acc[c] * alpha;
            for (int kv = 0; kv < kBlk; ++kv) a = fmaf(p_s[row * 65 + kv], v_s[kv * LD + col], a);
            acc[c] = a;
        }
    }
    float l_tot = l_run + __shfl_xor(l_run, 1);
    l_tot += __shfl_xor(l_tot, 2);
    const float inv = (l_tot > 0.f) ? 1.0f / l_tot : 0.f;
    const uint32_t orow_idx = qbase + row_in_block<RASTER>(grid, row);
    if (lse && part == 0) lse[(size_t)bh * L + orow_idx] = l_tot > 0.f ? m_run + logf(l_tot) : -INFINITY;
    float* orow = o + head_off + (size_t)orow_idx * D;
#pragma unroll
    for (int c = 0; c < D / 4; ++c) orow[part + 4 * c] = acc[c] * inv;
}

template <int D, bool RASTER, bool WEIGHTED>
hipError_t launch(const AttnArgs& a, hipStream_t s) {
    const size_t lds = (3 * kBlk * (D + 1) + kBlk * 65) * sizeof(float);
    static std::atomic<uint64_t> lds_set{0};
    hipError_t e = set_max_dynamic_lds((const void*)attn_fwd_f32_kernel<D, RASTER, WEIGHTED>, (int)lds, lds_set);
    if (e != hipSuccess) return e;
    RasterGrid grid{};
    if (RASTER) {
        grid.W = (uint32_t)a.W;
        grid.HW = (uint32_t)(a.H * a.W);
        grid.nHW = FastDiv((uint32_t)((a.H / 8) * (a.W / 8)));
        grid.nW = FastDiv((uint32_t)(a.W / 8));
    }
    hipLaunchKernelGGL((attn_fwd_f32_kernel<D, RASTER, WEIGHTED>), dim3(a.BH * a.nb), dim3(kThreads), lds, s,
                       (const float*)a.q, (const float*)a.k, (const float*)a.v, (float*)a.o, a.L,
                       a.nb, a.kv_count, a.kv_index, a.schedule, grid, a.scale, a.lse, a.kv_logw);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_attn_f32(const AttnArgs& a, hipStream_t s) {
    if (a.kv_logw) return a.d == 128 ? launch<128, false, true>(a, s) : launch<64, false, true>(a, s);
    if (a.raster) return a.d == 128 ? launch<128, true, false>(a, s) : launch<64, true, false>(a, s);
    return a.d == 128 ? launch<128, false, false>(a, s) : launch<64, false, false>(a, s);
}

}  // namespace nabla
