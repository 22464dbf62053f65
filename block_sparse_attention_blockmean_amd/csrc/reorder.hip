// Fractal flattening of the token axis (NABLA technical summary, "Metodologia: NABLA",
// item 1): frames stay in time order, each P x P spatial patch becomes a contiguous
// run of P*P tokens.  Pure data movement, HBM bound: every element is read once and
// written once, 16 bytes per lane.
#include "nabla_internal.h"

namespace nabla {
namespace {

constexpr int kThreads = 256;
constexpr int kChunksPerThread = 4;

// One lane moves one 16-byte chunk of one destination token per step; consecutive
// lanes take consecutive chunks, so stores are fully coalesced and loads are
// coalesced over each run of P source tokens that a patch row holds.
__global__ __launch_bounds__(kThreads) void reorder_kernel(
    const u32x4* __restrict__ src, u32x4* __restrict__ dst, uint32_t chunks_per_head,
    int chunk_shift, FastDiv div_pp, FastDiv div_p, FastDiv div_patches_frame,
    FastDiv div_nw, FastDiv div_hw, FastDiv div_w, int P, int PP, int nH, int nW, int H,
    int W, int inverse) {
    const size_t head_off = (size_t)blockIdx.y * chunks_per_head;
    const uint32_t base = blockIdx.x * (kThreads * kChunksPerThread) + threadIdx.x;
    u32x4 buf[kChunksPerThread];
    uint32_t dst_idx[kChunksPerThread];
#pragma unroll
    for (int u = 0; u < kChunksPerThread; ++u) {
        const uint32_t i = base + u * kThreads;
        dst_idx[u] = i;
        if (i < chunks_per_head) {
            const uint32_t tok = i >> chunk_shift;
            const uint32_t c = i & ((1u << chunk_shift) - 1);
            uint32_t src_tok;
            if (!inverse) {
                // destination is fractal position tok -> raster source token
                uint32_t patch, within, py, px, t, rem, hb, wb;
                div_pp.divmod(tok, patch, within);
                div_p.divmod(within, py, px);
                div_patches_frame.divmod(patch, t, rem);
                div_nw.divmod(rem, hb, wb);
                src_tok = (t * H + hb * P + py) * W + wb * P + px;
            } else {
                // destination is raster token tok -> fractal source position
                uint32_t t, rem, y, x, hb, py, wb, px;
                div_hw.divmod(tok, t, rem);
                div_w.divmod(rem, y, x);
                div_p.divmod(y, hb, py);
                div_p.divmod(x, wb, px);
                src_tok = ((t * nH + hb) * nW + wb) * PP + py * P + px;
            }
            buf[u] = __builtin_nontemporal_load(src + head_off + ((size_t)src_tok << chunk_shift) + c);
        }
    }
#pragma unroll
    for (int u = 0; u < kChunksPerThread; ++u) {
        if (dst_idx[u] < chunks_per_head) {
            __builtin_nontemporal_store(buf[u], dst + head_off + dst_idx[u]);
        }
    }
}

}  // namespace

hipError_t launch_reorder(const ReorderArgs& a, hipStream_t s) {
    const int nH = a.H / a.P, nW = a.W / a.P;
    const uint32_t chunks_per_head = (uint32_t)a.L << a.chunk_shift;
    const uint32_t per_block = kThreads * kChunksPerThread;
    dim3 grid((chunks_per_head + per_block - 1) / per_block, a.BH);
    hipLaunchKernelGGL(reorder_kernel, grid, dim3(kThreads), 0, s, (const u32x4*)a.src,
                       (u32x4*)a.dst, chunks_per_head, a.chunk_shift,
                       FastDiv((uint32_t)(a.P * a.P)), FastDiv((uint32_t)a.P),
                       FastDiv((uint32_t)(nH * nW)), FastDiv((uint32_t)nW),
                       FastDiv((uint32_t)(a.H * a.W)), FastDiv((uint32_t)a.W), a.P, a.P * a.P,
                       nH, nW, a.H, a.W, a.inverse);
    return hipGetLastError();
}

}  // namespace nabla
