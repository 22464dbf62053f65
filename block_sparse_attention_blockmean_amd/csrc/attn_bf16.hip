// Block-sparse flash attention, bf16 in / bf16 out, for 64-token blocks.
//
// Computes softmax attention only on the kept 64 x 64 tiles (NABLA technical summary,
// "Metodologia: NABLA", item 2, "Expansão"); a dropped tile contributes neither to the
// numerator nor to the normaliser.
//
// One workgroup = one 64-row query block, two waves of 32 query rows each.  For every
// kept KV block the workgroup stages K (row-major) and V (transposed, d-major) in LDS
// and each wave runs
//     S^T = K Q^T      v_mfma_f32_32x32x16_bf16, A = K from LDS, B = Q from VGPRs
//     online softmax   float32, exp2 with scale*log2(e) folded into one FMA
//     O^T += V^T P^T   v_mfma_f32_32x32x16_bf16, A = V^T from LDS, B = P from VGPRs
// Computing the transposed products makes every lane own one query column: its S^T
// accumulator already has the layout the P operand of the second product needs (the
// MFMA's k index is permuted identically in both operands, which leaves the sum
// unchanged), and the row statistics (max, sum, rescale) stay in the lane, with one
// exchange between lanes l and l^32 that split the 64 keys of the tile.
#include <math.h>

#include "nabla_internal.h"

namespace nabla {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int kBlk = 64;
constexpr int kThreads = 128;
constexpr int kPadK = 8;   // bf16 elements of padding per K row in LDS
constexpr int kPadV = 8;   // bf16 elements of padding per V^T row in LDS

// Position of key kv (0..63) inside a V^T row in LDS.  The S^T accumulator of lane l
// (half h = l / 32) holds keys 32*T + 8*M + 4*h + C (register 4*M + C of tile T); the
// P operand of k-step u is registers 8*(u%2) .. 8*(u%2)+7 of tile u/2, so k-step u,
// half h, element e needs key 32*(u/2) + 8*(2*(u%2) + e/4) + 4*h + e%4.  Storing that
// key at 16*u + 8*h + e makes the matching V^T operand one contiguous 16-byte read.
__device__ inline int vt_pos(int kv) {
    const int T = kv >> 5, M = (kv >> 3) & 3, H = (kv >> 2) & 1, C = kv & 3;
    return 32 * T + 16 * (M >> 1) + 8 * H + 4 * (M & 1) + C;
}

template <int D>
__global__ __launch_bounds__(kThreads, 2) void attn_fwd_bf16_kernel(
    const __bf16* __restrict__ q, const __bf16* __restrict__ k, const __bf16* __restrict__ v,
    __bf16* __restrict__ o, int L, int nb, const int32_t* __restrict__ kv_count,
    const int32_t* __restrict__ kv_index, float scale_log2e) {
    constexpr int KS = D / 16;        // k-steps of S^T = K Q^T
    constexpr int DT = D / 32;        // 32-row d tiles of O^T
    constexpr int LDK = D + kPadK;
    constexpr int LDV = kBlk + kPadV;
    __shared__ __attribute__((aligned(16))) __bf16 k_lds[kBlk * LDK];
    __shared__ __attribute__((aligned(16))) __bf16 vt_lds[D * LDV];

    // Workgroups are dealt round-robin to the 8 XCDs; remap so that each XCD walks a
    // contiguous range of (head, query block) and neighbouring query blocks, which
    // keep similar KV lists, share that XCD's L2.
    const int G = gridDim.x;
    const int full = (G / 8) * 8;
    int logical = blockIdx.x;
    if (logical < full) logical = (logical % 8) * (G / 8) + logical / 8;
    const int bh = logical / nb;
    const int qb = logical - bh * nb;

    const int tid = threadIdx.x;
    const int wave = tid >> 6;
    const int lane = tid & 63;
    const int h = lane >> 5;
    const int c32 = lane & 31;

    const size_t head_off = (size_t)bh * L * D;
    const __bf16* qh = q + head_off;
    const __bf16* kh = k + head_off;
    const __bf16* vh = v + head_off;

    // Q operand: lane holds Q[row][16 s + 8 h .. + 7] for s = 0..KS-1.
    const int qrow = qb * kBlk + wave * 32 + c32;
    bf16x8 qreg[KS];
#pragma unroll
    for (int s = 0; s < KS; ++s)
        qreg[s] = *reinterpret_cast<const bf16x8*>(qh + (size_t)qrow * D + 16 * s + 8 * h);

    f32x16 oacc[DT];
#pragma unroll
    for (int t = 0; t < DT; ++t)
#pragma unroll
        for (int r = 0; r < 16; ++r) oacc[t][r] = 0.f;
    float m_run = -INFINITY;   // running max of scaled logits (log2 domain)
    float l_run = 0.f;         // this lane's share of the running normaliser

    const int count = kv_count[(size_t)bh * nb + qb];
    const int32_t* list = kv_index + ((size_t)bh * nb + qb) * nb;

    for (int it = 0; it < count; ++it) {
        const int j = list[it];
        const __bf16* kt = kh + (size_t)j * kBlk * D;
        const __bf16* vt = vh + (size_t)j * kBlk * D;
        __syncthreads();
        // ---- stage K: 16-byte chunks, 16 lanes per 256-byte row
        {
            constexpr int CH = D / 8;                  // chunks per row
            constexpr int PER = kBlk * CH / kThreads;  // chunks per thread
            uint4 buf[PER];
#pragma unroll
            for (int u = 0; u < PER; ++u) {
                const int id = tid + u * kThreads;
                const int row = id / CH, ch = id % CH;
                buf[u] = *reinterpret_cast<const uint4*>(kt + (size_t)row * D + ch * 8);
            }
#pragma unroll
            for (int u = 0; u < PER; ++u) {
                const int id = tid + u * kThreads;
                const int row = id / CH, ch = id % CH;
                *reinterpret_cast<uint4*>(k_lds + row * LDK + ch * 8) = buf[u];
            }
        }
        // ---- stage V transposed: a unit is 4 consecutive keys x 8 consecutive d
        {
            constexpr int DC = D / 8;
            constexpr int UNITS = 16 * DC;
            constexpr int PER = UNITS / kThreads;
            uint4 buf[PER][4];
#pragma unroll
            for (int u = 0; u < PER; ++u) {
                const int id = tid + u * kThreads;
                const int kg = id & 15, dc = id >> 4;
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    buf[u][i] = *reinterpret_cast<const uint4*>(vt + (size_t)(4 * kg + i) * D + 8 * dc);
            }
#pragma unroll
            for (int u = 0; u < PER; ++u) {
                const int id = tid + u * kThreads;
                const int kg = id & 15, dc = id >> 4;
                const int pos = vt_pos(4 * kg);
                const uint32_t* w0 = reinterpret_cast<const uint32_t*>(&buf[u][0]);
                const uint32_t* w1 = reinterpret_cast<const uint32_t*>(&buf[u][1]);
                const uint32_t* w2 = reinterpret_cast<const uint32_t*>(&buf[u][2]);
                const uint32_t* w3 = reinterpret_cast<const uint32_t*>(&buf[u][3]);
#pragma unroll
                for (int c = 0; c < 8; ++c) {
                    // element c of each of the 4 rows: low or high half of word c/2
                    const int sh = (c & 1) * 16;
                    const uint32_t e0 = (w0[c >> 1] >> sh) & 0xffffu;
                    const uint32_t e1 = (w1[c >> 1] >> sh) & 0xffffu;
                    const uint32_t e2 = (w2[c >> 1] >> sh) & 0xffffu;
                    const uint32_t e3 = (w3[c >> 1] >> sh) & 0xffffu;
                    uint2 pk;
                    pk.x = e0 | (e1 << 16);
                    pk.y = e2 | (e3 << 16);
                    *reinterpret_cast<uint2*>(vt_lds + (8 * dc + c) * LDV + pos) = pk;
                }
            }
        }
        __syncthreads();

        // ---- S^T = K Q^T for this wave's 32 query columns, 64 keys in two 32-key tiles
        f32x16 sacc[2];
#pragma unroll
        for (int t = 0; t < 2; ++t) {
#pragma unroll
            for (int r = 0; r < 16; ++r) sacc[t][r] = 0.f;
#pragma unroll
            for (int s = 0; s < KS; ++s) {
                const bf16x8 a = *reinterpret_cast<const bf16x8*>(k_lds + (32 * t + c32) * LDK + 16 * s + 8 * h);
                sacc[t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qreg[s], sacc[t], 0, 0, 0);
            }
        }

        // ---- online softmax for query column c32 (keys split between lanes l, l^32)
        float mx = -INFINITY;
#pragma unroll
        for (int t = 0; t < 2; ++t)
#pragma unroll
            for (int r = 0; r < 16; ++r) mx = fmaxf(mx, sacc[t][r]);
        mx = fmaxf(mx, __shfl_xor(mx, 32));
        const float m_new = fmaxf(m_run, mx * scale_log2e);
        const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
        m_run = m_new;
        float psum = 0.f;
        bf16x8 pb[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const float p = __builtin_amdgcn_exp2f(fmaf(sacc[u >> 1][8 * (u & 1) + e], scale_log2e, -m_new));
                psum += p;
                pb[u][e] = (__bf16)p;
            }
        }
        l_run = l_run * alpha + psum;
#pragma unroll
        for (int t = 0; t < DT; ++t)
#pragma unroll
            for (int r = 0; r < 16; ++r) oacc[t][r] *= alpha;

        // ---- O^T += V^T P^T
#pragma unroll
        for (int t = 0; t < DT; ++t) {
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                const bf16x8 a = *reinterpret_cast<const bf16x8*>(vt_lds + (32 * t + c32) * LDV + 16 * u + 8 * h);
                oacc[t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, pb[u], oacc[t], 0, 0, 0);
            }
        }
    }

    // ---- normalise and store: lane holds O[qrow][32 t + 8 g + 4 h + c], c = 0..3
    const float l_tot = l_run + __shfl_xor(l_run, 32);
    const float inv = (l_tot > 0.f) ? 1.0f / l_tot : 0.f;
    __bf16* orow = o + head_off + (size_t)qrow * D;
#pragma unroll
    for (int t = 0; t < DT; ++t) {
#pragma unroll
        for (int g = 0; g < 4; ++g) {
            bf16x4 pk;
#pragma unroll
            for (int c = 0; c < 4; ++c) pk[c] = (__bf16)(oacc[t][4 * g + c] * inv);
            *reinterpret_cast<bf16x4*>(orow + 32 * t + 8 * g + 4 * h) = pk;
        }
    }
}

template <int D>
hipError_t launch(const AttnArgs& a, hipStream_t s) {
    const float scale_log2e = a.scale * 1.4426950408889634f;
    hipLaunchKernelGGL((attn_fwd_bf16_kernel<D>), dim3(a.BH * a.nb), dim3(kThreads), 0, s,
                       (const __bf16*)a.q, (const __bf16*)a.k, (const __bf16*)a.v, (__bf16*)a.o,
                       a.L, a.nb, a.kv_count, a.kv_index, scale_log2e);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_attn_bf16(const AttnArgs& a, hipStream_t s) {
    return a.d == 128 ? launch<128>(a, s) : launch<64>(a, s);
}

}  // namespace nabla
