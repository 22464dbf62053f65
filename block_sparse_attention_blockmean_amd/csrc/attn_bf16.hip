// Block-sparse flash attention, bf16 in / bf16 out, for 64-token blocks.
//
// Computes softmax attention only on the kept 64 x 64 tiles (NABLA technical summary,
// "Metodologia: NABLA", item 2, "Expansão"); a dropped tile contributes neither to the
// numerator nor to the normaliser.
//
// One workgroup = one 64-row query block, four waves.  Wave (qh, kh) takes query rows
// [32 qh, 32 qh + 32) against keys [32 kh, 32 kh + 32) of every kept KV tile, with its
// own running maximum, normaliser and output; the two key halves of each query half are
// merged once at the end.  Per tile, each wave runs
//     S^T = K Q^T      v_mfma_f32_32x32x16_bf16, A = 32 keys of K from LDS, B = Q (VGPRs)
//     online softmax   float32, exp2 with scale*log2(e) folded into one FMA
//     O^T += V^T P^T   v_mfma_f32_32x32x16_bf16, A = V^T from LDS, B = P (VGPRs)
// Computing the transposed products makes every lane own one query column: its S^T
// accumulator already has the layout the P operand of the second product needs (the
// MFMA's k index is permuted identically in both operands, which leaves the sum
// unchanged), and the row statistics stay in the lane, with one exchange between lanes
// l and l^32, which split the wave's 32 keys.
//
// Memory pipeline: K and V tiles go from global memory straight into LDS with the
// buffer form of the LDS DMA (buffer_load_dwordx4 ... lds, no VGPR staging), row-major
// with an XOR swizzle of the 16-byte chunks, and are double-buffered: at the top of
// iteration i, after one barrier, the workgroup issues K(i+1) and V(i+1), which have the
// whole iteration to land.  64 KiB of LDS per workgroup and ~170 VGPRs per wave put two
// workgroups on a CU, two waves on every SIMD.  V^T operands come out of the row-major V
// tile through the transposing LDS read (ds_read_b64_tr_b16).  The four buffers are
// separate LDS objects, so the compiler sees that reading one never waits for a copy
// into another.
#include <math.h>

#include <type_traits>

#include "attn_tile.h"
#include "nabla_internal.h"

namespace nabla {
namespace {

using namespace attn;

template <int D, bool RASTER, bool WEIGHTED>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(2, 2)))
void attn_fwd_bf16_kernel(const __bf16* __restrict__ q, const __bf16* __restrict__ k,
                          const __bf16* __restrict__ v, __bf16* __restrict__ o, int L, int nb,
                          const int32_t* __restrict__ kv_count, const int32_t* __restrict__ kv_index,
                          const int32_t* __restrict__ schedule, RasterGrid grid, float scale_log2e,
                          float* __restrict__ lse, const float* __restrict__ kv_logw) {
    using G = Tile<D>;
    constexpr int KS = D / 16;        // k-steps of S^T = K Q^T
    constexpr int DT = D / 32;        // 32-row d tiles of O^T
    const uint32_t stride = copy_stride<RASTER>(grid);   // between a tile's 4 KiB copies
    __shared__ __attribute__((aligned(1024))) char k_lds0[G::kBytes];
    __shared__ __attribute__((aligned(1024))) char k_lds1[G::kBytes];
    __shared__ __attribute__((aligned(1024))) char v_lds0[G::kBytes];
    __shared__ __attribute__((aligned(1024))) char v_lds1[G::kBytes];

    // Workgroups are dealt round-robin to the 8 XCDs; without a schedule, remap so that
    // each XCD walks a contiguous range of (head, query block).  With a schedule,
    // workgroups take query blocks in its order (heads in turn, longest lists first).
    const int nwg = gridDim.x;
    const int full = (nwg / 8) * 8;
    int logical = blockIdx.x;
    if (schedule) {
        logical = schedule[logical];
    } else if (logical < full) {
        logical = (logical % 8) * (nwg / 8) + logical / 8;
    }
    const int bh = logical / nb;
    const int qb = logical - bh * nb;

    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // uniform per wave
    const int qhalf = wave & 1;
    const int khalf = wave >> 1;
    const int lane = tid & 63;
    const int h = lane >> 5;
    const int c32 = lane & 31;

    const size_t head_off = (size_t)bh * L * D;
    const __bf16* qh = q + head_off;
    const int head_bytes = L * D * 2;
    const __amdgpu_buffer_rsrc_t k_rsrc =
        __builtin_amdgcn_make_buffer_rsrc((void*)(k + head_off), 0, head_bytes, kBufferFlags);
    const __amdgpu_buffer_rsrc_t v_rsrc =
        __builtin_amdgcn_make_buffer_rsrc((void*)(v + head_off), 0, head_bytes, kBufferFlags);
    const uint32_t k_copy = copy_lane_offset_in<D, false, RASTER>(grid, wave, lane);
    const uint32_t v_copy = copy_lane_offset_in<D, true, RASTER>(grid, wave, lane);

    const int count = kv_count[(size_t)bh * nb + qb];
    const int32_t* list = kv_index + ((size_t)bh * nb + qb) * nb;

    if (count > 0) {
        const uint32_t first = block_row<RASTER>(grid, list[0]) * G::kRowBytes;
        copy_tile<D>(k_rsrc, first, k_lds0, wave, k_copy, stride);
        copy_tile<D>(v_rsrc, first, v_lds0, wave, v_copy, stride);
    }

    // Q operand: lane holds Q[row][16 s + 8 h .. + 7] for s = 0..KS-1.
    // the lane's query row in the head (fractal or raster order)
    const uint32_t qrow = block_row<RASTER>(grid, qb) + row_in_block<RASTER>(grid, 32 * qhalf + c32);
    bf16x8 qreg[KS];
#pragma unroll
    for (int s = 0; s < KS; ++s)
        qreg[s] = *reinterpret_cast<const bf16x8*>(qh + (size_t)qrow * D + 16 * s + 8 * h);

    f32x16 oacc[DT];
#pragma unroll
    for (int t = 0; t < DT; ++t)
#pragma unroll
        for (int r = 0; r < 16; ++r) oacc[t][r] = 0.f;
    float m_run = -INFINITY;   // reference max of scaled logits (log2 domain), same in l, l^32
    float l_run = 0.f;         // this lane's share of the running normaliser

    // per-lane LDS byte offsets that do not change from tile to tile
    const int krow = 32 * khalf + c32;
    int k_off[KS];
#pragma unroll
    for (int s = 0; s < KS; ++s) k_off[s] = krow * G::kRowBytes + (((2 * s + h) ^ G::k_swz(krow)) * 16);
    // V^T operand of d tile t, k-step u, half p: rows 32 kh + 16 u + 8 p + 4 h + j16 / 4;
    // only the d tile changes the swizzled part, (16 u + 8 p) rows are a constant offset
    const int g16 = lane >> 4, j16 = lane & 15;
    int v_off[DT];
#pragma unroll
    for (int t = 0; t < DT; ++t) {
        const int row = 32 * khalf + 4 * h + (j16 >> 2);
        const int d = 32 * t + 16 * (g16 & 1) + 4 * (j16 & 3);
        v_off[t] = row * G::kRowBytes + (((d >> 3) ^ G::v_swz(row)) * 16) + ((d >> 2) & 1) * 8;
    }

    // KV block copied during iteration i: list[i+1], and the last block again at the last
    // iteration (into the buffer nothing reads any more), which keeps the copies unconditional
    int next_tile = list[count > 1 ? 1 : 0];   // in bounds also when count is 0 (then unused)

    // One tile; PAR = i % 2 selects the buffers holding K(i) and V(i).
    auto step = [&](auto par, int i) {
        constexpr int PAR = decltype(par)::value;
        const char* kbuf = PAR ? k_lds1 : k_lds0;
        const char* vbuf = PAR ? v_lds1 : v_lds0;
        // K(i) and V(i) have landed (issued one iteration ago); after the barrier every
        // wave sees them and is done with the buffers of tile i - 1, refilled now
        wait_vmcnt<0>();
        lds_barrier();
        // the tile's additive logit shift (log2 units): a sampled block's log(1 / pi)
        const float wl = WEIGHTED ? kv_logw[((size_t)bh * nb + qb) * nb + i] * 1.4426950408889634f : 0.f;
        const uint32_t nxt = block_row<RASTER>(grid, next_tile) * G::kRowBytes;
        char* k_dst = PAR ? k_lds0 : k_lds1;
        char* v_dst = PAR ? v_lds0 : v_lds1;

        // ---- S^T = K Q^T for this wave's 32 keys and 32 query columns (all K operands
        // requested first; each MFMA waits only for its own)
        f32x16 sacc;
#pragma unroll
        for (int r = 0; r < 16; ++r) sacc[r] = 0.f;
        bf16x8 ka[KS];
#pragma unroll
        for (int s = 0; s < KS; ++s) ka[s] = *reinterpret_cast<const bf16x8*>(kbuf + k_off[s]);
        __builtin_amdgcn_sched_barrier(0);
        // the wave's copies of K(i+1), one after every other MFMA
#pragma unroll
        for (int s = 0; s < KS; ++s) {
            sacc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka[s], qreg[s], sacc, 0, 0, 0);
            constexpr int kEvery = KS / G::kCopiesPerWave;
            if (s % kEvery == 0)
                __builtin_amdgcn_raw_ptr_buffer_load_lds(k_rsrc, (lds_void*)(k_dst + (4 * (s / kEvery) + wave) * 1024), 16,
                                                         k_copy, nxt + (s / kEvery) * stride, 0, 0);
            __builtin_amdgcn_sched_barrier(0);
        }

        // ---- online softmax for query column c32 (keys split between lanes l, l^32).
        // The reference maximum m_run only moves when a tile's maximum exceeds it by
        // more than 8 (log2 units), so P stays below 2^8 and the rescale of O and l is
        // rare; normalising by l at the end makes the result independent of m_run.
        float mx = -INFINITY;
#pragma unroll
        for (int r = 0; r < 16; ++r) mx = fmaxf(mx, sacc[r]);
        {
            const auto pr = __builtin_amdgcn_permlane32_swap(__float_as_uint(mx), __float_as_uint(mx), false, false);
            mx = fmaxf(__uint_as_float(pr[0]), __uint_as_float(pr[1])) * scale_log2e + wl;
        }
        if (__ballot(mx > m_run + 8.0f)) {
            const float m_new = fmaxf(m_run, mx);
            const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
            m_run = m_new;
            l_run *= alpha;
#pragma unroll
            for (int t = 0; t < DT; ++t)
#pragma unroll
                for (int r = 0; r < 16; ++r) oacc[t][r] *= alpha;
        }

        // ---- O^T += V^T P^T over the wave's two 16-key k-steps; P of k-step u is
        // accumulator entries 8u .. 8u+7
        bf16x8 pb[2];
#pragma unroll
        for (int u = 0; u < 2; ++u)
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const float pe = __builtin_amdgcn_exp2f(fmaf(sacc[8 * u + e], scale_log2e, wl - m_run));
                l_run += pe;
                pb[u][e] = (__bf16)pe;
            }
#pragma unroll
        for (int u = 0; u < 2; ++u)
#pragma unroll
            for (int t = 0; t < DT; ++t) {
                // the wave's copies of V(i+1), one after every other MFMA
                constexpr int kEveryV = 2 * DT / G::kCopiesPerWave;
                const int m = u * DT + t;
                if (m % kEveryV == 0)
                    __builtin_amdgcn_raw_ptr_buffer_load_lds(v_rsrc, (lds_void*)(v_dst + (4 * (m / kEveryV) + wave) * 1024), 16,
                                                             v_copy, nxt + (m / kEveryV) * stride, 0, 0);
                const s16x4 v0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                    (lds_s16x4*)(vbuf + v_off[t] + (16 * u) * G::kRowBytes));
                const s16x4 v1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                    (lds_s16x4*)(vbuf + v_off[t] + (16 * u + 8) * G::kRowBytes));
                const bf16x8 a = __builtin_bit_cast(bf16x8, __builtin_shufflevector(v0, v1, 0, 1, 2, 3, 4, 5, 6, 7));
                oacc[t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, pb[u], oacc[t], 0, 0, 0);
            }
        // the tile the next iteration copies, read after this one's last LDS wait so that
        // the scalar load is done by the barrier that opens the next iteration
        __builtin_amdgcn_sched_barrier(0);
        next_tile = list[min(i + 2, count - 1)];
    };

    using P0 = std::integral_constant<int, 0>;
    using P1 = std::integral_constant<int, 1>;
    for (int i = 0; i < count; i += 2) {
        step(P0{}, i);
        if (i + 1 < count) step(P1{}, i + 1);
    }

    // ---- merge the key halves: wave (qh, 1) hands its partial output, maximum and
    // normaliser to wave (qh, 0), which finishes query rows 32 qh .. 32 qh + 31.  The
    // last iteration's copies (of the last block again, into buffers no longer read) must
    // land before the buffers are reused; the barrier then ends every read of them.
    wait_vmcnt<0>();
    lds_barrier();
    float* xo = reinterpret_cast<float*>(qhalf ? k_lds1 : k_lds0);   // DT*16*64 floats
    float* xs = reinterpret_cast<float*>(v_lds0) + qhalf * 128;      // m, l per lane
    static_assert(DT * 16 * 64 * 4 <= G::kBytes, "partial output exceeds one tile buffer");
    if (khalf == 1) {
#pragma unroll
        for (int t = 0; t < DT; ++t)
#pragma unroll
            for (int r = 0; r < 16; ++r) xo[(t * 16 + r) * 64 + lane] = oacc[t][r];
        xs[lane] = m_run;
        xs[64 + lane] = l_run;
    }
    lds_barrier();
    if (khalf == 0) {
        const float m_p = xs[lane];
        const float l_p = xs[64 + lane];
        const float m = fmaxf(m_run, m_p);
        const float a_s = m_run == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(m_run - m);
        const float a_p = m_p == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(m_p - m);
        float l = l_run * a_s + l_p * a_p;
        {
            const auto pr = __builtin_amdgcn_permlane32_swap(__float_as_uint(l), __float_as_uint(l), false, false);
            l = __uint_as_float(pr[0]) + __uint_as_float(pr[1]);
        }
        const float inv = (l > 0.f) ? 1.0f / l : 0.f;
        // log-sum-exp of the row's scaled logits: P = exp2(s * scale * log2(e) - m) / l,
        // so the sum of exp(s * scale) is 2^m * l
        if (lse && h == 0)
            lse[(size_t)bh * L + qrow] = l > 0.f ? (m + __log2f(l)) * 0.69314718055994531f : -INFINITY;
        // lane holds O[qrow][32 t + 8 g + 4 h + c], c = 0..3
        __bf16* orow = o + head_off + (size_t)qrow * D;
#pragma unroll
        for (int t = 0; t < DT; ++t)
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                bf16x4 pk;
#pragma unroll
                for (int c = 0; c < 4; ++c) {
                    const int r = 4 * g + c;
                    pk[c] = (__bf16)((oacc[t][r] * a_s + xo[(t * 16 + r) * 64 + lane] * a_p) * inv);
                }
                *reinterpret_cast<bf16x4*>(orow + 32 * t + 8 * g + 4 * h) = pk;
            }
    }
}

template <int D, bool RASTER, bool WEIGHTED>
hipError_t launch(const AttnArgs& a, hipStream_t s) {
    const float scale_log2e = a.scale * 1.4426950408889634f;
    RasterGrid grid{};
    if (RASTER) {
        grid.W = (uint32_t)a.W;
        grid.HW = (uint32_t)(a.H * a.W);
        grid.nHW = FastDiv((uint32_t)((a.H / 8) * (a.W / 8)));
        grid.nW = FastDiv((uint32_t)(a.W / 8));
    }
    hipLaunchKernelGGL((attn_fwd_bf16_kernel<D, RASTER, WEIGHTED>), dim3(a.BH * a.nb), dim3(kThreads), 0, s,
                       (const __bf16*)a.q, (const __bf16*)a.k, (const __bf16*)a.v, (__bf16*)a.o,
                       a.L, a.nb, a.kv_count, a.kv_index, a.schedule, grid, scale_log2e, a.lse, a.kv_logw);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_attn_bf16(const AttnArgs& a, hipStream_t s) {
    if (a.kv_logw) return a.d == 128 ? launch<128, false, true>(a, s) : launch<64, false, true>(a, s);
    if (a.raster) return a.d == 128 ? launch<128, true, false>(a, s) : launch<64, true, false>(a, s);
    return a.d == 128 ? launch<128, false, false>(a, s) : launch<64, false, false>(a, s);
}

}  // namespace nabla
