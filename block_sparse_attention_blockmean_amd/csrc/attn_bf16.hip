// Block-sparse flash attention, bf16 in / bf16 out, for 64-token blocks.
//
// Computes softmax attention only on the kept 64 x 64 tiles (NABLA technical summary,
// "Metodologia: NABLA", item 2, "Expansão"); a dropped tile contributes neither to the
// numerator nor to the normaliser.
//
// One workgroup = one 64-row query block, two waves of 32 query rows each.  Per kept
// KV block, each wave runs
//     S^T = K Q^T      v_mfma_f32_32x32x16_bf16, A = K from LDS, B = Q from VGPRs
//     online softmax   float32, exp2 with scale*log2(e) folded into one FMA
//     O^T += V^T P^T   v_mfma_f32_32x32x16_bf16, A = V^T from LDS, B = P from VGPRs
// Computing the transposed products makes every lane own one query column: its S^T
// accumulator already has the layout the P operand of the second product needs (the
// MFMA's k index is permuted identically in both operands, which leaves the sum
// unchanged), and the row statistics stay in the lane, with one exchange between
// lanes l and l^32, which split the 64 keys of a tile.
//
// Memory pipeline: K and V tiles go from global memory straight into LDS
// (global_load_lds_dwordx4, no VGPR staging), row-major with an XOR swizzle of the
// 16-byte chunks.  V^T operands come out of the row-major V tile through the
// transposing LDS read (ds_read_b64_tr_b16).  One K and one V buffer (32 KiB per
// workgroup, so four workgroups = two waves per SIMD fit a CU): K of the next tile
// streams in during the softmax and P V, right after every wave has read the current
// K, and V of the next tile during the next S^T and softmax.  Barriers between waves
// are plain s_barrier with explicit waits, so copies stay in flight across them.
#include <math.h>

#include "nabla_internal.h"

namespace nabla {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef __attribute__((address_space(3))) void lds_void;
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;

constexpr int kBlk = 64;
constexpr int kThreads = 128;

template <int D>
struct Tile {
    static constexpr int kRowBytes = 2 * D;             // one token row of K or V
    static constexpr int kChunks = D / 8;               // 16-byte chunks per row
    static constexpr int kRowsPerLine = 256 / kRowBytes;  // rows per 256-byte LDS bank line
    static constexpr int kBytes = kBlk * kRowBytes;
    static constexpr int kLoadsPerWave = kBytes / 1024 / 2;  // 1 KB per wave-wide load
    // K is read 16 bytes per lane from 16 consecutive rows at one chunk: spread the
    // rows over all chunk slots of a bank line.
    __device__ static inline int k_swz(int row) { return (row / kRowsPerLine) & (kChunks - 1); }
    // V is read 8 bytes per lane, 4 rows x 64 bytes per 16 lanes: spread groups of
    // 4 chunks over the bank line.
    __device__ static inline int v_swz(int row) { return 4 * ((row / kRowsPerLine) & (kChunks / 4 - 1)); }
};

// Wave-wide copy of one 64 x D tile from global memory into LDS.  Load u of wave w
// fills bytes [1024 (2u + w), +1024) of the LDS tile, 16 bytes per lane in lane order;
// the lane picks the global chunk that belongs in that slot under the swizzle.  The
// tile base is uniform and the lane offset 32-bit, so the load takes the scalar-base
// form; the LDS destination (M0) is uniform as well.
template <int D, bool kIsV>
__device__ inline uint32_t tile_lane_offset(int u, int wave, int lane) {
    using G = Tile<D>;
    const int o = (2 * u + wave) * 1024 + lane * 16;
    const int row = o / G::kRowBytes;
    const int slot = (o % G::kRowBytes) / 16;
    const int chunk = slot ^ (kIsV ? G::v_swz(row) : G::k_swz(row));
    return (uint32_t)(row * G::kRowBytes + chunk * 16);
}

template <int D, bool kIsV>
__device__ inline void load_tile(const __bf16* g_tile, char* lds_tile, int wave, int lane) {
    using G = Tile<D>;
    const char* src = reinterpret_cast<const char*>(g_tile);
#pragma unroll
    for (int u = 0; u < G::kLoadsPerWave; ++u) {
        uint32_t off = tile_lane_offset<D, kIsV>(u, wave, lane);
        // keep the offset a 32-bit register at the load, so it is not widened to a
        // 64-bit pointer and hoisted out of the tile loop
        asm volatile("" : "+v"(off));
        __builtin_amdgcn_global_load_lds(src + off, (lds_void*)(lds_tile + (2 * u + wave) * 1024),
                                         16, 0, 0);
    }
}

template <int N>
__device__ inline void wait_vmcnt() {
    asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

// Workgroup barrier for LDS hand-offs that leaves tile copies in flight.  A
// __syncthreads() is a fenced barrier and drains every outstanding vector-memory
// operation first, which would cancel the prefetch; here only this wave's LDS reads
// are completed (lgkmcnt), and every place that needs a copy to have landed waits for
// it explicitly with wait_vmcnt before the barrier.  The memory clobber keeps the
// compiler from moving memory accesses across it.
__device__ inline void lds_barrier() {
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

template <int D>
__global__ __launch_bounds__(kThreads, 2) void attn_fwd_bf16_kernel(
    const __bf16* __restrict__ q, const __bf16* __restrict__ k, const __bf16* __restrict__ v,
    __bf16* __restrict__ o, int L, int nb, const int32_t* __restrict__ kv_count,
    const int32_t* __restrict__ kv_index, const int32_t* __restrict__ schedule,
    float scale_log2e) {
    using G = Tile<D>;
    constexpr int KS = D / 16;        // k-steps of S^T = K Q^T
    constexpr int DT = D / 32;        // 32-row d tiles of O^T
    __shared__ __attribute__((aligned(1024))) char k_lds[G::kBytes];
    __shared__ __attribute__((aligned(1024))) char v_lds[G::kBytes];

    // Workgroups are dealt round-robin to the 8 XCDs; remap so that each XCD walks a
    // contiguous range of (head, query block) and neighbouring query blocks, which
    // keep similar KV lists, share that XCD's L2.
    // With a schedule, workgroups take query blocks in its order (longest lists first).
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
    const int lane = tid & 63;
    const int h = lane >> 5;
    const int c32 = lane & 31;

    const size_t head_off = (size_t)bh * L * D;
    const __bf16* qh = q + head_off;
    const __bf16* kh = k + head_off;
    const __bf16* vh = v + head_off;

    const int count = kv_count[(size_t)bh * nb + qb];
    const int32_t* list = kv_index + ((size_t)bh * nb + qb) * nb;
    // Q operand: lane holds Q[row][16 s + 8 h .. + 7] for s = 0..KS-1.
    const int qrow = qb * kBlk + wave * 32 + c32;
    bf16x8 qreg[KS];
#pragma unroll
    for (int s = 0; s < KS; ++s)
        qreg[s] = *reinterpret_cast<const bf16x8*>(qh + (size_t)qrow * D + 16 * s + 8 * h);

    // issue order K0, V0; iteration i issues K(i+1) after its S^T and V(i+1) at its end
    if (count > 0) {
        load_tile<D, false>(kh + (size_t)list[0] * kBlk * D, k_lds, wave, lane);
        load_tile<D, true>(vh + (size_t)list[0] * kBlk * D, v_lds, wave, lane);
    }

    f32x16 oacc[DT];
#pragma unroll
    for (int t = 0; t < DT; ++t)
#pragma unroll
        for (int r = 0; r < 16; ++r) oacc[t][r] = 0.f;
    float m_run = -INFINITY;   // reference max of scaled logits (log2 domain)
    float l_run = 0.f;         // this lane's share of the running normaliser

    // per-lane LDS byte offsets that do not change from tile to tile
    int k_off[2][KS];
#pragma unroll
    for (int t = 0; t < 2; ++t) {
        const int row = 32 * t + c32;
#pragma unroll
        for (int s = 0; s < KS; ++s)
            k_off[t][s] = row * G::kRowBytes + (((2 * s + h) ^ G::k_swz(row)) * 16);
    }
    const int g16 = lane >> 4, j16 = lane & 15;
    int v_off[DT][4][2];
#pragma unroll
    for (int t = 0; t < DT; ++t)
#pragma unroll
        for (int u = 0; u < 4; ++u)
#pragma unroll
            for (int p = 0; p < 2; ++p) {
                const int row = 16 * u + 4 * h + 8 * p + (j16 >> 2);
                const int d = 32 * t + 16 * (g16 & 1) + 4 * (j16 & 3);
                v_off[t][u][p] = row * G::kRowBytes + (((d >> 3) ^ G::v_swz(row)) * 16) + ((d >> 2) & 1) * 8;
            }

    // K0 has landed once only V0 may be pending
    wait_vmcnt<G::kLoadsPerWave>();
    lds_barrier();

    for (int it = 0; it < count; ++it) {
        // K(it) is in LDS and visible: every wave waited for it (in the prologue or at
        // the end of the previous iteration) before a barrier
        const char* kbuf = k_lds;

        // ---- S^T = K Q^T for this wave's 32 query columns, 64 keys in two 32-key tiles.
        // Operands are requested a quarter tile ahead: a group of reads, then the
        // MFMAs that use them while the next group lands.
        constexpr int KG = KS / 4;   // k-steps per group
        f32x16 sacc[2];
#pragma unroll
        for (int t = 0; t < 2; ++t)
#pragma unroll
            for (int r = 0; r < 16; ++r) sacc[t][r] = 0.f;
#pragma unroll
        for (int grp = 0; grp < 4; ++grp) {
            bf16x8 ka[KG][2];
#pragma unroll
            for (int s = 0; s < KG; ++s)
#pragma unroll
                for (int t = 0; t < 2; ++t)
                    ka[s][t] = *reinterpret_cast<const bf16x8*>(kbuf + k_off[t][grp * KG + s]);
#pragma unroll
            for (int s = 0; s < KG; ++s)
#pragma unroll
                for (int t = 0; t < 2; ++t)
                    sacc[t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka[s][t], qreg[grp * KG + s],
                                                                      sacc[t], 0, 0, 0);
            __builtin_amdgcn_sched_group_barrier(0x100, 2 * KG, 0);   // this group's K reads
            __builtin_amdgcn_sched_group_barrier(0x008, 2 * KG, 0);   // then its MFMAs
        }

        // every wave is done with k_lds: stream in the next K during the softmax and P V
        lds_barrier();
        const bool more = it + 1 < count;
        if (more) load_tile<D, false>(kh + (size_t)list[it + 1] * kBlk * D, k_lds, wave, lane);

        // ---- online softmax for query column c32 (keys split between lanes l, l^32).
        // The reference maximum m_run only moves when a tile's maximum exceeds it by
        // more than 8 (log2 units), so P stays below 2^8 and the rescale of O and l is
        // rare; normalising by l at the end makes the result independent of m_run.
        float mx = -INFINITY;
#pragma unroll
        for (int t = 0; t < 2; ++t)
#pragma unroll
            for (int r = 0; r < 16; ++r) mx = fmaxf(mx, sacc[t][r]);
        mx = fmaxf(mx, __shfl_xor(mx, 32)) * scale_log2e;
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

        // V(it) has landed once at most K(it+1), issued after it, is pending
        if (more) wait_vmcnt<G::kLoadsPerWave>(); else wait_vmcnt<0>();
        lds_barrier();

        // ---- O^T += V^T P^T, k-step by k-step: P of step u needs only its own 8 exps,
        // and the V^T operands (two transposing 8-byte reads each) of step u+1 are
        // requested while step u multiplies.
        s16x4 vr[2][DT][2];
#pragma unroll
        for (int t = 0; t < DT; ++t)
#pragma unroll
            for (int p = 0; p < 2; ++p)
                vr[0][t][p] = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(v_lds + v_off[t][0][p]));
        float psum = 0.f;
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            if (u + 1 < 4) {
#pragma unroll
                for (int t = 0; t < DT; ++t)
#pragma unroll
                    for (int p = 0; p < 2; ++p)
                        vr[(u + 1) & 1][t][p] =
                            __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(v_lds + v_off[t][u + 1][p]));
            }
            bf16x8 pb;
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const float pe = __builtin_amdgcn_exp2f(fmaf(sacc[u >> 1][8 * (u & 1) + e], scale_log2e, -m_run));
                psum += pe;
                pb[e] = (__bf16)pe;
            }
#pragma unroll
            for (int t = 0; t < DT; ++t) {
                const bf16x8 a = __builtin_bit_cast(
                    bf16x8, __builtin_shufflevector(vr[u & 1][t][0], vr[u & 1][t][1], 0, 1, 2, 3, 4, 5, 6, 7));
                oacc[t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, pb, oacc[t], 0, 0, 0);
            }
        }
        l_run += psum;
        // K(it+1) has landed (nothing was issued after it); after the barrier every
        // wave is done with v_lds and sees K(it+1): stream in the next V
        if (more) wait_vmcnt<0>();
        lds_barrier();
        if (more) load_tile<D, true>(vh + (size_t)list[it + 1] * kBlk * D, v_lds, wave, lane);
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
                       a.L, a.nb, a.kv_count, a.kv_index, a.schedule, scale_log2e);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_attn_bf16(const AttnArgs& a, hipStream_t s) {
    return a.d == 128 ? launch<128>(a, s) : launch<64>(a, s);
}

}  // namespace nabla
