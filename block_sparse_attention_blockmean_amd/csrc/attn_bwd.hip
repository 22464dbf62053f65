// Gradient of block-sparse attention for 64-token blocks: dQ, dK, dV of sum(O * dO)
// where O is the attention over the kept 64 x 64 tiles (NABLA technical summary,
// "Metodologia: NABLA", item 2, "Expansão"; a dropped tile is in neither the numerator
// nor the normaliser, so it passes no gradient either).  With P the kept-tile softmax,
// recomputed from the log-sum-exp the forward saved:
//     D_a  = sum_c dO_ac O_ac                           (row dot)
//     dV_t = sum_a P_at dO_a,   dP_at = dO_a . v_t,   dS_at = P_at (dP_at - D_a)
//     dQ_a = scale sum_t dS_at k_t,   dK_t = scale sum_a dS_at q_a
// dQ walks each query block's KV list; dK and dV walk, for each KV block, the list of
// query blocks that keep it (the transpose of the lists, built here through a bitmap).
// Both sweeps recompute S and dP, so no partial sums are shared between workgroups and
// the result does not depend on the order the workgroups run in.
//
// bf16: MFMA v_mfma_f32_32x32x16_bf16 with float32 accumulation; P and dS are rounded
// to bf16 as MFMA operands; gradients are written in bf16.  float32: plain FMAs.
//
// Token order: every kernel takes the blocks either as runs of 64 rows (fractal order)
// or, with RASTER, as 8 x 8 patches of a raster T x H x W grid (the fractal reorder of
// the NABLA summary, "Metodologia: NABLA", item 1, folded into the addressing: a patch
// is eight runs of eight consecutive tokens).  Lists number blocks the same way in both;
// the arithmetic, and so every result bit, is the same.
#include <math.h>

#include <algorithm>
#include <type_traits>

#include "attn_tile.h"
#include "nabla_internal.h"

namespace nabla {
namespace {

using namespace attn;

constexpr float kLog2e = 1.4426950408889634f;

// Workgroup -> logical item: the schedule's order when given, otherwise each XCD
// (workgroups are dealt round-robin to the 8 XCDs) walks a contiguous range.
__device__ inline int logical_item(const int32_t* schedule) {
    const int nwg = gridDim.x;
    const int full = (nwg / 8) * 8;
    const int w = blockIdx.x;
    if (schedule) return schedule[w];
    return w < full ? (w % 8) * (nwg / 8) + w / 8 : w;
}

// ---------------------------------------------------------------------------
// D = rowsum(dO * O) in float32, one group of 16-byte lanes per row.
// ---------------------------------------------------------------------------
template <typename T, int D>
__global__ __launch_bounds__(256) void bwd_rowdot_kernel(const T* __restrict__ o, const T* __restrict__ dout,
                                                         float* __restrict__ drow, long long rows) {
    constexpr int kElems = 16 / (int)sizeof(T);   // elements per 16-byte chunk
    constexpr int kLanes = D / kElems;            // lanes per row: 8, 16 or 32
    constexpr int kRows = 256 / kLanes;
    typedef T vec __attribute__((ext_vector_type(kElems)));
    const int tid = threadIdx.x;
    const long long row = (long long)blockIdx.x * kRows + tid / kLanes;
    const int part = tid % kLanes;
    float acc = 0.f;
    if (row < rows) {
        const vec a = *reinterpret_cast<const vec*>(o + row * D + part * kElems);
        const vec b = *reinterpret_cast<const vec*>(dout + row * D + part * kElems);
#pragma unroll
        for (int e = 0; e < kElems; ++e) acc = fmaf((float)a[e], (float)b[e], acc);
    }
#pragma unroll
    for (int off = kLanes / 2; off > 0; off >>= 1) acc += __shfl_xor(acc, off);
    if (row < rows && part == 0) drow[row] = acc;
}

// ---------------------------------------------------------------------------
// Transposed lists: bits[bh][j] has bit i set when query block i keeps KV block j;
// each row is then expanded into the ascending list of those i.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void bwd_zero_kernel(uint32_t* __restrict__ p, long long n) {
    for (long long i = (long long)blockIdx.x * 256 + threadIdx.x; i < n; i += (long long)gridDim.x * 256) p[i] = 0u;
}

__global__ __launch_bounds__(256) void bwd_scatter_kernel(const int32_t* __restrict__ kv_count,
                                                          const int32_t* __restrict__ kv_index, int nb, int words,
                                                          uint32_t* __restrict__ bits) {
    const int row = blockIdx.x;   // bh * nb + i
    const int bh = row / nb;
    const int i = row - bh * nb;
    const int cnt = min(max(kv_count[row], 0), nb);
    const int32_t* list = kv_index + (size_t)row * nb;
    for (int e = threadIdx.x; e < cnt; e += 256) {
        const int j = list[e];
        if (j >= 0 && j < nb) atomicOr(&bits[((size_t)bh * nb + j) * words + (i >> 5)], 1u << (i & 31));
    }
}

__global__ __launch_bounds__(64) void bwd_qlist_kernel(const uint32_t* __restrict__ bits, int nb, int words,
                                                       int32_t* __restrict__ q_count, int32_t* __restrict__ q_index) {
    const int row = blockIdx.x;   // bh * nb + j
    const int lane = threadIdx.x;
    uint32_t w = lane < words ? bits[(size_t)row * words + lane] : 0u;
    const int n = __popc(w);
    int incl = n;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
        const int y = __shfl_up(incl, off);
        if (lane >= off) incl += y;
    }
    int pos = incl - n;
    int32_t* out = q_index + (size_t)row * nb;
    while (w) {
        out[pos++] = lane * 32 + __ffs(w) - 1;
        w &= w - 1;
    }
    if (lane == 63) q_count[row] = incl;
}

// ---------------------------------------------------------------------------
// dQ, bf16.  One workgroup per query block, four waves: wave (qh, kh) takes query rows
// [32 qh, +32) against keys [32 kh, +32) of every kept tile.  Transposed products, so
// that each lane owns one query column and its log-sum-exp and D stay in the lane:
//     S^T  = K Q^T     A = K rows (LDS),  B = Q (VGPRs)
//     dP^T = V dO^T    A = V rows (LDS),  B = dO (VGPRs)
//     dS^T = P^T (dP^T - D),  P^T = exp2(S^T scale log2(e) - lse log2(e))
//     dQ^T += K^T dS^T A = K^T through the transposing LDS read, B = dS^T (VGPRs)
// K and V tiles are double-buffered through the LDS DMA, both with the row-read
// swizzle.  The two key halves are summed through LDS at the end.
// ---------------------------------------------------------------------------
template <int D, bool RASTER>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(2, 2)))
void bwd_dq_bf16_kernel(const __bf16* __restrict__ q, const __bf16* __restrict__ k, const __bf16* __restrict__ v,
                        const __bf16* __restrict__ dout, const float* __restrict__ lse,
                        const float* __restrict__ drow, __bf16* __restrict__ dq, int L, int nb,
                        const int32_t* __restrict__ kv_count, const int32_t* __restrict__ kv_index,
                        const int32_t* __restrict__ schedule, RasterGrid grid, float scale_log2e, float scale) {
    using G = Tile<D>;
    constexpr int KS = D / 16;
    constexpr int DT = D / 32;
    __shared__ __attribute__((aligned(1024))) char k_lds0[G::kBytes];
    __shared__ __attribute__((aligned(1024))) char k_lds1[G::kBytes];
    __shared__ __attribute__((aligned(1024))) char v_lds0[G::kBytes];
    __shared__ __attribute__((aligned(1024))) char v_lds1[G::kBytes];

    const int logical = logical_item(schedule);
    const int bh = logical / nb;
    const int qb = logical - bh * nb;
    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int qhalf = wave & 1;
    const int khalf = wave >> 1;
    const int lane = tid & 63;
    const int h = lane >> 5;
    const int c32 = lane & 31;
    const int g16 = lane >> 4, j16 = lane & 15;

    const size_t head_off = (size_t)bh * L * D;
    const int head_bytes = L * D * 2;
    const __amdgpu_buffer_rsrc_t k_rsrc =
        __builtin_amdgcn_make_buffer_rsrc((void*)(k + head_off), 0, head_bytes, kBufferFlags);
    const __amdgpu_buffer_rsrc_t v_rsrc =
        __builtin_amdgcn_make_buffer_rsrc((void*)(v + head_off), 0, head_bytes, kBufferFlags);
    const uint32_t lane_copy = copy_lane_offset_in<D, false, RASTER>(grid, wave, lane);
    const uint32_t stride = copy_stride<RASTER>(grid);   // between a tile's 4 KiB copies

    const int count = kv_count[(size_t)bh * nb + qb];
    const int32_t* list = kv_index + ((size_t)bh * nb + qb) * nb;
    if (count > 0) {
        const uint32_t first = block_row<RASTER>(grid, list[0]) * G::kRowBytes;
        copy_tile<D>(k_rsrc, first, k_lds0, wave, lane_copy, stride);
        copy_tile<D>(v_rsrc, first, v_lds0, wave, lane_copy, stride);
    }

    const int qrow = block_row<RASTER>(grid, qb) + row_in_block<RASTER>(grid, 32 * qhalf + c32);
    bf16x8 qreg[KS], doreg[KS];
#pragma unroll
    for (int s = 0; s < KS; ++s) {
        qreg[s] = *reinterpret_cast<const bf16x8*>(q + head_off + (size_t)qrow * D + 16 * s + 8 * h);
        doreg[s] = *reinterpret_cast<const bf16x8*>(dout + head_off + (size_t)qrow * D + 16 * s + 8 * h);
    }
    const float lse2 = count > 0 ? lse[(size_t)bh * L + qrow] * kLog2e : 0.f;
    const float dd = drow[(size_t)bh * L + qrow];

    f32x16 dqacc[DT];
#pragma unroll
    for (int t = 0; t < DT; ++t)
#pragma unroll
        for (int r = 0; r < 16; ++r) dqacc[t][r] = 0.f;

    const int krow = 32 * khalf + c32;
    int k_off[KS];
#pragma unroll
    for (int s = 0; s < KS; ++s) k_off[s] = krow * G::kRowBytes + (((2 * s + h) ^ G::k_swz(krow)) * 16);
    // K^T operand of d tile t, k-step u, half p: rows 32 kh + 16 u + 8 p + 4 h + j16 / 4.
    // The row swizzle repeats every 16 rows, so u is a constant offset but p is not.
    int t_off[DT][2];
#pragma unroll
    for (int t = 0; t < DT; ++t)
#pragma unroll
        for (int p = 0; p < 2; ++p) {
            const int row = 32 * khalf + 8 * p + 4 * h + (j16 >> 2);
            const int d = 32 * t + 16 * (g16 & 1) + 4 * (j16 & 3);
            t_off[t][p] = row * G::kRowBytes + (((d >> 3) ^ G::k_swz(row)) * 16) + ((d >> 2) & 1) * 8;
        }

    int next_tile = list[count > 1 ? 1 : 0];
    auto step = [&](auto par, int i) {
        constexpr int PAR = decltype(par)::value;
        const char* kbuf = PAR ? k_lds1 : k_lds0;
        const char* vbuf = PAR ? v_lds1 : v_lds0;
        // tile i has landed; after the barrier every wave is done with tile i - 1
        wait_vmcnt<0>();
        lds_barrier();
        const uint32_t nxt = block_row<RASTER>(grid, next_tile) * G::kRowBytes;
        char* k_dst = PAR ? k_lds0 : k_lds1;
        char* v_dst = PAR ? v_lds0 : v_lds1;
        constexpr int kEvery = KS / G::kCopiesPerWave;

        f32x16 sacc, dpacc;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            sacc[r] = 0.f;
            dpacc[r] = 0.f;
        }
        bf16x8 ka[KS], va[KS];
#pragma unroll
        for (int s = 0; s < KS; ++s) ka[s] = *reinterpret_cast<const bf16x8*>(kbuf + k_off[s]);
#pragma unroll
        for (int s = 0; s < KS; ++s) va[s] = *reinterpret_cast<const bf16x8*>(vbuf + k_off[s]);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int s = 0; s < KS; ++s) {
            sacc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka[s], qreg[s], sacc, 0, 0, 0);
            if (s % kEvery == 0)
                __builtin_amdgcn_raw_ptr_buffer_load_lds(k_rsrc, (lds_void*)(k_dst + (kWaves * (s / kEvery) + wave) * 1024),
                                                         16, lane_copy, nxt + (s / kEvery) * stride, 0, 0);
            __builtin_amdgcn_sched_barrier(0);
        }
#pragma unroll
        for (int s = 0; s < KS; ++s) {
            dpacc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va[s], doreg[s], dpacc, 0, 0, 0);
            if (s % kEvery == 0)
                __builtin_amdgcn_raw_ptr_buffer_load_lds(v_rsrc, (lds_void*)(v_dst + (kWaves * (s / kEvery) + wave) * 1024),
                                                         16, lane_copy, nxt + (s / kEvery) * stride, 0, 0);
            __builtin_amdgcn_sched_barrier(0);
        }

        bf16x8 dsb[2];
#pragma unroll
        for (int u = 0; u < 2; ++u)
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const int r = 8 * u + e;
                const float p = __builtin_amdgcn_exp2f(fmaf(sacc[r], scale_log2e, -lse2));
                dsb[u][e] = (__bf16)(p * (dpacc[r] - dd));
            }
#pragma unroll
        for (int u = 0; u < 2; ++u)
#pragma unroll
            for (int t = 0; t < DT; ++t) {
                const s16x4 a0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                    (lds_s16x4*)(kbuf + t_off[t][0] + (16 * u) * G::kRowBytes));
                const s16x4 a1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                    (lds_s16x4*)(kbuf + t_off[t][1] + (16 * u) * G::kRowBytes));
                const bf16x8 a = __builtin_bit_cast(bf16x8, __builtin_shufflevector(a0, a1, 0, 1, 2, 3, 4, 5, 6, 7));
                dqacc[t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, dsb[u], dqacc[t], 0, 0, 0);
            }
        __builtin_amdgcn_sched_barrier(0);
        next_tile = list[min(i + 2, count - 1)];
    };

    using P0 = std::integral_constant<int, 0>;
    using P1 = std::integral_constant<int, 1>;
    for (int i = 0; i < count; i += 2) {
        step(P0{}, i);
        if (i + 1 < count) step(P1{}, i + 1);
    }

    // sum the key halves: wave (qh, 1) hands its partial dQ^T to wave (qh, 0)
    wait_vmcnt<0>();
    lds_barrier();
    float* xo = reinterpret_cast<float*>(qhalf ? k_lds1 : k_lds0);
    static_assert(DT * 16 * 64 * 4 <= G::kBytes, "partial dQ exceeds one tile buffer");
    if (khalf == 1) {
#pragma unroll
        for (int t = 0; t < DT; ++t)
#pragma unroll
            for (int r = 0; r < 16; ++r) xo[(t * 16 + r) * 64 + lane] = dqacc[t][r];
    }
    lds_barrier();
    if (khalf == 0) {
        __bf16* orow = dq + head_off + (size_t)qrow * D;
#pragma unroll
        for (int t = 0; t < DT; ++t)
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                bf16x4 pk;
#pragma unroll
                for (int c = 0; c < 4; ++c) {
                    const int r = 4 * g + c;
                    pk[c] = (__bf16)((dqacc[t][r] + xo[(t * 16 + r) * 64 + lane]) * scale);
                }
                *reinterpret_cast<bf16x4*>(orow + 32 * t + 8 * g + 4 * h) = pk;
            }
    }
}

// ---------------------------------------------------------------------------
// dK, dV, bf16.  One workgroup per KV block, four waves: wave (kh, qh) takes keys
// [32 kh, +32) against query rows [32 qh, +32) of every query block that keeps the KV
// block.  Plain products, so that each lane owns one key column:
//     S  = Q K^T       A = Q rows (LDS),   B = K rows (LDS, resident)
//     dP = dO V^T      A = dO rows (LDS),  B = V rows (LDS, resident)
//     P = exp2(S scale log2(e) - lse log2(e)),  dS = P (dP - D)   (per query row)
//     dV^T += dO^T P   A = dO^T through the transposing LDS read, B = P (VGPRs)
// then, after a barrier that frees the dO tile for the next query block's copy,
//     dK^T += Q^T dS   A = Q^T through the transposing LDS read, B = dS (VGPRs)
// K and V stay in LDS for the whole sweep.  Q is double-buffered (the next query
// block's Q is copied at the top of an iteration); dO has one buffer, refilled once
// every wave has formed its dP.  16 + 16 + 2 x 16 + 16 KiB = 80 KiB of LDS at d = 128:
// two workgroups fill a CU's 160 KiB, with no room for a buffer of the row statistics,
// which are loaded into registers.  Vector-memory waits count in issue order, so the
// order of issue decides what each wait covers: per query block the statistics loads
// go out first, then the next Q copy, and the next dO copy last.  A wait for the
// statistics then never waits for a copy, the block's dO copy has S and P to land
// behind, and the next Q copy has the whole block.  The two query halves are summed
// through LDS at the end.
// ---------------------------------------------------------------------------
template <int D, bool RASTER>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(2, 2)))
void bwd_dkdv_bf16_kernel(const __bf16* __restrict__ q, const __bf16* __restrict__ k, const __bf16* __restrict__ v,
                          const __bf16* __restrict__ dout, const float* __restrict__ lse,
                          const float* __restrict__ drow, __bf16* __restrict__ dk, __bf16* __restrict__ dv, int L,
                          int nb, const int32_t* __restrict__ q_count, const int32_t* __restrict__ q_index,
                          const int32_t* __restrict__ schedule, RasterGrid grid, float scale_log2e, float scale) {
    using G = Tile<D>;
    constexpr int KS = D / 16;
    constexpr int DT = D / 32;
    // vector-memory operations a wave issues per query block, in issue order: the row
    // statistics (two groups of four 16-byte loads), the next Q copy, the next dO copy
    constexpr int kStatLoads = 8;
    constexpr int kQCopies = G::kCopiesPerWave;
    constexpr int kDoCopies = G::kCopiesPerWave;
    __shared__ __attribute__((aligned(1024))) char k_t[G::kBytes];
    __shared__ __attribute__((aligned(1024))) char v_t[G::kBytes];
    __shared__ __attribute__((aligned(1024))) char q_t0[G::kBytes];
    __shared__ __attribute__((aligned(1024))) char q_t1[G::kBytes];
    __shared__ __attribute__((aligned(1024))) char do_t[G::kBytes];

    const int logical = logical_item(schedule);
    const int bh = logical / nb;
    const int kb = logical - bh * nb;
    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int khalf = wave & 1;
    const int qhalf = wave >> 1;
    const int lane = tid & 63;
    const int h = lane >> 5;
    const int c32 = lane & 31;
    const int g16 = lane >> 4, j16 = lane & 15;

    const size_t head_off = (size_t)bh * L * D;
    const int head_bytes = L * D * 2;
    const __amdgpu_buffer_rsrc_t q_rsrc =
        __builtin_amdgcn_make_buffer_rsrc((void*)(q + head_off), 0, head_bytes, kBufferFlags);
    const __amdgpu_buffer_rsrc_t k_rsrc =
        __builtin_amdgcn_make_buffer_rsrc((void*)(k + head_off), 0, head_bytes, kBufferFlags);
    const __amdgpu_buffer_rsrc_t v_rsrc =
        __builtin_amdgcn_make_buffer_rsrc((void*)(v + head_off), 0, head_bytes, kBufferFlags);
    const __amdgpu_buffer_rsrc_t do_rsrc =
        __builtin_amdgcn_make_buffer_rsrc((void*)(dout + head_off), 0, head_bytes, kBufferFlags);
    const uint32_t lane_copy = copy_lane_offset_in<D, false, RASTER>(grid, wave, lane);
    const uint32_t stride = copy_stride<RASTER>(grid);   // between a tile's 4 KiB copies

    const int count = q_count[(size_t)bh * nb + kb];
    const int32_t* list = q_index + ((size_t)bh * nb + kb) * nb;
    const uint32_t kv_first = block_row<RASTER>(grid, kb);
    copy_tile<D>(k_rsrc, kv_first * G::kRowBytes, k_t, wave, lane_copy, stride);
    copy_tile<D>(v_rsrc, kv_first * G::kRowBytes, v_t, wave, lane_copy, stride);
    if (count > 0) {
        const uint32_t first = block_row<RASTER>(grid, list[0]) * G::kRowBytes;
        copy_tile<D>(q_rsrc, first, q_t0, wave, lane_copy, stride);
        copy_tile<D>(do_rsrc, first, do_t, wave, lane_copy, stride);
    }

    f32x16 dvacc[DT], dkacc[DT];
#pragma unroll
    for (int t = 0; t < DT; ++t)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            dvacc[t][r] = 0.f;
            dkacc[t][r] = 0.f;
        }

    // A rows (queries) of the Q / dO tiles and B rows (keys) of the K / V tiles.  The
    // two rows differ by a multiple of 32, over which the row swizzle repeats, so the B
    // offsets are the A offsets plus one wave-uniform constant.
    const int arow = 32 * qhalf + c32;
    const int brow = 32 * khalf + c32;
    const int b_shift = (brow - arow) * G::kRowBytes;
    static_assert(32 % (G::kRowsPerLine * G::kChunks) == 0, "row swizzle period must divide 32");
    int a_off[KS];
#pragma unroll
    for (int s = 0; s < KS; ++s) a_off[s] = arow * G::kRowBytes + (((2 * s + h) ^ G::k_swz(arow)) * 16);
    // dO^T / Q^T operand of d tile t, k-step u, half p: rows 32 qh + 16 u + 8 p + 4 h + j16 / 4
    // (the row swizzle repeats every 16 rows: u is a constant offset, p is not)
    int t_off[DT][2];
#pragma unroll
    for (int t = 0; t < DT; ++t)
#pragma unroll
        for (int p = 0; p < 2; ++p) {
            const int row = 32 * qhalf + 8 * p + 4 * h + (j16 >> 2);
            const int d = 32 * t + 16 * (g16 & 1) + 4 * (j16 & 3);
            t_off[t][p] = row * G::kRowBytes + (((d >> 3) ^ G::k_swz(row)) * 16) + ((d >> 2) & 1) * 8;
        }
    // the lane's 16 query rows of a block: 32 qh + 8 g + 4 h + c for accumulator entry 4 g + c,
    // four consecutive rows per g in either order (a raster patch row holds 8), g's rows
    // stat_g rows after g - 1's
    const size_t stat_off = (size_t)bh * L + row_in_block<RASTER>(grid, 32 * qhalf + 4 * h);
    const uint32_t stat_g = RASTER ? grid.W : 8u;

    auto step = [&](auto par, int i) {
        constexpr int PAR = decltype(par)::value;
        const char* qbuf = PAR ? q_t1 : q_t0;
        char* q_next = PAR ? q_t0 : q_t1;
        const int qblk = list[i];
        // Q of query block qblk has landed (only its dO copy, the last one issued, may
        // still be in flight), and every wave is done with the previous block
        wait_vmcnt<kDoCopies>();
        lds_barrier();
        // the row statistics first, then the next block's Q into the other buffer: a
        // wait for the statistics never waits for that copy.  The copy is unconditional
        // (the last block copies its own Q again into a buffer nothing reads), so the
        // compiler's waits stay exact.
        const size_t qrow0 = block_row<RASTER>(grid, qblk);
        float4 ls[4], dr[4];
#pragma unroll
        for (int g = 0; g < 4; ++g)
            ls[g] = *reinterpret_cast<const float4*>(lse + stat_off + qrow0 + g * stat_g);
#pragma unroll
        for (int g = 0; g < 4; ++g)
            dr[g] = *reinterpret_cast<const float4*>(drow + stat_off + qrow0 + g * stat_g);
        const uint32_t nxt = block_row<RASTER>(grid, list[min(i + 1, count - 1)]) * G::kRowBytes;
        __builtin_amdgcn_sched_barrier(0);
        copy_tile<D>(q_rsrc, nxt, q_next, wave, lane_copy, stride);
        __builtin_amdgcn_sched_barrier(0);

        // S, then P (the log-sum-exp and S die here)
        f32x16 sacc;
#pragma unroll
        for (int r = 0; r < 16; ++r) sacc[r] = 0.f;
#pragma unroll
        for (int s = 0; s < KS; ++s) {
            const bf16x8 a = *reinterpret_cast<const bf16x8*>(qbuf + a_off[s]);
            const bf16x8 b = *reinterpret_cast<const bf16x8*>(k_t + b_shift + a_off[s]);
            sacc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, sacc, 0, 0, 0);
        }
        // the products are issued before the wait for the statistics (and, behind them
        // in issue order, this block's dO copy)
        __builtin_amdgcn_sched_barrier(0);
        float p[16];
        bf16x8 pb[2], dsb[2];
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const float l2 = ls[r / 4][r % 4] * kLog2e;
            p[r] = __builtin_amdgcn_exp2f(fmaf(sacc[r], scale_log2e, -l2));
            pb[r / 8][r % 8] = (__bf16)p[r];
        }
        // dO of qblk: this wave's share landed (only the statistics loads and the Q
        // copy were issued after it), then every wave's
        __builtin_amdgcn_sched_barrier(0);
        wait_vmcnt<kStatLoads + kQCopies>();
        lds_barrier();
        // dV, then dP and dS
#pragma unroll
        for (int u = 0; u < 2; ++u)
#pragma unroll
            for (int t = 0; t < DT; ++t) {
                const s16x4 a0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                    (lds_s16x4*)(do_t + t_off[t][0] + (16 * u) * G::kRowBytes));
                const s16x4 a1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                    (lds_s16x4*)(do_t + t_off[t][1] + (16 * u) * G::kRowBytes));
                const bf16x8 a = __builtin_bit_cast(bf16x8, __builtin_shufflevector(a0, a1, 0, 1, 2, 3, 4, 5, 6, 7));
                dvacc[t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, pb[u], dvacc[t], 0, 0, 0);
            }
        f32x16 dpacc;
#pragma unroll
        for (int r = 0; r < 16; ++r) dpacc[r] = 0.f;
#pragma unroll
        for (int s = 0; s < KS; ++s) {
            const bf16x8 a = *reinterpret_cast<const bf16x8*>(do_t + a_off[s]);
            const bf16x8 b = *reinterpret_cast<const bf16x8*>(v_t + b_shift + a_off[s]);
            dpacc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, dpacc, 0, 0, 0);
        }
#pragma unroll
        for (int g = 0; g < 4; ++g)
#pragma unroll
            for (int c = 0; c < 4; ++c)
                dsb[g / 2][4 * (g % 2) + c] = (__bf16)(p[4 * g + c] * (dpacc[4 * g + c] - dr[g][c]));
        // every wave has read this dO: its buffer takes the next block's dO
        lds_barrier();
        copy_tile<D>(do_rsrc, nxt, do_t, wave, lane_copy, stride);
#pragma unroll
        for (int u = 0; u < 2; ++u)
#pragma unroll
            for (int t = 0; t < DT; ++t) {
                const s16x4 a0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                    (lds_s16x4*)(qbuf + t_off[t][0] + (16 * u) * G::kRowBytes));
                const s16x4 a1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                    (lds_s16x4*)(qbuf + t_off[t][1] + (16 * u) * G::kRowBytes));
                const bf16x8 a = __builtin_bit_cast(bf16x8, __builtin_shufflevector(a0, a1, 0, 1, 2, 3, 4, 5, 6, 7));
                dkacc[t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, dsb[u], dkacc[t], 0, 0, 0);
            }
    };

    using P0 = std::integral_constant<int, 0>;
    using P1 = std::integral_constant<int, 1>;
    for (int i = 0; i < count; i += 2) {
        step(P0{}, i);
        if (i + 1 < count) step(P1{}, i + 1);
    }

    // sum the query halves: wave (kh, 1) hands its partial dV^T, dK^T to wave (kh, 0)
    wait_vmcnt<0>();
    lds_barrier();
    float* xv = reinterpret_cast<float*>(khalf ? q_t0 : k_t);
    float* xk = reinterpret_cast<float*>(khalf ? q_t1 : v_t);
    static_assert(DT * 16 * 64 * 4 <= G::kBytes, "partial dK / dV exceeds one tile buffer");
    if (qhalf == 1) {
#pragma unroll
        for (int t = 0; t < DT; ++t)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                xv[(t * 16 + r) * 64 + lane] = dvacc[t][r];
                xk[(t * 16 + r) * 64 + lane] = dkacc[t][r];
            }
    }
    lds_barrier();
    if (qhalf == 0) {
        const size_t key = (size_t)kv_first + row_in_block<RASTER>(grid, brow);
        __bf16* vrow = dv + head_off + key * D;
        __bf16* krow_out = dk + head_off + key * D;
#pragma unroll
        for (int t = 0; t < DT; ++t)
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                bf16x4 pv, pk;
#pragma unroll
                for (int c = 0; c < 4; ++c) {
                    const int r = 4 * g + c;
                    pv[c] = (__bf16)(dvacc[t][r] + xv[(t * 16 + r) * 64 + lane]);
                    pk[c] = (__bf16)((dkacc[t][r] + xk[(t * 16 + r) * 64 + lane]) * scale);
                }
                *reinterpret_cast<bf16x4*>(vrow + 32 * t + 8 * g + 4 * h) = pv;
                *reinterpret_cast<bf16x4*>(krow_out + 32 * t + 8 * g + 4 * h) = pk;
            }
    }
}

// ---------------------------------------------------------------------------
// float32 versions: plain FMAs, four threads per row, tiles in LDS (accuracy first).
// ---------------------------------------------------------------------------
template <int D, bool RASTER>
__global__ __launch_bounds__(256) void bwd_dq_f32_kernel(const float* __restrict__ q, const float* __restrict__ k,
                                                         const float* __restrict__ v, const float* __restrict__ dout,
                                                         const float* __restrict__ lse,
                                                         const float* __restrict__ drow, float* __restrict__ dq,
                                                         int L, int nb, const int32_t* __restrict__ kv_count,
                                                         const int32_t* __restrict__ kv_index,
                                                         const int32_t* __restrict__ schedule, RasterGrid grid,
                                                         float scale) {
    constexpr int LD = D + 1;
    extern __shared__ float lds[];
    float* q_s = lds;                  // [64][LD]
    float* do_s = q_s + kBlk * LD;     // [64][LD]
    float* k_s = do_s + kBlk * LD;     // [64][LD]
    float* v_s = k_s + kBlk * LD;      // [64][LD]
    float* ds_s = v_s + kBlk * LD;     // [64][65]

    const int logical = logical_item(schedule);
    const int bh = logical / nb;
    const int qb = logical - bh * nb;
    const int tid = threadIdx.x;
    const int row = tid >> 2;
    const int part = tid & 3;
    const size_t head_off = (size_t)bh * L * D;
    const uint32_t qbase = block_row<RASTER>(grid, qb);
    for (int i = tid; i < kBlk * D; i += 256) {
        const size_t src = head_off + (size_t)(qbase + row_in_block<RASTER>(grid, i / D)) * D + i % D;
        q_s[(i / D) * LD + i % D] = q[src];
        do_s[(i / D) * LD + i % D] = dout[src];
    }
    const int count = kv_count[(size_t)bh * nb + qb];
    const int32_t* list = kv_index + ((size_t)bh * nb + qb) * nb;
    const uint32_t my_row = qbase + row_in_block<RASTER>(grid, row);
    const float lse_r = count > 0 ? lse[(size_t)bh * L + my_row] : 0.f;
    const float d_r = drow[(size_t)bh * L + my_row];
    float acc[D / 4];
#pragma unroll
    for (int c = 0; c < D / 4; ++c) acc[c] = 0.f;

    for (int it = 0; it < count; ++it) {
        const uint32_t tb = block_row<RASTER>(grid, list[it]);
        __syncthreads();
        for (int i = tid; i < kBlk * D; i += 256) {
            const size_t src = head_off + (size_t)(tb + row_in_block<RASTER>(grid, i / D)) * D + i % D;
            k_s[(i / D) * LD + i % D] = k[src];
            v_s[(i / D) * LD + i % D] = v[src];
        }
        __syncthreads();
#pragma unroll 4
        for (int c = 0; c < 16; ++c) {
            const int kv = part + 4 * c;
            float s = 0.f, dp = 0.f;
            for (int e = 0; e < D; ++e) {
                s = fmaf(q_s[row * LD + e], k_s[kv * LD + e], s);
                dp = fmaf(do_s[row * LD + e], v_s[kv * LD + e], dp);
            }
            const float p = expf(s * scale - lse_r);
            ds_s[row * 65 + kv] = p * (dp - d_r);
        }
        __syncthreads();
#pragma unroll
        for (int c = 0; c < D / 4; ++c) {
            const int col = part + 4 * c;
            float a = acc[c];
            for (int kv = 0; kv < kBlk; ++kv) a = fmaf(ds_s[row * 65 + kv], k_s[kv * LD + col], a);
            acc[c] = a;
        }
    }
    float* out = dq + head_off + (size_t)my_row * D;
#pragma unroll
    for (int c = 0; c < D / 4; ++c) out[part + 4 * c] = acc[c] * scale;
}

template <int D, bool RASTER>
__global__ __launch_bounds__(256) void bwd_dkdv_f32_kernel(const float* __restrict__ q, const float* __restrict__ k,
                                                           const float* __restrict__ v,
                                                           const float* __restrict__ dout,
                                                           const float* __restrict__ lse,
                                                           const float* __restrict__ drow, float* __restrict__ dk,
                                                           float* __restrict__ dv, int L, int nb,
                                                           const int32_t* __restrict__ q_count,
                                                           const int32_t* __restrict__ q_index,
                                                           const int32_t* __restrict__ schedule, RasterGrid grid,
                                                           float scale) {
    constexpr int LD = D + 1;
    extern __shared__ float lds[];
    float* k_s = lds;                  // [64][LD]
    float* v_s = k_s + kBlk * LD;      // [64][LD]
    float* q_s = v_s + kBlk * LD;      // [64][LD]
    float* do_s = q_s + kBlk * LD;     // [64][LD]
    float* buf = do_s + kBlk * LD;     // [64][65]: P, then dS, key-major
    float* st = buf + kBlk * 65;       // lse [64], D [64] of the query block

    const int logical = logical_item(schedule);
    const int bh = logical / nb;
    const int kb = logical - bh * nb;
    const int tid = threadIdx.x;
    const int key = tid >> 2;
    const int part = tid & 3;
    const size_t head_off = (size_t)bh * L * D;
    const uint32_t kbase = block_row<RASTER>(grid, kb);
    for (int i = tid; i < kBlk * D; i += 256) {
        const size_t src = head_off + (size_t)(kbase + row_in_block<RASTER>(grid, i / D)) * D + i % D;
        k_s[(i / D) * LD + i % D] = k[src];
        v_s[(i / D) * LD + i % D] = v[src];
    }
    const int count = q_count[(size_t)bh * nb + kb];
    const int32_t* list = q_index + ((size_t)bh * nb + kb) * nb;
    float accv[D / 4], acck[D / 4];
#pragma unroll
    for (int c = 0; c < D / 4; ++c) {
        accv[c] = 0.f;
        acck[c] = 0.f;
    }
    for (int it = 0; it < count; ++it) {
        const uint32_t qrow0 = block_row<RASTER>(grid, list[it]);
        __syncthreads();
        for (int i = tid; i < kBlk * D; i += 256) {
            const size_t src = head_off + (size_t)(qrow0 + row_in_block<RASTER>(grid, i / D)) * D + i % D;
            q_s[(i / D) * LD + i % D] = q[src];
            do_s[(i / D) * LD + i % D] = dout[src];
        }
        if (tid < kBlk) {
            const size_t r = (size_t)bh * L + qrow0 + row_in_block<RASTER>(grid, tid);
            st[tid] = lse[r];
            st[kBlk + tid] = drow[r];
        }
        __syncthreads();
        float ds[16];
#pragma unroll 4
        for (int c = 0; c < 16; ++c) {
            const int qi = part + 4 * c;
            float s = 0.f, dp = 0.f;
            for (int e = 0; e < D; ++e) {
                s = fmaf(q_s[qi * LD + e], k_s[key * LD + e], s);
                dp = fmaf(do_s[qi * LD + e], v_s[key * LD + e], dp);
            }
            const float p = expf(s * scale - st[qi]);
            buf[key * 65 + qi] = p;
            ds[c] = p * (dp - st[kBlk + qi]);
        }
        __syncthreads();
#pragma unroll
        for (int c = 0; c < D / 4; ++c) {
            const int col = part + 4 * c;
            float a = accv[c];
            for (int qi = 0; qi < kBlk; ++qi) a = fmaf(buf[key * 65 + qi], do_s[qi * LD + col], a);
            accv[c] = a;
        }
        __syncthreads();
#pragma unroll
        for (int c = 0; c < 16; ++c) buf[key * 65 + part + 4 * c] = ds[c];
        __syncthreads();
#pragma unroll
        for (int c = 0; c < D / 4; ++c) {
            const int col = part + 4 * c;
            float a = acck[c];
            for (int qi = 0; qi < kBlk; ++qi) a = fmaf(buf[key * 65 + qi], q_s[qi * LD + col], a);
            acck[c] = a;
        }
    }
    const size_t out_off = head_off + (size_t)(kbase + row_in_block<RASTER>(grid, key)) * D;
    float* vout = dv + out_off;
    float* kout = dk + out_off;
#pragma unroll
    for (int c = 0; c < D / 4; ++c) {
        vout[part + 4 * c] = accv[c];
        kout[part + 4 * c] = acck[c] * scale;
    }
}

// ---------------------------------------------------------------------------
// launchers
// ---------------------------------------------------------------------------
template <typename T, int D>
hipError_t launch_rowdot(const AttnBwdArgs& a, hipStream_t s) {
    constexpr int kLanes = D / (16 / (int)sizeof(T));
    constexpr int kRows = 256 / kLanes;
    const long long rows = (long long)a.BH * a.L;
    hipLaunchKernelGGL((bwd_rowdot_kernel<T, D>), dim3((unsigned)((rows + kRows - 1) / kRows)), dim3(256), 0, s,
                       (const T*)a.o, (const T*)a.dout, a.drow, rows);
    return hipGetLastError();
}

hipError_t launch_qlists(const AttnBwdArgs& a, hipStream_t s) {
    const int words = (a.nb + 31) / 32;
    const long long n = (long long)a.BH * a.nb * words;
    hipLaunchKernelGGL(bwd_zero_kernel, dim3((unsigned)std::min<long long>((n + 255) / 256, 4096)), dim3(256), 0, s,
                       a.bits, n);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(bwd_scatter_kernel, dim3(a.BH * a.nb), dim3(256), 0, s, a.kv_count, a.kv_index, a.nb, words,
                       a.bits);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(bwd_qlist_kernel, dim3(a.BH * a.nb), dim3(64), 0, s, a.bits, a.nb, words, a.q_count,
                       a.q_index);
    return hipGetLastError();
}

// The raster grid of 8 x 8 patches (unused in fractal order).
RasterGrid raster_grid(const AttnBwdArgs& a) {
    RasterGrid g{};
    if (a.raster) {
        g.W = (uint32_t)a.W;
        g.HW = (uint32_t)(a.H * a.W);
        g.nHW = FastDiv((uint32_t)((a.H / 8) * (a.W / 8)));
        g.nW = FastDiv((uint32_t)(a.W / 8));
    }
    return g;
}

template <int D, bool RASTER>
hipError_t launch_bf16(const AttnBwdArgs& a, hipStream_t s) {
    const float sl2 = a.scale * kLog2e;
    const RasterGrid grid = raster_grid(a);
    hipLaunchKernelGGL((bwd_dq_bf16_kernel<D, RASTER>), dim3(a.BH * a.nb), dim3(kThreads), 0, s, (const __bf16*)a.q,
                       (const __bf16*)a.k, (const __bf16*)a.v, (const __bf16*)a.dout, a.lse, a.drow, (__bf16*)a.dq,
                       a.L, a.nb, a.kv_count, a.kv_index, a.sched_q, grid, sl2, a.scale);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL((bwd_dkdv_bf16_kernel<D, RASTER>), dim3(a.BH * a.nb), dim3(kThreads), 0, s,
                       (const __bf16*)a.q, (const __bf16*)a.k, (const __bf16*)a.v, (const __bf16*)a.dout, a.lse,
                       a.drow, (__bf16*)a.dk, (__bf16*)a.dv, a.L, a.nb, a.q_count, a.q_index, a.sched_k, grid, sl2,
                       a.scale);
    return hipGetLastError();
}

template <int D, bool RASTER>
hipError_t launch_f32(const AttnBwdArgs& a, hipStream_t s) {
    const size_t lds = (4 * kBlk * (D + 1) + kBlk * 65 + 2 * kBlk) * sizeof(float);
    static std::atomic<uint64_t> set_q{0}, set_k{0};
    hipError_t e = set_max_dynamic_lds((const void*)bwd_dq_f32_kernel<D, RASTER>, (int)lds, set_q);
    if (e != hipSuccess) return e;
    e = set_max_dynamic_lds((const void*)bwd_dkdv_f32_kernel<D, RASTER>, (int)lds, set_k);
    if (e != hipSuccess) return e;
    const RasterGrid grid = raster_grid(a);
    hipLaunchKernelGGL((bwd_dq_f32_kernel<D, RASTER>), dim3(a.BH * a.nb), dim3(256), lds, s, (const float*)a.q,
                       (const float*)a.k, (const float*)a.v, (const float*)a.dout, a.lse, a.drow, (float*)a.dq, a.L,
                       a.nb, a.kv_count, a.kv_index, a.sched_q, grid, a.scale);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL((bwd_dkdv_f32_kernel<D, RASTER>), dim3(a.BH * a.nb), dim3(256), lds, s, (const float*)a.q,
                       (const float*)a.k, (const float*)a.v, (const float*)a.dout, a.lse, a.drow, (float*)a.dk,
                       (float*)a.dv, a.L, a.nb, a.q_count, a.q_index, a.sched_k, grid, a.scale);
    return hipGetLastError();
}

template <bool RASTER>
hipError_t launch_sweeps(const AttnBwdArgs& a, hipStream_t s) {
    if (a.bf16) return a.d == 128 ? launch_bf16<128, RASTER>(a, s) : launch_bf16<64, RASTER>(a, s);
    return a.d == 128 ? launch_f32<128, RASTER>(a, s) : launch_f32<64, RASTER>(a, s);
}

}  // namespace

hipError_t launch_attn_bwd(const AttnBwdArgs& a, hipStream_t s) {
    hipError_t e = a.bf16 ? (a.d == 128 ? launch_rowdot<__bf16, 128>(a, s) : launch_rowdot<__bf16, 64>(a, s))
                          : (a.d == 128 ? launch_rowdot<float, 128>(a, s) : launch_rowdot<float, 64>(a, s));
    if (e != hipSuccess) return e;
    e = launch_qlists(a, s);
    if (e != hipSuccess) return e;
    e = launch_schedule(a.kv_count, a.BH, a.nb, a.sched_q, s);
    if (e != hipSuccess) return e;
    e = launch_schedule(a.q_count, a.BH, a.nb, a.sched_k, s);
    if (e != hipSuccess) return e;
    return a.raster ? launch_sweeps<true>(a, s) : launch_sweeps<false>(a, s);
}

}  // namespace nabla
