// Block-sparse flash attention, bf16 in / bf16 out, for 64-token blocks.
//
// Computes softmax attention only on the kept 64 x 64 tiles (NABLA technical summary,
// "Metodologia: NABLA", item 2, "Expansão"); a dropped tile contributes neither to the
// numerator nor to the normaliser.
//
// One workgroup = two 64-row query blocks (a pair), four waves: waves 0, 1 take query
// rows [0, 32) and [32, 64) of the first block, waves 2, 3 those of the second.  The
// workgroup walks the union of the two blocks' ascending KV lists; each KV tile is copied
// into LDS once, and a wave computes on it only if its own block keeps it.  Video blocks
// that are neighbours in time keep largely the same KV blocks, so a pair of them shares
// most of its tile copies (the mask step's start order pairs each block with the block
// of the next frame at the same patch position).  Every wave accumulates its block's
// tiles in its list's ascending order whatever the partner, so results do not depend on
// the pairing or the start order.  Per tile, a wave that keeps it runs
//     S^T = K Q^T      v_mfma_f32_32x32x16_bf16 over both 32-key halves, A = K from
//                      LDS, B = Q (VGPRs)
//     online softmax   float32, exp2 with scale*log2(e) folded into one FMA
//     O^T += V^T P^T   v_mfma_f32_32x32x16_bf16, A = V^T from LDS, B = P (VGPRs)
// Computing the transposed products makes every lane own one query column: its S^T
// accumulator already has the layout the P operand of the second product needs (the
// MFMA's k index is permuted identically in both operands, which leaves the sum
// unchanged), and the row statistics stay in the lane, with one exchange between lanes
// l and l^32, which split each 32-key half.
//
// Memory pipeline: K and V tiles go from global memory straight into LDS with the
// buffer form of the LDS DMA (buffer_load_dwordx4 ... lds, no VGPR staging), row-major
// with an XOR swizzle of the 16-byte chunks, and are double-buffered: at the top of
// iteration i, after one barrier, the workgroup issues the copies of tile i+1 (each wave
// its share, spread between its MFMAs), which have the whole iteration to land.  64 KiB
// of LDS per workgroup puts two workgroups on a CU, two waves on every SIMD.  V^T
// operands come out of the row-major V tile through the transposing LDS read
// (ds_read_b64_tr_b16).  The four buffers are separate LDS objects, so the compiler sees
// that reading one never waits for a copy into another.
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
                          const __bf16* __restrict__ v, __bf16* __restrict__ o, int L, int nb, int total,
                          const int32_t* __restrict__ kv_count, const int32_t* __restrict__ kv_index,
                          const int32_t* __restrict__ schedule, RasterGrid grid, float scale_log2e,
                          float* __restrict__ lse, const float* __restrict__ kv_logw) {
    using G = Tile<D>;
    constexpr int KS = D / 16;        // k-steps of S^T = K Q^T per 32-key half
    constexpr int DT = D / 32;        // 32-row d tiles of O^T
    constexpr int kEnd = 0x7fffffff;  // past the end of a list
    const uint32_t stride = copy_stride<RASTER>(grid);   // between a tile's 4 KiB copies
    __shared__ __attribute__((aligned(1024))) char k_lds0[G::kBytes];
    __shared__ __attribute__((aligned(1024))) char k_lds1[G::kBytes];
    __shared__ __attribute__((aligned(1024))) char v_lds0[G::kBytes];
    __shared__ __attribute__((aligned(1024))) char v_lds1[G::kBytes];

    // Work item -> a pair of query blocks (flat ids (b*heads + h)*nb + i).  Workgroups are
    // dealt round-robin to the 8 XCDs; without a schedule, remap so that each XCD walks a
    // contiguous range of pairs (2j, 2j+1).  With a schedule, workgroup j takes its
    // entries 2j and 2j+1.
    const int nwg = gridDim.x;
    const int full = (nwg / 8) * 8;
    int item = blockIdx.x;
    if (!schedule && item < full) item = (item % 8) * (nwg / 8) + item / 8;
    const bool has_b = 2 * item + 1 < total;
    const int qa = schedule ? schedule[2 * item] : 2 * item;
    const int qb = has_b ? (schedule ? schedule[2 * item + 1] : 2 * item + 1) : qa;
    const int bha = qa / nb, bhb = qb / nb;

    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // uniform per wave
    const int slot = wave >> 1;       // 0: block qa, 1: block qb
    const int qhalf = wave & 1;       // query rows 32 qhalf .. 32 qhalf + 31 of the slot's block
    const bool active = slot == 0 || has_b;
    const int lane = tid & 63;
    const int h = lane >> 5;
    const int c32 = lane & 31;

    const int head_bytes = L * D * 2;
    const __amdgpu_buffer_rsrc_t ka_rsrc =
        __builtin_amdgcn_make_buffer_rsrc((void*)(k + (size_t)bha * L * D), 0, head_bytes, kBufferFlags);
    const __amdgpu_buffer_rsrc_t va_rsrc =
        __builtin_amdgcn_make_buffer_rsrc((void*)(v + (size_t)bha * L * D), 0, head_bytes, kBufferFlags);
    const __amdgpu_buffer_rsrc_t kb_rsrc =
        __builtin_amdgcn_make_buffer_rsrc((void*)(k + (size_t)bhb * L * D), 0, head_bytes, kBufferFlags);
    const __amdgpu_buffer_rsrc_t vb_rsrc =
        __builtin_amdgcn_make_buffer_rsrc((void*)(v + (size_t)bhb * L * D), 0, head_bytes, kBufferFlags);
    const uint32_t k_copy = copy_lane_offset_in<D, false, RASTER>(grid, wave, lane);
    const uint32_t v_copy = copy_lane_offset_in<D, true, RASTER>(grid, wave, lane);

    // The union walk: keys of the first list are its KV blocks; those of the second are
    // its KV blocks, shifted past nb when the two blocks belong to different heads (their
    // tiles then never coincide, and the walk takes the first list, then the second).
    const int ca = kv_count[qa];
    const int cb = has_b ? kv_count[qb] : 0;
    const int32_t* la = kv_index + (size_t)qa * nb;
    const int32_t* lb = kv_index + (size_t)qb * nb;
    const int offb = bhb != bha ? nb : 0;
    int ia = 0, ib = 0;
    int key_a = ca > 0 ? la[0] : kEnd;
    int key_b = cb > 0 ? lb[0] + offb : kEnd;
    // next tile of the union: its key, whether each list holds it, and its place in each
    auto pop = [&](int& key, bool& in_a, bool& in_b, int& pos_a, int& pos_b) {
        key = min(key_a, key_b);
        in_a = key_a == key && key != kEnd;
        in_b = key_b == key && key != kEnd;
        pos_a = ia;
        pos_b = ib;
        if (in_a) {
            ++ia;
            key_a = ia < ca ? la[ia] : kEnd;
        }
        if (in_b) {
            ++ib;
            key_b = ib < cb ? lb[ib] + offb : kEnd;
        }
    };
    // byte offset of a key's tile in its head, and that head's K and V
    auto tile_at = [&](int key, __amdgpu_buffer_rsrc_t& kr, __amdgpu_buffer_rsrc_t& vr) -> uint32_t {
        const bool second = key >= nb;
        kr = second ? kb_rsrc : ka_rsrc;
        vr = second ? vb_rsrc : va_rsrc;
        return block_row<RASTER>(grid, second ? key - nb : key) * G::kRowBytes;
    };

    int cur, nxt, cpa, cpb, npa, npb;
    bool cin_a, cin_b, nin_a, nin_b;
    pop(cur, cin_a, cin_b, cpa, cpb);
    pop(nxt, nin_a, nin_b, npa, npb);
    if (cur != kEnd) {
        __amdgpu_buffer_rsrc_t kr, vr;
        const uint32_t first = tile_at(cur, kr, vr);
        copy_tile<D>(kr, first, k_lds0, wave, k_copy, stride);
        copy_tile<D>(vr, first, v_lds0, wave, v_copy, stride);
    }

    // this wave's block, head and query row (fractal or raster order)
    const int my_q = slot ? qb : qa;
    const int my_bh = slot ? bhb : bha;
    const int my_blk = my_q - my_bh * nb;
    const size_t head_off = (size_t)my_bh * L * D;
    const uint32_t qrow = block_row<RASTER>(grid, my_blk) + row_in_block<RASTER>(grid, 32 * qhalf + c32);
    // Q operand: lane holds Q[row][16 s + 8 h .. + 7] for s = 0..KS-1.
    bf16x8 qreg[KS];
#pragma unroll
    for (int s = 0; s < KS; ++s)
        qreg[s] = active ? *reinterpret_cast<const bf16x8*>(q + head_off + (size_t)qrow * D + 16 * s + 8 * h)
                         : bf16x8{};

    f32x16 oacc[DT];
#pragma unroll
    for (int t = 0; t < DT; ++t)
#pragma unroll
        for (int r = 0; r < 16; ++r) oacc[t][r] = 0.f;
    float m_run = -INFINITY;   // reference max of scaled logits (log2 domain), same in l, l^32
    float l_run = 0.f;         // this lane's share of the running normaliser

    // per-lane LDS byte offsets that do not change from tile to tile; the second 32-key
    // half is 32 rows further on (the swizzles repeat every 16 rows)
    const int krow = c32;
    int k_off[KS];
#pragma unroll
    for (int s = 0; s < KS; ++s) k_off[s] = krow * G::kRowBytes + (((2 * s + h) ^ G::k_swz(krow)) * 16);
    // V^T operand of d tile t, k-step u (16 keys), half p: rows 16 u + 8 p + 4 h + j16 / 4;
    // only the d tile changes the swizzled part, (16 u + 8 p) rows are a constant offset
    const int g16 = lane >> 4, j16 = lane & 15;
    int v_off[DT];
#pragma unroll
    for (int t = 0; t < DT; ++t) {
        const int row = 4 * h + (j16 >> 2);
        const int d = 32 * t + 16 * (g16 & 1) + 4 * (j16 & 3);
        v_off[t] = row * G::kRowBytes + (((d >> 3) ^ G::v_swz(row)) * 16) + ((d >> 2) & 1) * 8;
    }
    const float* logw_row = WEIGHTED ? kv_logw + (size_t)my_q * nb : nullptr;

    // One union tile; PAR selects the buffers holding it.  The copy issued here is that of
    // the next tile, or of this tile again after the last one (into buffers nothing reads
    // any more), which keeps the copies unconditional.
    auto step = [&](auto par) {
        constexpr int PAR = decltype(par)::value;
        const char* kbuf = PAR ? k_lds1 : k_lds0;
        const char* vbuf = PAR ? v_lds1 : v_lds0;
        // this tile has landed (issued one iteration ago); after the barrier every wave
        // sees it and is done with the buffers of the previous tile, refilled now
        wait_vmcnt<0>();
        lds_barrier();
        __amdgpu_buffer_rsrc_t kr, vr;
        const uint32_t nxt_byte = tile_at(nxt != kEnd ? nxt : cur, kr, vr);
        char* k_dst = PAR ? k_lds0 : k_lds1;
        char* v_dst = PAR ? v_lds0 : v_lds1;
        constexpr int kEveryK = 2 * KS / G::kCopiesPerWave;   // one K copy per kEveryK MFMAs
        constexpr int kEveryV = 4 * DT / G::kCopiesPerWave;   // one V copy per kEveryV MFMAs
        const bool mine = slot ? cin_b : cin_a;

        if (mine) {
            // the tile's additive logit shift (log2 units): a sampled block's log(1 / pi)
            const float wl = WEIGHTED ? logw_row[slot ? cpb : cpa] * 1.4426950408889634f : 0.f;
            // ---- S^T = K Q^T for the 64 keys (two 32-key halves) and the wave's 32 query
            // columns; the wave's copies of the next K tile go between the MFMAs
            f32x16 sacc[2];
#pragma unroll
            for (int kh = 0; kh < 2; ++kh) {
#pragma unroll
                for (int r = 0; r < 16; ++r) sacc[kh][r] = 0.f;
                bf16x8 ka[KS];
#pragma unroll
                for (int s = 0; s < KS; ++s)
                    ka[s] = *reinterpret_cast<const bf16x8*>(kbuf + k_off[s] + kh * 32 * G::kRowBytes);
                __builtin_amdgcn_sched_barrier(0);
#pragma unroll
                for (int s = 0; s < KS; ++s) {
                    sacc[kh] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka[s], qreg[s], sacc[kh], 0, 0, 0);
                    const int m = kh * KS + s;
                    if (m % kEveryK == 0)
                        __builtin_amdgcn_raw_ptr_buffer_load_lds(
                            kr, (lds_void*)(k_dst + (4 * (m / kEveryK) + wave) * 1024), 16, k_copy,
                            nxt_byte + (m / kEveryK) * stride, 0, 0);
                    __builtin_amdgcn_sched_barrier(0);
                }
            }

            // ---- online softmax for query column c32 (keys split between lanes l, l^32).
            // The reference maximum m_run only moves when a tile's maximum exceeds it by
            // more than 8 (log2 units), so P stays below 2^8 and the rescale of O and l is
            // rare; normalising by l at the end makes the result independent of m_run.
            float mx = -INFINITY;
#pragma unroll
            for (int kh = 0; kh < 2; ++kh)
#pragma unroll
                for (int r = 0; r < 16; ++r) mx = fmaxf(mx, sacc[kh][r]);
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

            // ---- O^T += V^T P^T over four 16-key k-steps; P of k-step u is accumulator
            // entries 8 (u % 2) .. + 7 of key half u / 2
            bf16x8 pb[4];
#pragma unroll
            for (int u = 0; u < 4; ++u)
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    const float pe =
                        __builtin_amdgcn_exp2f(fmaf(sacc[u >> 1][8 * (u & 1) + e], scale_log2e, wl - m_run));
                    l_run += pe;
                    pb[u][e] = (__bf16)pe;
                }
#pragma unroll
            for (int u = 0; u < 4; ++u)
#pragma unroll
                for (int t = 0; t < DT; ++t) {
                    const int m = u * DT + t;
                    if (m % kEveryV == 0)
                        __builtin_amdgcn_raw_ptr_buffer_load_lds(
                            vr, (lds_void*)(v_dst + (4 * (m / kEveryV) + wave) * 1024), 16, v_copy,
                            nxt_byte + (m / kEveryV) * stride, 0, 0);
                    const s16x4 v0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                        (lds_s16x4*)(vbuf + v_off[t] + (16 * u) * G::kRowBytes));
                    const s16x4 v1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                        (lds_s16x4*)(vbuf + v_off[t] + (16 * u + 8) * G::kRowBytes));
                    const bf16x8 a =
                        __builtin_bit_cast(bf16x8, __builtin_shufflevector(v0, v1, 0, 1, 2, 3, 4, 5, 6, 7));
                    oacc[t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, pb[u], oacc[t], 0, 0, 0);
                }
        } else {
            // a tile only the partner keeps: just this wave's share of the next copies
            copy_tile<D>(kr, nxt_byte, k_dst, wave, k_copy, stride);
            copy_tile<D>(vr, nxt_byte, v_dst, wave, v_copy, stride);
        }
        // the tile after next, read after this one's last LDS wait so that its scalar
        // loads are done by the barrier that opens the next iteration
        __builtin_amdgcn_sched_barrier(0);
        cur = nxt;
        cin_a = nin_a;
        cin_b = nin_b;
        cpa = npa;
        cpb = npb;
        pop(nxt, nin_a, nin_b, npa, npb);
    };

    using P0 = std::integral_constant<int, 0>;
    using P1 = std::integral_constant<int, 1>;
    while (cur != kEnd) {
        step(P0{});
        if (cur == kEnd) break;
        step(P1{});
    }
    // the last copies (of the last tile again, into buffers no longer read) land before
    // the workgroup retires
    wait_vmcnt<0>();
    if (!active) return;

    float l = l_run;
    {
        const auto pr = __builtin_amdgcn_permlane32_swap(__float_as_uint(l), __float_as_uint(l), false, false);
        l = __uint_as_float(pr[0]) + __uint_as_float(pr[1]);
    }
    const float inv = (l > 0.f) ? 1.0f / l : 0.f;
    // log-sum-exp of the row's scaled logits: P = exp2(s * scale * log2(e) - m) / l, so
    // the sum of exp(s * scale) is 2^m * l
    if (lse && h == 0)
        lse[(size_t)my_bh * L + qrow] = l > 0.f ? (m_run + __log2f(l)) * 0.69314718055994531f : -INFINITY;
    // lane holds O[qrow][32 t + 8 g + 4 h + c], c = 0..3
    __bf16* orow = o + head_off + (size_t)qrow * D;
#pragma unroll
    for (int t = 0; t < DT; ++t)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
            bf16x4 pk;
#pragma unroll
            for (int c = 0; c < 4; ++c) pk[c] = (__bf16)(oacc[t][4 * g + c] * inv);
            *reinterpret_cast<bf16x4*>(orow + 32 * t + 8 * g + 4 * h) = pk;
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
    const int total = a.BH * a.nb;   // query blocks, two per workgroup
    hipLaunchKernelGGL((attn_fwd_bf16_kernel<D, RASTER, WEIGHTED>), dim3((total + 1) / 2), dim3(kThreads), 0, s,
                       (const __bf16*)a.q, (const __bf16*)a.k, (const __bf16*)a.v, (__bf16*)a.o,
                       a.L, a.nb, total, a.kv_count, a.kv_index, a.schedule, grid, scale_log2e, a.lse,
                       a.kv_logw);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_attn_bf16(const AttnArgs& a, hipStream_t s) {
    if (a.kv_logw) return a.d == 128 ? launch<128, false, true>(a, s) : launch<64, false, true>(a, s);
    if (a.raster) return a.d == 128 ? launch<128, true, false>(a, s) : launch<64, true, false>(a, s);
    return a.d == 128 ? launch<128, false, false>(a, s) : launch<64, false, false>(a, s);
}

}  // namespace nabla
