// Adaptive block mask (NABLA technical summary, "Metodologia: NABLA", item 2, with the
// STA union of item 3):
//   pool_kernel        block means of Q and K (one HBM pass over both, float32 sums)
//   map_select_kernel  reduced map S = Qp Kp^T * scale on float32 MFMA, row softmax,
//                      the CDF cutoff found by bisection on float32 bit patterns, the
//                      STA OR, and compaction of each row into an ascending kept list.
#include <math.h>

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

template <typename T, int D, int N>
__global__ __launch_bounds__(256) void pool_kernel(const T* __restrict__ q,
                                                    const T* __restrict__ k,
                                                    float* __restrict__ qp,
                                                    float* __restrict__ kp, int total_blocks) {
    constexpr int EPC = Elem<T>::kPerChunk;
    constexpr int CHUNKS = D / EPC;          // 16-byte chunks per token
    constexpr int G = 64 / CHUNKS;           // tokens per load instruction
    constexpr int ITERS = N / G;
    const int wave = (blockIdx.x * 256 + threadIdx.x) >> 6;
    const int lane = threadIdx.x & 63;
    if (wave >= 2 * total_blocks) return;
    const bool is_k = wave >= total_blocks;
    const int blk = is_k ? wave - total_blocks : wave;
    const T* src = (is_k ? k : q) + (size_t)blk * N * D;
    float* dst = (is_k ? kp : qp) + (size_t)blk * D;
    const int c = lane % CHUNKS;
    const int g = lane / CHUNKS;

    u32x4 raw[ITERS];
#pragma unroll
    for (int r = 0; r < ITERS; ++r) {
        raw[r] = __builtin_nontemporal_load(
            reinterpret_cast<const u32x4*>(src + (size_t)(r * G + g) * D) + c);
    }
    float acc[EPC];
#pragma unroll
    for (int e = 0; e < EPC; ++e) acc[e] = 0.f;
#pragma unroll
    for (int r = 0; r < ITERS; ++r) {
        float v[EPC];
        Elem<T>::unpack(raw[r], v);
#pragma unroll
        for (int e = 0; e < EPC; ++e) acc[e] += v[e];
    }
#pragma unroll
    for (int off = CHUNKS; off < 64; off <<= 1) {
#pragma unroll
        for (int e = 0; e < EPC; ++e) acc[e] += __shfl_xor(acc[e], off);
    }
    if (g == 0) {
        constexpr float inv = 1.0f / N;      // N is a power of two: exact
        float* o = dst + c * EPC;
#pragma unroll
        for (int e = 0; e < EPC; e += 4) {
            *reinterpret_cast<f32x4*>(o + e) =
                f32x4{acc[e] * inv, acc[e + 1] * inv, acc[e + 2] * inv, acc[e + 3] * inv};
        }
    }
}

// ---------------------------------------------------------------------------
// Reduced map + softmax + CDF cutoff + STA + lists.
// A workgroup owns 16 query blocks (rows) of one head.
// Phase 1: each wave computes 16x16 tiles of S with v_mfma_f32_16x16x4_f32 (float32
//   operands, float32 accumulation) and parks them in LDS.
// Phase 2: each wave takes whole rows: softmax, then the cutoff.  Keeping block j
//   iff F_j > thr is the same as keeping every block whose value is at least v*, the
//   smallest row value with g(v*) > thr, where g(u) = sum of the row values <= u.
//   g only grows with u, and for non-negative floats the bit patterns order like
//   the values, so v* is found by bisection over 32-bit patterns: 31 masked sums.
// ---------------------------------------------------------------------------
constexpr int kRows = 16;
constexpr int kMaxChunks = (NABLA_MAX_BLOCKS + 63) / 64;

__device__ inline float wave_sum(float x) {
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) x += __shfl_xor(x, off);
    return x;
}
__device__ inline float wave_max(float x) {
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) x = fmaxf(x, __shfl_xor(x, off));
    return x;
}
__device__ inline uint32_t wave_max_u32(uint32_t x) {
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) x = max(x, (uint32_t)__shfl_xor((int)x, off));
    return x;
}

template <int D>
__global__ __launch_bounds__(256) void map_select_kernel(
    const float* __restrict__ qp, const float* __restrict__ kp, int nb, int ld_s, float scale,
    float thr, int sta, int nH, int nW, int rt, int rh, int rw, int32_t* __restrict__ kv_count,
    int32_t* __restrict__ kv_index, uint32_t* __restrict__ bitmap) {
    extern __shared__ float s_lds[];   // [kRows][ld_s]
    constexpr int KC = D / 4;          // k values per lane per MFMA chain
    const int wave = threadIdx.x >> 6;
    const int lane = threadIdx.x & 63;
    const int bh = blockIdx.y;
    const int row0 = blockIdx.x * kRows;
    const float* qh = qp + (size_t)bh * nb * D;
    const float* kh = kp + (size_t)bh * nb * D;
    const int n_chunks = (nb + 63) >> 6;
    const int ld_pad = n_chunks * 64;

    // ---- phase 1: S tiles.  The k index of the MFMA (lane / 16) selects a
    // contiguous quarter of d in both operands, so operand loads are 16-byte vectors.
    {
        const int li = lane & 15;
        const int kq = lane >> 4;
        float a[KC];
        const int qrow = row0 + li;
        if (qrow < nb) {
            const f32x4* src = reinterpret_cast<const f32x4*>(qh + (size_t)qrow * D + kq * KC);
#pragma unroll
            for (int v = 0; v < KC / 4; ++v) {
                f32x4 t = src[v];
                a[4 * v] = t[0]; a[4 * v + 1] = t[1]; a[4 * v + 2] = t[2]; a[4 * v + 3] = t[3];
            }
        } else {
#pragma unroll
            for (int v = 0; v < KC; ++v) a[v] = 0.f;
        }
        const int n_ct = ld_pad / 16;
        for (int ct = wave; ct < n_ct; ct += 4) {
            const int j = ct * 16 + li;
            float b[KC];
            if (j < nb) {
                const f32x4* src = reinterpret_cast<const f32x4*>(kh + (size_t)j * D + kq * KC);
#pragma unroll
                for (int v = 0; v < KC / 4; ++v) {
                    f32x4 t = src[v];
                    b[4 * v] = t[0]; b[4 * v + 1] = t[1]; b[4 * v + 2] = t[2]; b[4 * v + 3] = t[3];
                }
            } else {
#pragma unroll
                for (int v = 0; v < KC; ++v) b[v] = 0.f;
            }
            f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int s = 0; s < KC; ++s) acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a[s], b[s], acc, 0, 0, 0);
            // lane holds S[4*(lane/16) + r][16*ct + lane%16]
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int i = 4 * kq + r;
                s_lds[i * ld_s + j] = (j < nb) ? acc[r] * scale : -INFINITY;
            }
        }
    }
    __syncthreads();

    // ---- phase 2: one row per wave at a time.
    const int nwords = (nb + 31) >> 5;
    for (int r = wave; r < kRows; r += 4) {
        const int row = row0 + r;
        if (row >= nb) break;
        const float* srow = s_lds + r * ld_s;
        float v[kMaxChunks];
        float mx = -INFINITY;
#pragma unroll
        for (int m = 0; m < kMaxChunks; ++m) {
            if (m < n_chunks) {
                v[m] = srow[m * 64 + lane];
                mx = fmaxf(mx, v[m]);
            }
        }
        mx = wave_max(mx);
        float sum = 0.f;
#pragma unroll
        for (int m = 0; m < kMaxChunks; ++m) {
            if (m < n_chunks) {
                v[m] = expf(v[m] - mx);      // padding (-inf) becomes 0
                sum += v[m];
            }
        }
        sum = wave_sum(sum);
        uint32_t vmax_bits = 0;
#pragma unroll
        for (int m = 0; m < kMaxChunks; ++m) {
            if (m < n_chunks) {
                v[m] = v[m] / sum;
                vmax_bits = max(vmax_bits, __float_as_uint(v[m]));
            }
        }
        vmax_bits = wave_max_u32(vmax_bits);
        // smallest bit pattern u with g(u) > thr, searched in (lo, hi]; g(0) = 0 <= thr.
        uint32_t lo = 0, hi = vmax_bits;
        while (hi - lo > 1) {
            const uint32_t mid = lo + ((hi - lo) >> 1);
            float g = 0.f;
#pragma unroll
            for (int m = 0; m < kMaxChunks; ++m) {
                if (m < n_chunks) g += (__float_as_uint(v[m]) <= mid) ? v[m] : 0.f;
            }
            g = wave_sum(g);
            if (g > thr) hi = mid; else lo = mid;
        }
        // If even the whole row sums to <= thr (thr within rounding of 1), hi stays at
        // the row maximum, which keeps the largest block.
        const uint32_t cut = hi;

        int qt = 0, qh_ = 0, qw = 0;
        if (sta) {
            const int pf = nH * nW;
            qt = row / pf;
            const int rem = row - qt * pf;
            qh_ = rem / nW;
            qw = rem - qh_ * nW;
        }
        int32_t* out_idx = kv_index + ((size_t)bh * nb + row) * nb;
        uint32_t* out_bits = bitmap ? bitmap + ((size_t)bh * nb + row) * nwords : nullptr;
        int base = 0;
#pragma unroll
        for (int m = 0; m < kMaxChunks; ++m) {
            if (m < n_chunks) {
                const int j = m * 64 + lane;
                bool keep = false;
                if (j < nb) {
                    keep = __float_as_uint(v[m]) >= cut;
                    if (sta && !keep) {
                        const int pf = nH * nW;
                        const int kt = j / pf;
                        const int rem = j - kt * pf;
                        const int kh_ = rem / nW;
                        const int kw = rem - kh_ * nW;
                        keep = abs(kt - qt) <= rt && abs(kh_ - qh_) <= rh && abs(kw - qw) <= rw;
                    }
                }
                const uint64_t ballot = __ballot(keep);
                const int pos = base + __popcll(ballot & ((1ull << lane) - 1ull));
                if (keep) out_idx[pos] = j;
                base += __popcll(ballot);
                if (out_bits) {
                    if (lane == 0 && 2 * m < nwords) out_bits[2 * m] = (uint32_t)ballot;
                    if (lane == 1 && 2 * m + 1 < nwords) out_bits[2 * m + 1] = (uint32_t)(ballot >> 32);
                }
            }
        }
        if (lane == 0) kv_count[(size_t)bh * nb + row] = base;
    }
}

template <typename T, int D>
hipError_t launch_pool(const MaskArgs& a, hipStream_t s) {
    const int total = a.BH * a.nb;
    const int waves = 2 * total;
    hipLaunchKernelGGL((pool_kernel<T, D, 64>), dim3((waves + 3) / 4), dim3(256), 0, s,
                       (const T*)a.q, (const T*)a.k, a.qp, a.kp, total);
    return hipGetLastError();
}

template <int D>
hipError_t launch_map_select(const MaskArgs& a, hipStream_t s) {
    const int n_chunks = (a.nb + 63) / 64;
    const int ld_s = n_chunks * 64 + 16;
    const size_t lds = (size_t)kRows * ld_s * sizeof(float);
    static bool attr_set = false;
    if (!attr_set) {
        hipError_t e = hipFuncSetAttribute((const void*)map_select_kernel<D>,
                                           hipFuncAttributeMaxDynamicSharedMemorySize,
                                           kRows * ((kMaxChunks * 64) + 16) * (int)sizeof(float));
        if (e != hipSuccess) return e;
        attr_set = true;
    }
    dim3 grid((a.nb + kRows - 1) / kRows, a.BH);
    hipLaunchKernelGGL((map_select_kernel<D>), grid, dim3(256), lds, s, a.qp, a.kp, a.nb, ld_s,
                       a.scale, a.thr, a.sta, a.nH, a.nW, a.rt, a.rh, a.rw, a.kv_count,
                       a.kv_index, a.bitmap);
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
    return (a.d == 128) ? launch_map_select<128>(a, s) : launch_map_select<64>(a, s);
}

}  // namespace nabla
