// Internal declarations shared by the host API and the kernel launchers.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <atomic>

#include "nabla.h"

namespace nabla {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// Divide-by-invariant-integer with one multiply-high (Granlund & Montgomery 1994,
// "Division by invariant integers using multiplication", round-up variant):
// for 1 <= d < 2^31 and n < 2^31, n / d = (umulhi(n, magic) + n) >> shift with
// shift = ceil(log2 d) and magic = floor(2^32 (2^shift - d) / d) + 1.
struct FastDiv {
    uint32_t d, magic, shift;
    FastDiv() : d(1), magic(0), shift(0) {}
    explicit FastDiv(uint32_t div) : d(div) {
        shift = 0;
        while ((1u << shift) < div) ++shift;
        magic = (uint32_t)(((uint64_t(1) << 32) * ((uint64_t(1) << shift) - div)) / div + 1);
        if (div == 1) magic = 0;
    }
    __host__ __device__ inline uint32_t div(uint32_t n) const {
#ifdef __HIP_DEVICE_COMPILE__
        uint32_t hi = __umulhi(n, magic);
#else
        uint32_t hi = (uint32_t)(((uint64_t)n * magic) >> 32);
#endif
        return (hi + n) >> shift;
    }
    __host__ __device__ inline void divmod(uint32_t n, uint32_t& q, uint32_t& r) const {
        q = div(n);
        r = n - q * d;
    }
};

// Raises a kernel's dynamic-LDS limit on the current device.  The attribute is per
// device, so `done` remembers (one bit per device id below 64) where it has been set;
// concurrent first calls may both set it, which is harmless.
inline hipError_t set_max_dynamic_lds(const void* kernel, int bytes, std::atomic<uint64_t>& done) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    const uint64_t bit = (dev >= 0 && dev < 64) ? (uint64_t(1) << dev) : 0;
    if (bit && (done.load(std::memory_order_acquire) & bit)) return hipSuccess;
    e = hipFuncSetAttribute(kernel, hipFuncAttributeMaxDynamicSharedMemorySize, bytes);
    if (e == hipSuccess && bit) done.fetch_or(bit, std::memory_order_release);
    return e;
}

struct ReorderArgs {
    const void* src;
    void* dst;
    int BH, T, H, W, P, L;
    int chunk_shift;   // log2(16-byte chunks per token)
    int inverse;
};
hipError_t launch_reorder(const ReorderArgs& a, hipStream_t s);

// IBCS clustering: centroids per query block and Lloyd rounds.
constexpr int kIbcsClusters = 8;
constexpr int kIbcsIters = 4;

struct MaskArgs {
    const void* q;
    const void* k;
    int BH, nb, d, N;
    int T, nH, nW;          // tile grid (frames, patch rows, patch columns) for STA
    float thr, scale;
    int sta;                // 0 = off
    int rt, rh, rw;         // STA radii in tiles
    int32_t* kv_count;
    int32_t* kv_index;
    uint32_t* bitmap;       // may be null
    int32_t* schedule;      // may be null
    float* qp;              // unused (Q is pooled inside the map kernel); null
    float* kp;              // workspace: pooled K, [BH, nb, d] float32 (IBCS) or the split
                            // half form [BH, nb][hi d | lo d] (NABLA's map), 4 nb d bytes per head
    int32_t* kexp;          // workspace [BH, nb]: exponents of the split form (NABLA)
    float* scores;          // IBCS workspace [BH, groups, nb] score rows (rows sum to one)
    int bf16;
    int raster;             // 0: q, k in fractal order; 1: raster order, 8 x 8 patches per block
    int H, W;               // token grid, for the raster order
    int sip_budget;         // > 0: sampled selection with this expected budget per row (no CDF cut)
    const float* uniforms;  // SIP draws [BH, nb, nb]
    float* kv_logw;         // SIP out: log(1 / pi) per list entry [BH, nb, nb]
    int ibcs;               // 1: rows of the map are IBCS centroids (Q is clustered, not pooled)
    int ibcs_group;         // IBCS query blocks per cluster group (1: 64 queries, 2: 128)
    float* cent;            // IBCS workspace [BH, groups * kIbcsClusters, d] centroids
    float* cent_w;          // IBCS workspace [BH, groups * kIbcsClusters] cluster weights
};
hipError_t launch_build_mask(const MaskArgs& a, hipStream_t s);

// The allocation-free mask entry's scratch: a device array of kScratchBytes per GPU
// (scratch.hip).  device_scratch returns its address on the current device, resolved once
// per device.
constexpr size_t kScratchBytes = NABLA_NOALLOC_SCRATCH_BYTES;
hipError_t device_scratch(void** ptr, size_t* bytes);
hipError_t launch_ibcs_cluster(const MaskArgs& a, hipStream_t s);

struct AttnArgs {
    const void* q;
    const void* k;
    const void* v;
    void* o;
    int BH, L, nb, d;
    const int32_t* kv_count;
    const int32_t* kv_index;
    const int32_t* schedule;   // may be null
    float scale;
    float* lse;                // may be null: natural-log log-sum-exp per query row [BH, L]
    int raster;                // 0: blocks are runs of 64 rows; 1: raster T x H x W with 8 x 8 patches
    int H, W;                  // grid of the raster order
    const float* kv_logw;      // may be null: additive logit shift per list entry [BH, nb, nb]
};
hipError_t launch_attn_bf16(const AttnArgs& a, hipStream_t s);
hipError_t launch_attn_f32(const AttnArgs& a, hipStream_t s);

// Start order of the mask step's schedule output: pairs of query blocks of neighbouring
// frames, heads in turn, each head's pairs by decreasing combined count (mask.hip).
hipError_t launch_pair_schedule(const MaskArgs& a, const int32_t* counts, int32_t* schedule, hipStream_t s);

// Start order of BH*nb items, heads in turn, each head's items by decreasing count.
hipError_t launch_schedule(const int32_t* counts, int BH, int nb, int32_t* schedule, hipStream_t s);

struct AttnBwdArgs {
    const void* q;
    const void* k;
    const void* v;
    const void* o;
    const void* dout;
    const float* lse;          // [BH, L], natural log
    void* dq;
    void* dk;
    void* dv;
    int BH, L, nb, d;
    const int32_t* kv_count;
    const int32_t* kv_index;
    float scale;
    int bf16;
    int raster;                // 0: blocks are runs of 64 rows; 1: raster T x H x W with 8 x 8 patches
    int H, W;                  // grid of the raster order
    // workspace
    float* drow;               // [BH, L]   rowsum(dO * O)
    uint32_t* bits;            // [BH, nb, ceil(nb/32)]  transposed mask
    int32_t* q_count;          // [BH, nb]
    int32_t* q_index;          // [BH, nb, nb]
    int32_t* sched_q;          // [BH * nb]  start order of the dQ sweep
    int32_t* sched_k;          // [BH * nb]  start order of the dK/dV sweep
};
hipError_t launch_attn_bwd(const AttnBwdArgs& a, hipStream_t s);

}  // namespace nabla
