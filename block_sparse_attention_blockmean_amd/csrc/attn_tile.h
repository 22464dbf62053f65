// Tile machinery shared by the bf16 attention kernels (forward and gradient): MFMA
// operand types, the swizzled LDS layout of a 64-token tile, the buffer form of the
// LDS DMA that fills it, and the waits and barrier that hand tiles between waves.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace nabla {
namespace attn {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef __attribute__((address_space(3))) void lds_void;
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;

constexpr int kBlk = 64;
constexpr int kWaves = 4;             // waves per workgroup
constexpr int kThreads = 64 * kWaves;
// Third dword of a raw buffer resource on gfx9-family GPUs: 32-bit data format, no
// swizzle, no stride.
constexpr int kBufferFlags = 0x00020000;

template <int D>
struct Tile {
    static constexpr int kRowBytes = 2 * D;             // one token row of K or V
    static constexpr int kChunks = D / 8;               // 16-byte chunks per row
    static constexpr int kRowsPerLine = 256 / kRowBytes;  // rows per 256-byte LDS bank line
    static constexpr int kBytes = kBlk * kRowBytes;
    static constexpr int kCopiesPerWave = kBytes / 1024 / kWaves;  // 1 KiB per copy
    // K is read 16 bytes per lane from 16 consecutive rows at one chunk: spread the
    // rows over all chunk slots of a bank line.
    __device__ static inline int k_swz(int row) { return (row / kRowsPerLine) & (kChunks - 1); }
    // V is read 8 bytes per lane, 4 rows x 64 bytes per 16 lanes: spread groups of
    // 4 chunks over the bank line.
    __device__ static inline int v_swz(int row) { return 4 * ((row / kRowsPerLine) & (kChunks / 4 - 1)); }
};

// Copy u of wave w fills bytes [1024 (4u + w), +1024) of the LDS tile, 16 bytes per lane
// in lane order; the lane fetches the global chunk that belongs in that slot under the
// swizzle.  Copy u covers rows 4 KiB further down than copy u - 1 and the swizzle of a
// row depends only on its position within 16 rows (d = 128) or 32 rows (d = 64), which
// copy u shares with copy 0, so the lane part is that of copy 0 and u adds 4 KiB.
template <int D, bool kIsV>
__device__ inline uint32_t copy_lane_offset(int wave, int lane) {
    using G = Tile<D>;
    const int o = wave * 1024 + lane * 16;
    const int row = o / G::kRowBytes;
    const int slot = (o % G::kRowBytes) / 16;
    const int chunk = slot ^ (kIsV ? G::v_swz(row) : G::k_swz(row));
    return (uint32_t)(row * G::kRowBytes + chunk * 16);
}

// The wave's share of one tile copy (buffer form of the LDS DMA: uniform tile offset in
// soffset, 32-bit lane offset, uniform LDS destination in M0; offsets past the buffer
// read zeros).
template <int D>
__device__ inline void copy_tile(__amdgpu_buffer_rsrc_t rsrc, uint32_t tile_byte, char* lds_tile, int wave,
                                 uint32_t lane_off) {
    using G = Tile<D>;
#pragma unroll
    for (int u = 0; u < G::kCopiesPerWave; ++u)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, (lds_void*)(lds_tile + (4 * u + wave) * 1024), 16,
                                                 lane_off, tile_byte + u * 4096, 0, 0);
}

// s_waitcnt vmcnt(N) through the builtin, which the compiler's own wait accounting
// understands (an asm wait would leave it assuming the copies are still pending).
// gfx9 encoding: vmcnt in bits 3:0 and 15:14, expcnt 6:4 and lgkmcnt 11:8 left at their
// maxima (no wait).
template <int N>
__device__ inline void wait_vmcnt() {
    static_assert(N >= 0 && N < 64, "vmcnt is 6 bits");
    __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (0x7 << 4) | (0xf << 8));
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

}  // namespace attn
}  // namespace nabla
