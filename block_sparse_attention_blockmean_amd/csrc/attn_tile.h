// Tile machinery shared by the bf16 attention kernels (forward and gradient): MFMA
// operand types, the swizzled LDS layout of a 64-token tile, the buffer form of the
// LDS DMA that fills it, and the waits and barrier that hand tiles between waves.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "nabla_internal.h"

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
    static_assert(kChunks == 16 || kChunks == 8, "d = 128 or 64");
    // Tiles read as rows (16 bytes per lane, 16 consecutive rows at one chunk) and, in
    // the gradient kernels, also through the transposing read (8 bytes per lane; each
    // 32 lanes cover 4 consecutive rows, aligned to 4, times 4 consecutive chunks from a
    // multiple of 4).  The swizzle is an XOR with a bijection f of the row's position in
    // 16 bank lines: row reads need f one-to-one there; the transposing read needs the
    // rows sharing a bank line to differ in f's top bits, so that their 4-chunk groups
    // land apart.  d = 128 (one row per bank line): f = rows' bits 1:0 above bits 3:2.
    // d = 64 (two rows per line, 8 chunks): f = line bit 0 above line bits 2:1.
    __device__ static inline int k_swz(int row) {
        const int line = row / kRowsPerLine;
        if constexpr (kChunks == 16) return ((line & 3) << 2) | ((line >> 2) & 3);
        else return ((line & 1) << 2) | ((line >> 1) & 3);
    }
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

// Where the 64 tokens of block b sit in a [L, D] head.
//   Fractal order: block b is rows [64 b, 64 b + 64).
//   Raster order with 8 x 8 patches (one patch per block): block b is patch
//   (t, ph, pw) = (b / nHW, (b % nHW) / nW, b % nW), and its row r is raster token
//   t HW + (8 ph + r / 8) W + 8 pw + r % 8 - eight runs of eight consecutive tokens.
struct RasterGrid {
    uint32_t W, HW;       // tokens per raster row, per frame
    FastDiv nHW, nW;      // patches per frame, per patch row
};

template <bool RASTER>
__device__ inline uint32_t block_row(const RasterGrid& g, uint32_t b) {
    if (!RASTER) return b * kBlk;
    uint32_t t, rem, ph, pw;
    g.nHW.divmod(b, t, rem);
    g.nW.divmod(rem, ph, pw);
    return t * g.HW + 8 * (ph * g.W + pw);
}

template <bool RASTER>
__device__ inline uint32_t row_in_block(const RasterGrid& g, int r) {
    return RASTER ? (uint32_t)((r >> 3) * g.W + (r & 7)) : (uint32_t)r;
}

// Byte distance in the head between copy u and copy u + 1 of a tile: 4 KiB of rows,
// which in raster order is 4096 / (2 D) / 8 patch rows, 512 W bytes for any D.
template <bool RASTER>
__device__ inline uint32_t copy_stride(const RasterGrid& g) {
    return RASTER ? 512u * g.W : 4096u;
}

// copy_lane_offset for either token order (the swizzle is that of the LDS row).
template <int D, bool kIsV, bool RASTER>
__device__ inline uint32_t copy_lane_offset_in(const RasterGrid& g, int wave, int lane) {
    using G = Tile<D>;
    const int o = wave * 1024 + lane * 16;
    const int row = o / G::kRowBytes;
    const int slot = (o % G::kRowBytes) / 16;
    const int chunk = slot ^ (kIsV ? G::v_swz(row) : G::k_swz(row));
    return row_in_block<RASTER>(g, row) * G::kRowBytes + chunk * 16;
}

// The wave's share of one tile copy (buffer form of the LDS DMA: uniform tile offset in
// soffset, 32-bit lane offset, uniform LDS destination in M0; offsets past the buffer
// read zeros).  `stride` is the byte distance between consecutive 4 KiB copies.
template <int D>
__device__ inline void copy_tile(__amdgpu_buffer_rsrc_t rsrc, uint32_t tile_byte, char* lds_tile, int wave,
                                 uint32_t lane_off, uint32_t stride = 4096) {
    using G = Tile<D>;
#pragma unroll
    for (int u = 0; u < G::kCopiesPerWave; ++u)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, (lds_void*)(lds_tile + (4 * u + wave) * 1024), 16,
                                                 lane_off, tile_byte + u * stride, 0, 0);
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
