// gfx950 measurement kernels beside the library's read probe: the vector
// attention kernel's K/V tile stream with none of its arithmetic, so its
// HBM rate (and, kept in L2, its per-CU rate) can be set beside the
// kernels that carry that stream.
#include <hip/hip_runtime.h>

#include <cstdint>

#include "vrt_internal.h"

namespace vrt {
namespace {

// 16 bytes per lane, memory -> LDS (global_load_lds_dwordx4: lane i writes
// bytes [16i, 16i + 16) after the wave-uniform LDS address in M0), through
// inline asm as in the attention kernels: every read of a stage is ordered
// after its DMA by a vmcnt wait and a workgroup barrier.  M0 is saved and
// restored around the instruction, with the one wait state an M0 write needs
// before an LDS DMA.  NT: the non-temporal hint the vector attention kernel
// gives its tile loads; without it, plain loads as the GEMMs use.
template <bool NT>
__device__ __forceinline__ void dma16_hint(const char* g, char* l) {
    const unsigned lds = __builtin_amdgcn_readfirstlane((unsigned)(__UINTPTR_TYPE__)l);
    unsigned saved;
    if constexpr (NT) {
        asm volatile(
            "s_mov_b32 %0, m0\n\t"
            "s_mov_b32 m0, %2\n\t"
            "s_nop 0\n\t"
            "global_load_lds_dwordx4 %1, off nt\n\t"
            "s_mov_b32 m0, %0"
            : "=&s"(saved)
            : "v"((unsigned long long)(__UINTPTR_TYPE__)g), "s"(lds)
            : "memory");
    } else {
        asm volatile(
            "s_mov_b32 %0, m0\n\t"
            "s_mov_b32 m0, %2\n\t"
            "s_nop 0\n\t"
            "global_load_lds_dwordx4 %1, off\n\t"
            "s_mov_b32 m0, %0"
            : "=&s"(saved)
            : "v"((unsigned long long)(__UINTPTR_TYPE__)g), "s"(lds)
            : "memory");
    }
}
// wait until no vector-memory operation of this wave is outstanding
__device__ __forceinline__ void wait_vm0() {
    __builtin_amdgcn_s_waitcnt((0x7 << 4) | (0xF << 8));
}

// ------------------------------------------------ tile-stream probe ----
// Measurement only: the vector attention kernel's tile stream with no
// arithmetic.  Workgroup w takes regions (w heads + h) mod n_regions for
// h < heads; from each it reads `tiles` consecutive 8 KB K tiles and the 8 KB
// V tiles kv_off bytes further on, a 16 KB tile at a time, through two LDS
// stages with one workgroup barrier per tile and the same DMA
// (global_load_lds_dwordx4, with that kernel's non-temporal hint when NT),
// `passes` times over.  The first tile of a region is read from row row_lo
// and the last up to row row_hi; rows outside fetch the nearest row read, as
// the attention kernel's edge tiles do (row_lo 0, row_hi 63: whole tiles).
template <bool NT>
__global__ __launch_bounds__(256) void k_tile_probe(const char* __restrict__ buf, long long region_stride,
                                                    long long kv_off, int n_regions, int heads, int tiles,
                                                    int passes, int row_lo, int row_hi, unsigned magic,
                                                    unsigned* sink) {
    __shared__ __attribute__((aligned(16))) char lds[2 * 16384];
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int lane = threadIdx.x & 63;
    const int ntt = heads * tiles;
    // the next tile to issue: region `reg`, tile `it` of it (advanced by
    // counters, so a tile's issue is a few scalar adds)
    const int r0 = (int)(((long long)blockIdx.x * heads) % n_regions);
    int reg = r0, it = 0;
    // the lane's 16-byte chunk: row wave * 16 + lane / 8 (+ 8 in the second
    // instruction) of the 64-row tile, chunk lane % 8 of the 128-byte row
    const int row0 = wave * 16 + (lane >> 3);
    const char* lane_k = buf + (lane & 7) * 16;
    auto issue = [&](int st) {
        const char* k = lane_k + (long long)reg * region_stride + (long long)it * 8192;
        char* l = lds + st * 16384 + wave * 2 * 1024;
        const int rlo = it == 0 ? row_lo : 0, rhi = it == tiles - 1 ? row_hi : 63;
#pragma unroll
        for (int i = 0; i < 2; ++i) {   // 8 instructions of 1 KB per half tile, 2 per wave
            const int rr = min(max(row0 + 8 * i, rlo), rhi);   // 0 <= rr <= 63
            dma16_hint<NT>(k + rr * 128, l + i * 1024);
            dma16_hint<NT>(k + kv_off + rr * 128, l + 8192 + i * 1024);
        }
        if (++it == tiles) {
            it = 0;
            if (++reg == n_regions) reg = 0;
        }
    };
    for (int p = 0; p < passes; ++p) {
        reg = r0;
        it = 0;
        issue(0);
        for (int T = 0; T < ntt; ++T) {
            wait_vm0();
            __syncthreads();   // tile T landed for every wave; the other stage is free
            if (T + 1 < ntt) issue((T + 1) & 1);
        }
    }
    if (*(const unsigned*)(lds + 4 * threadIdx.x) == magic) sink[0] = 1u;
}

}  // namespace

hipError_t launch_tile_probe(const char* buf, long long region_stride, long long kv_off, int n_regions, int n_wg,
                             int heads, int tiles, int passes, int row_lo, int row_hi, bool nt, unsigned* sink,
                             hipStream_t s) {
    if (nt)
        VRT_LAUNCH(k_tile_probe<true>, dim3((unsigned)n_wg), dim3(256), 0, s, buf, region_stride, kv_off, n_regions,
                   heads, tiles, passes, row_lo, row_hi, 0x9e3779b9u, sink);
    else
        VRT_LAUNCH(k_tile_probe<false>, dim3((unsigned)n_wg), dim3(256), 0, s, buf, region_stride, kv_off, n_regions,
                   heads, tiles, passes, row_lo, row_hi, 0x9e3779b9u, sink);
    return hipSuccess;
}

}  // namespace vrt
