// Device helpers shared by the attention kernels (vrt_kernels.hip, vrt_mfma.hip):
// typed global loads and stores, bf16 conversions, the NEOX rotation of keys
// and queries, the HBM -> LDS tile DMA and its waits.  Internal; each
// translation unit gets its own copies.
#pragma once

#include <hip/hip_runtime.h>

#include "vrt_internal.h"

namespace vrt {
namespace {


typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

struct F32T { static constexpr int E = 4; };
struct BF16T { static constexpr int E = 2; };

// Global-memory accesses go through address-space-1 pointers: the ring and
// I/O addresses arrive as integers in the kernel arguments, and through a
// generic pointer the compiler would emit flat loads, which also count on the
// LDS wait counter and so make every LDS wait in the tile loop wait for the
// next tiles' HBM loads too.
#define VRT_GLOBAL __attribute__((address_space(1)))
template <int B> struct Raw;
template <> struct Raw<2> { typedef unsigned short T; };
template <> struct Raw<4> { typedef unsigned int T; };
template <> struct Raw<8> { typedef unsigned int T __attribute__((ext_vector_type(2))); };
template <> struct Raw<16> { typedef unsigned int T __attribute__((ext_vector_type(4))); };
template <class T>
__device__ __forceinline__ T gld(const void* p) {
    typedef typename Raw<sizeof(T)>::T R;
    const R r = *(const VRT_GLOBAL R*)(__UINTPTR_TYPE__)p;
    return __builtin_bit_cast(T, r);
}
template <class T>
__device__ __forceinline__ void gst(void* p, T v) {
    typedef typename Raw<sizeof(T)>::T R;
    *(VRT_GLOBAL R*)(__UINTPTR_TYPE__)p = __builtin_bit_cast(R, v);
}
// A store with the non-temporal hint.  The vector attention kernel writes the
// rows it appends this way: it reads them back through its own tile stream,
// and on the 256-stream serving step ordinary stores of those 5 MB of rows
// made the launch 6 % slower.  Its split-K partials too: with ordinary stores
// the 32-stream x 26-layer decode step took 5.7 % longer.  The separate append kernel and the compaction
// copy keep ordinary stores: the attention launch right after them reads
// their rows, and the hint made that catch-up step 2-3 % slower.  Ordering and
// visibility are those of any other store.
template <class T>
__device__ __forceinline__ void gst_nt(void* p, T v) {
    typedef typename Raw<sizeof(T)>::T R;
    __builtin_nontemporal_store(__builtin_bit_cast(R, v), (VRT_GLOBAL R*)(__UINTPTR_TYPE__)p);
}

__device__ __forceinline__ float bf_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// float -> bfloat16 bits, round to nearest even (NaN stays NaN).
__device__ __forceinline__ uint32_t to_bf16(float f) {
    uint32_t u = __float_as_uint(f);
    if ((u & 0x7fffffffu) > 0x7f800000u) return 0x7fc0u;
    u += 0x7fffu + ((u >> 16) & 1u);
    return u >> 16;
}

__device__ __forceinline__ float dot2bf(uint32_t a, uint32_t b, float c) {
    return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a),
                                           __builtin_bit_cast(bf16x2_t, b), c, false);
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

__device__ __forceinline__ long long floor_div(long long a, long long b) {
    long long q = a / b;
    return (a % b != 0 && (a < 0)) ? q - 1 : q;
}

// ---------------------------------------------------------------- RoPE ----
// angle = pos * omega_i in fp64 (a float32 angle is off by up to ~0.03 rad at
// positions near 1e6); omega_i = theta^(-2i/D) comes from the host in fp64.
// The angle is first reduced by multiples of 2*pi with the additive method of
// Cody and Waite (1980): 2*pi is split into three doubles, the first two with
// 30 significant bits, so k*c1 and k*c2 are exact for |k| < 2^23 and the three
// fused steps leave the reduced angle accurate to about one ulp.  sincos then
// runs on an argument in [-pi, pi]; beyond |x| = 2.6e7 the library reduces it.
__device__ __forceinline__ void rope_angle(long long pos, double omega, double* c, double* s) {
    double x = (double)pos * omega;
    if (fabs(x) < 2.6e7) {
        const double k = rint(x * 0.15915494309189535);  // x / (2 pi), nearest integer
        x = fma(-k, 6.283185303211212, x);
        x = fma(-k, 3.9683743166540886e-09, x);
        x = fma(-k, 2.068073192717642e-18, x);
    }
    sincos(x, s, c);
}

// NEOX pair (i, i + D/2): y0 = x0 cos - x1 sin, y1 = x1 cos + x0 sin, in fp64,
// rounded once to fp32.
__device__ __forceinline__ void rope_rot(float x0, float x1, double c, double s, float* y0,
                                         float* y1) {
    const double a = (double)x0 * c;
    const double b = (double)x1 * s;
    const double e = (double)x1 * c;
    const double f = (double)x0 * s;
    *y0 = (float)(a - b);
    *y1 = (float)(e + f);
}

// (cos, sin) of a rotation angle x = p * omega_i, 0 <= p < 2^31.  The
// fp64 angle is reduced by 2 pi with a four-part Cody-Waite split whose first
// three parts have 24 significant bits, so k * c_j is exact for |k| < 2^29
// (every angle below 3.3e9 rad, which covers all positions the library
// accepts) and the reduced angle is accurate to about 1e-15 rad; the
// hardware sine / cosine then run on it in revolutions (1.2e-7 abs. error).
struct CosSin { float c, s; };
__device__ __forceinline__ CosSin rope_cs(double x) {
    const double k = rint(x * 0x1.45f306dc9c883p-3);      // x / (2 pi)
    x = fma(-k, 0x1.921fb60000000p+2, x);
    x = fma(-k, -0x1.777a5c0000000p-23, x);
    x = fma(-k, -0x1.ee59da0000000p-48, x);
    x = fma(-k, 0x1.98a2e03707345p-75, x);
    const float r = (float)(x * 0x1.45f306dc9c883p-3);
    return CosSin{__builtin_amdgcn_cosf(r), __builtin_amdgcn_sinf(r)};
}

// One NEOX rotation per storage type.  fp32 storage: fp64 sin / cos and an
// fp64 rotation rounded once to fp32 (rope_angle, rope_rot).  bf16 storage:
// the exactly reduced angle and the hardware sine / cosine (rope_cs) and an
// fp32 rotation; its error (~1e-7 of the values) is far below the bf16
// rounding of the result.  Keys are written by one function per storage
// type whichever kernel appends them, so ring contents do not depend on the
// path that wrote them.
template <class E> struct Angle;
template <> struct Angle<F32T> { double c, s; };
template <> struct Angle<BF16T> { float c, s; };
template <class E> __device__ __forceinline__ Angle<E> rope_of(long long pos, double omega);
template <> __device__ __forceinline__ Angle<F32T> rope_of<F32T>(long long pos, double omega) {
    Angle<F32T> a;
    rope_angle(pos, omega, &a.c, &a.s);
    return a;
}
template <> __device__ __forceinline__ Angle<BF16T> rope_of<BF16T>(long long pos, double omega) {
    const CosSin r = rope_cs((double)pos * omega);
    return Angle<BF16T>{r.c, r.s};
}
__device__ __forceinline__ void rope_pair(float x0, float x1, Angle<F32T> a, float* y0, float* y1) {
    rope_rot(x0, x1, a.c, a.s, y0, y1);
}
__device__ __forceinline__ void rope_pair(float x0, float x1, Angle<BF16T> a, float* y0, float* y1) {
    *y0 = __fmaf_rn(x0, a.c, -(x1 * a.s));
    *y1 = __fmaf_rn(x1, a.c, x0 * a.s);
}

template <class E> __device__ __forceinline__ void ld4(const char* p, float (&x)[4]);
template <> __device__ __forceinline__ void ld4<F32T>(const char* p, float (&x)[4]) {
    const float4 v = gld<float4>(p);
    x[0] = v.x; x[1] = v.y; x[2] = v.z; x[3] = v.w;
}
template <> __device__ __forceinline__ void ld4<BF16T>(const char* p, float (&x)[4]) {
    const uint2 v = gld<uint2>(p);
    x[0] = bf_lo(v.x); x[1] = bf_hi(v.x); x[2] = bf_lo(v.y); x[3] = bf_hi(v.y);
}
// Four consecutive elements in the storage type; G: global memory, else LDS.
template <class E, bool G> __device__ __forceinline__ void st4(char* p, const float (&x)[4]);
template <> __device__ __forceinline__ void st4<F32T, true>(char* p, const float (&x)[4]) {
    gst<float4>(p, make_float4(x[0], x[1], x[2], x[3]));
}
template <> __device__ __forceinline__ void st4<F32T, false>(char* p, const float (&x)[4]) {
    *(float4*)p = make_float4(x[0], x[1], x[2], x[3]);
}
__device__ __forceinline__ uint2 pack_bf16x4(const float (&x)[4]) {
    uint2 v;
    v.x = to_bf16(x[0]) | (to_bf16(x[1]) << 16);
    v.y = to_bf16(x[2]) | (to_bf16(x[3]) << 16);
    return v;
}
template <> __device__ __forceinline__ void st4<BF16T, true>(char* p, const float (&x)[4]) {
    gst<uint2>(p, pack_bf16x4(x));
}
template <> __device__ __forceinline__ void st4<BF16T, false>(char* p, const float (&x)[4]) {
    *(uint2*)p = pack_bf16x4(x);
}
// Four consecutive elements in the storage type, stored with gst_nt.
template <class E> __device__ __forceinline__ void st4_ring(char* p, const float (&x)[4]);
template <> __device__ __forceinline__ void st4_ring<F32T>(char* p, const float (&x)[4]) {
    gst_nt<float4>(p, make_float4(x[0], x[1], x[2], x[3]));
}
template <> __device__ __forceinline__ void st4_ring<BF16T>(char* p, const float (&x)[4]) {
    gst_nt<uint2>(p, pack_bf16x4(x));
}

template <int CPR>
__device__ __forceinline__ int ksw(int r) { return CPR == 8 ? ((r >> 1) & 7) : (r & 15); }
// V rows: a transposing read covers 4 consecutive rows; XOR the chunk index so
// those 4 rows fall on distinct banks (128-byte rows pair up as r, r+2; 256-byte
// rows all start on bank 0).
template <class E, int CPR>
__device__ __forceinline__ int vsw(int r) {
    if constexpr (E::E == 4) return 0;
    return CPR == 8 ? (((r >> 1) & 1) << 2) : ((r & 3) << 2);
}

typedef short v4i16 __attribute__((ext_vector_type(4)));
#define VRT_LDS __attribute__((address_space(3)))

// 16 bytes per lane, HBM -> LDS (global_load_lds_dwordx4: lane i writes
// bytes [16i, 16i + 16) after the wave-uniform LDS address in M0).  Issued
// through inline asm on purpose: the compiler does not track LDS writes
// made this way, so it does not make every later LDS read of the tile loop
// wait for the DMA of the tile being prefetched.  Every read of a stage is
// ordered after its DMA explicitly (wait_vm, then a workgroup barrier).
// Untracked vector-memory operations can only make the compiler's own
// vmcnt waits stricter, never weaker.
// M0 is saved and restored around the instruction (the compiler reserves
// it), with the one wait state an M0 write needs before an LDS DMA.
// The loads carry the non-temporal hint: the vector kernel reads each window
// row once per launch, and streaming them past the caches' retention raised
// the serving step from 66.8 % to 69.9 % and the decode step from 68.3 % to
// 76.1 % of peak HBM bandwidth (measured back to back on one MI355X).
__device__ __forceinline__ void dma16(const char* g, char* l) {
    const unsigned lds = __builtin_amdgcn_readfirstlane((unsigned)(__UINTPTR_TYPE__)l);
    unsigned saved;
    asm volatile(
        "s_mov_b32 %0, m0\n\t"
        "s_mov_b32 m0, %2\n\t"
        "s_nop 0\n\t"
        "global_load_lds_dwordx4 %1, off nt\n\t"
        "s_mov_b32 m0, %0"
        : "=&s"(saved)
        : "v"((unsigned long long)(__UINTPTR_TYPE__)g), "s"(lds)
        : "memory");
}
// The same with a wave-uniform 64-bit base in SGPRs and a 32-bit per-lane
// byte offset (global_load_lds with saddr): no 64-bit address per lane.
__device__ __forceinline__ void dma16s(const char* base, unsigned off, char* l) {
    const unsigned lds = __builtin_amdgcn_readfirstlane((unsigned)(__UINTPTR_TYPE__)l);
    unsigned saved;
    asm volatile(
        "s_mov_b32 %0, m0\n\t"
        "s_mov_b32 m0, %3\n\t"
        "s_nop 0\n\t"
        "global_load_lds_dwordx4 %1, %2\n\t"
        "s_mov_b32 m0, %0"
        : "=&s"(saved)
        : "v"(off), "s"(base), "s"(lds)
        : "memory");
}
// lane id read through volatile asm: recomputed where used instead of being
// kept live (or spilled) across a loop
__device__ __forceinline__ int lane_id_v() {
    int l;
    asm volatile("v_mbcnt_lo_u32_b32 %0, -1, 0\n\tv_mbcnt_hi_u32_b32 %0, -1, %0" : "=v"(l));
    return l;
}
// wait until at most N vector-memory operations of this wave are outstanding
template <int N>
__device__ __forceinline__ void wait_vm() {
    static_assert(N >= 0 && N < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((N & 0xF) | ((N >> 4) << 14) | (0x7 << 4) | (0xF << 8));
}

}  // namespace
}  // namespace vrt
