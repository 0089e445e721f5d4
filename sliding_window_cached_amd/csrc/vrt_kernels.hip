// gfx950 kernels for streamed windowed-causal attention.
//
//   k_rope_append  NEOX RoPE (theta^(-2i/d) frequencies, angle formed in fp64) of the
//                  new keys, then the rotated keys and the raw values are
//                  written to their ring slots (Voxtral Realtime streaming-plan
//                  page, "SHIPPED" section: the chunk's K/V go to rows
//                  [n_kv_before, n_kv_total); family doc, Streaming row item 5:
//                  decoder token cur goes to slot cur % n_ctx).
//   k_compact      copies the last `kept` rows of a ring slice to its front
//                  (streaming-plan page, "Unbounded length": compact_enc_ring).
//                  Source and destination may overlap; every chunk is staged
//                  through LDS before any of it is written back.
//   k_attn         windowed-causal attention, fp32 accumulation: a query at
//                  absolute position p sees keys in (p - W, p].  Keys are
//                  visited in 64-key tiles that start at multiples of 64 in
//                  absolute position, in ascending order; keys outside a
//                  query's window get probability exactly 0 and tiles with no
//                  key for a query are exact no-ops for it, so a query's
//                  result does not depend on which other queries share its
//                  workgroup, on ring slots or on compaction: chunked feeding
//                  reproduces the offline pass bit for bit.
//   k_attn_mfma    the same attention for sub-batches of 32 or more bf16
//                  frames (the catch-up path), with both products on the
//                  matrix cores and the same absolute tile grid.
//   k_dec_combine  log-sum-exp merge of split-K partials in ascending split
//                  order (decode step).
//
// Numerics: -ffp-contract=off for the whole library; every fused multiply-add
// below is written out.  bf16 storage: q, k, v and the softmax weights enter
// the dot products as bf16 (v_dot2_f32_bf16, fp32 accumulate); fp32 storage
// keeps everything in fp32.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <mutex>

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

// ---------------------------------------------------------- K1: append ----
// One workgroup per (unit, group of 4 frames).  Each thread rotates 4 NEOX
// pairs of one (frame, kv head) row; the angles of the workgroup's frames are
// computed once into LDS and shared by all heads.
template <class E, int D, bool MOD>
__global__ __launch_bounds__(256) void k_rope_append(AppendArgs a, StateTable t) {
    constexpr int FR = 4, H2 = D / 2, CG = H2 / 4, VCH = D * E::E / 16;
    __shared__ Angle<E> cs[FR * H2];
    const UnitMap& m = a.m;
    const int nfb = (m.n + FR - 1) / FR;
    const int unit = blockIdx.x / nfb, fb = blockIdx.x - unit * nfb;
    const int si = unit / m.nl, li = unit - si * m.nl;
    const long long p0 = t.p0[si];
    const int nkv = t.n_kv[si];
    const int f0 = fb * FR, nf = min(FR, m.n - f0);
    for (int x = threadIdx.x; x < nf * H2; x += blockDim.x) {
        const int f = x / H2, i = x - f * H2;
        if (a.g.rope) cs[x] = rope_of<E>(p0 + f0 + f, a.g.omega[i]);
    }
    __syncthreads();
    const int hkv = a.g.hkv;
    const long long cu = (long long)t.call_idx[si] * m.nl_call + m.l_off + li;
    // input rows hold Dio elements per head; ring rows D (a head narrower than
    // 64, only without rotation, is stored zero-padded)
    const int Dio = a.g.Dio;
    const long long row_elems = (long long)hkv * Dio;
    const long long in0 = (cu * m.n_total + m.t0 + f0) * row_elems * E::E;
    const char* kin = (const char*)a.k + in0;
    const char* vin = (const char*)a.v + in0;
    char* layer = (char*)t.ring[si] + (long long)(m.layer0 + m.l_off + li) * a.g.layer_bytes;
    for (int x = threadIdx.x; x < nf * hkv * CG; x += blockDim.x) {
        const int c = x % CG, fh = x / CG, h = fh % hkv, f = fh / hkv;
        const long long pos = p0 + f0 + f;
        const long long slot = MOD ? (pos % a.g.slots) : (long long)(nkv + f0 + f);
        const char* src = kin + ((long long)f * row_elems + (long long)h * Dio) * E::E;
        float x0[4] = {0.f, 0.f, 0.f, 0.f}, x1[4] = {0.f, 0.f, 0.f, 0.f}, y0[4], y1[4];
        if (4 * c < Dio) ld4<E>(src + 4 * c * E::E, x0);
        if (H2 + 4 * c < Dio) ld4<E>(src + (H2 + 4 * c) * E::E, x1);
        if (a.g.rope) {
#pragma unroll
            for (int q = 0; q < 4; ++q) rope_pair(x0[q], x1[q], cs[f * H2 + 4 * c + q], &y0[q], &y1[q]);
        } else {
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                y0[q] = x0[q];
                y1[q] = x1[q];
            }
        }
        char* dst = layer + (long long)h * a.g.slice_bytes + slot * (D * E::E);
        st4<E, true>(dst + 4 * c * E::E, y0);
        st4<E, true>(dst + (H2 + 4 * c) * E::E, y1);
    }
    for (int x = threadIdx.x; x < nf * hkv * VCH; x += blockDim.x) {
        const int c = x % VCH, fh = x / VCH, h = fh % hkv, f = fh / hkv;
        const long long pos = p0 + f0 + f;
        const long long slot = MOD ? (pos % a.g.slots) : (long long)(nkv + f0 + f);
        const uint4 val = 16 * c < Dio * E::E
                              ? gld<uint4>(vin + ((long long)f * row_elems + (long long)h * Dio) * E::E + 16 * c)
                              : make_uint4(0u, 0u, 0u, 0u);
        gst<uint4>(layer + a.g.v_off + (long long)h * a.g.slice_bytes + slot * (D * E::E) + 16 * c,
                   val);
    }
}

// --------------------------------------------------------- K2: compact ----
// One workgroup per (entry, kv head, K|V).  Rows [shift, shift + kept) move to
// [0, kept) in ascending chunks; each chunk is read completely into LDS (the
// barrier waits for every load, since the LDS stores consume them) before any
// row of it is written, and a later chunk's source never overlaps an earlier
// chunk's destination (destination < source), so overlap is safe.
template <class E, int D>
__global__ __launch_bounds__(256) void k_compact(CompactArgs a, CompactTable t) {
    constexpr int ROWB = D * E::E;
    constexpr int CHUNK = 16384 / ROWB;  // rows per 16 KB chunk
    __shared__ uint4 stage[16384 / 16];
    const int b = blockIdx.x;
    const int which = b & 1;
    const int rest = b >> 1;
    const int h = rest % a.g.hkv, e = rest / a.g.hkv;
    char* base = (char*)t.layer_ring[e] + (which ? a.g.v_off : 0) + (long long)h * a.g.slice_bytes;
    const char* src = base + (long long)t.shift[e] * ROWB;
    for (int r0 = 0; r0 < a.kept; r0 += CHUNK) {
        const int nr = min(CHUNK, a.kept - r0);
        const int n16 = nr * ROWB / 16;
        for (int x = threadIdx.x; x < n16; x += blockDim.x)
            stage[x] = gld<uint4>(src + (long long)r0 * ROWB + 16LL * x);
        __syncthreads();
        for (int x = threadIdx.x; x < n16; x += blockDim.x)
            gst<uint4>(base + (long long)r0 * ROWB + 16LL * x, stage[x]);
        __syncthreads();
    }
}

// Wave-wide reductions: xor-butterfly inside each row of 16 lanes with DPP
// (quad_perm [1,0,3,2], quad_perm [2,3,0,1], row_half_mirror, row_mirror; with
// every quad / half-row already holding one value the mirrors act as xor 4 /
// xor 8), then the four row results combined as (r0 + r1) + (r2 + r3) from
// readlane.  Each step combines the same two values on both partner lanes,
// so every lane ends with bit-identical results.
template <int CTRL>
__device__ __forceinline__ float dpp(float v) {
    return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), CTRL, 0xf, 0xf, false));
}
__device__ __forceinline__ float row_max16(float v) {
    v = fmaxf(v, dpp<0xB1>(v));
    v = fmaxf(v, dpp<0x4E>(v));
    v = fmaxf(v, dpp<0x141>(v));
    v = fmaxf(v, dpp<0x140>(v));
    return v;
}
__device__ __forceinline__ float row_sum16(float v) {
    v = v + dpp<0xB1>(v);
    v = v + dpp<0x4E>(v);
    v = v + dpp<0x141>(v);
    v = v + dpp<0x140>(v);
    return v;
}
__device__ __forceinline__ float lane_f(float v, int l) {
    return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), l));
}
__device__ __forceinline__ float wave_max(float v) {
    v = row_max16(v);
    return fmaxf(fmaxf(lane_f(v, 0), lane_f(v, 16)), fmaxf(lane_f(v, 32), lane_f(v, 48)));
}
__device__ __forceinline__ float wave_sum(float v) {
    v = row_sum16(v);
    return (lane_f(v, 0) + lane_f(v, 16)) + (lane_f(v, 32) + lane_f(v, 48));
}

// ------------------------------------------------------ K3: attention ----
// One workgroup of 4 waves per (unit, group of `hg` kv heads, query chunk,
// key split).  For each head of the group its rows are the (query position j,
// q head of the kv group) pairs r = j * group + gh; wave w owns rows w, w + 4,
// ...  Keys are visited in 64-key tiles that start at multiples of 64 in
// absolute position, in ascending order, head after head; the tile stream of
// the whole group runs through one pipeline, so a workgroup fills it once.
// Each tile goes HBM -> LDS directly (global_load_lds_dwordx4: no VGPR
// staging, no transposition), each wave issuing a quarter of it; while tile
// `it` is consumed the next NST-1 tiles are in flight.  Scores are formed with
// lane = key (K rows read as 16-byte chunks, XOR-swizzled so 16 consecutive
// rows hit distinct banks), weights with lane = output dim (V kept row-major
// and read with the gfx950 transposing LDS read, which hands each lane its
// dim for 4 consecutive keys as two bf16 pairs).
//
// Rows of a tile outside the workgroup's key range are fetched from the
// nearest in-range row instead: finite values with weight exactly 0, so no
// zero-fill is needed and uninitialised LDS is never multiplied.
//
// APPEND: the new frames of the call all belong to query chunk 0, so the
// workgroups whose key range ends at the newest frame (chunk 0; in split mode
// the last split) also rotate and write the new K/V rows of their kv heads
// before any tile holding them is read.
template <class E, int D, int NST_>
struct Tl {
    static constexpr int RB = D * E::E;          // bytes per K / V row
    static constexpr int CPR = RB / 16;          // 16-byte chunks per row
    static constexpr int TILE = kTile * RB;      // bytes of one K (or V) tile
    static constexpr int NST = NST_;             // LDS stages (tiles); NST - 1 stream while one is read
    static constexpr int IPW = CPR / 4;          // DMA instructions per wave per K (or V) tile
    static constexpr int LPW = 2 * IPW;          // DMA instructions per wave per tile
    static constexpr int PRB = kTile * E::E;     // bytes of one P row
    static constexpr int QCAP = kQsBytes;        // rotated query rows of the head group
    static constexpr int BYTES = NST * 2 * TILE + QCAP + 4 * PRB;
};
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

// RPW: rows per wave (1 when a head has at most 4 rows; then the wave's query
// row of the current head is kept in registers for that head's key loop).
// LOOK: (left, right) windows without rotation (moonshine streaming encoder):
// the launch answers look_nout queries that lag the newest frame, each seeing
// look_f frames past itself; the oldest look_pend of them come from the q rows
// the state keeps waiting.
template <class E, int D, bool MOD, bool SPLIT, bool APPEND, int RPW, bool LOOK>
__global__ __launch_bounds__(256) void k_attn(AttnArgs a, StateTable t) {
    using L = Tl<E, D, attn_stages(E::E == 2 ? 1 : 0, D, SPLIT)>;
    constexpr int H2 = D / 2, CG = H2 / 4, DPL = D / 64;
    __shared__ __attribute__((aligned(16))) char lds[L::BYTES];
    char* Qs = lds + L::NST * 2 * L::TILE;
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // uniform per wave
    char* Pw = Qs + L::QCAP + wave * L::PRB;

    // Workgroup -> work item.  Workgroups go to the 8 XCDs round robin.
    // Without splits each XCD is given a contiguous run of items (consecutive
    // units, all head groups), so no XCD streams only one head group of every
    // other unit: measured on the 256-stream serving workload, the plain
    // mapping left whole XCDs 15 % slower than others.  With splits the work
    // per unit follows its context length, so contiguous runs would hand the
    // long units to a few XCDs; there the plain order deals the splits of
    // every unit across all XCDs instead.
    int b = blockIdx.x;
    if (!SPLIT) {
        const int nb = gridDim.x, x = blockIdx.x & 7, s8 = blockIdx.x >> 3;
        const int base = nb >> 3, rem = nb & 7;
        b = x < rem ? x * (base + 1) + s8 : rem * (base + 1) + (x - rem) * base + s8;
    }
    const int split = SPLIT ? b % a.n_splits : 0;
    if (SPLIT) b /= a.n_splits;
    const int qc = b % a.n_qchunks;
    b /= a.n_qchunks;
    const int ngb = a.g.hkv / a.hg;
    const int g0 = (b % ngb) * a.hg;          // first kv head of the group
    const int unit = b / ngb;
    const int hg = a.hg;
    const UnitMap& m = a.m;
    const int si = unit / m.nl, li = unit - si * m.nl;
    const long long cu = (long long)t.call_idx[si] * m.nl_call + m.l_off + li;

    const int W = a.g.window, group = a.g.group;
    const long long avail = t.p0[si] - t.n_kv[si];             // abs_base / first position
    const int npend = LOOK ? a.look_pend : 0;                   // queries answered from waiting rows
    const long long pq0 = t.p0[si] - npend + (long long)qc * a.qchunk;  // first query of the chunk
    const int nq = min(a.qchunk, (LOOK ? a.look_nout : m.n) - qc * a.qchunk);
    const int R = nq * group;                                   // rows per head
    const int fut = LOOK ? a.look_f : 0;                        // frames a query sees past itself
    long long wlo = max(avail, pq0 - W + 1);
    long long whi = pq0 + nq - 1;
    if (LOOK) whi = min(t.p0[si] + m.n - 1, whi + fut);         // up to the newest frame written
    bool appender = APPEND && qc == 0;
    if (SPLIT) {
        const long long s_abs = floor_div(wlo, a.split_len) + split;
        if (s_abs > floor_div(whi, a.split_len)) return;  // split past the window: nothing
        appender = appender && s_abs == floor_div(whi, a.split_len);
        wlo = max(wlo, s_abs * a.split_len);
        whi = min(whi, s_abs * a.split_len + a.split_len - 1);
    }

    char* layer = (char*)t.ring[si] + (long long)(m.layer0 + m.l_off + li) * a.g.layer_bytes;
    const long long tfirst = floor_div(wlo, kTile);
    const int nt = (int)(floor_div(whi, kTile) - tfirst + 1);   // tiles per head
    const int ntt = nt * hg;                                    // tiles of the group

    // this wave's quarter of the loads of group tile `T` into stage `st`
    auto issue = [&](int T, int st) {
        const int hh = T / nt, it = T - hh * nt;
        const char* Kg = layer + (long long)(g0 + hh) * a.g.slice_bytes;
        const char* Vg = Kg + a.g.v_off;
        const long long TB = (tfirst + it) * kTile;
        // 0 <= TB < 2^31 (positions are below 2^31), so 32-bit arithmetic is exact
        const long long sb = MOD ? (long long)((unsigned)TB % (unsigned)a.g.slots) : (TB - avail);
        const int rlo = (int)max(0LL, wlo - TB), rhi = (int)min(63LL, whi - TB);
        char* ks = lds + st * 2 * L::TILE;
        char* vs = ks + L::TILE;
#pragma unroll
        for (int i = 0; i < L::IPW; ++i) {
            const int ins = wave * L::IPW + i;         // instruction index within the tile
            const int q = ins * 64 + lane;             // 16-byte chunk this lane fills
            const int r = q / L::CPR, pc = q % L::CPR;
            const int rr = min(max(r, rlo), rhi);
            const long long off = (sb + rr) * L::RB;
            dma16(Kg + off + 16 * (pc ^ ksw<L::CPR>(r)), ks + ins * 1024);
            dma16(Vg + off + 16 * (pc ^ vsw<E, L::CPR>(r)), vs + ins * 1024);
        }
    };
    // a tile holds new rows iff it reaches the first new frame
    auto has_new = [&](int T) {
        const int it = T % nt;
        return APPEND && appender && (tfirst + it) * kTile + kTile - 1 >= t.p0[si];
    };

    // ---- prologue: rotated queries of every head -> Qs (dtype E) and the new
    // K/V rows.  One (head, row, 4-pair group) item per thread, so every input
    // load is independent; each thread's first item is loaded before the tile
    // DMAs go out, so those loads do not queue behind the tiles.
    // io rows: Dio elements per head (= D except for lookahead heads narrower
    // than the 64-element ring rows, whose extra dims are zeros)
    constexpr bool kNarrow = LOOK;
    const int Dio = kNarrow ? a.g.Dio : D;
    const long long qrow = (long long)a.g.hq * Dio;
    const long long krow = (long long)a.g.hkv * Dio;
    const int nkv = t.n_kv[si];
    const int items = hg * R * CG;
    struct Item {
        float x0[4], x1[4], k0[4], k1[4];
        uint4 vch[L::CPR / CG];
    };
    auto load_item = [&](int x, Item& it) {
        const int c = x % CG, r = (x / CG) % R, hh = x / (CG * R);
        const int j = r / group, gh = r - j * group;
        const int g = g0 + hh;
        const int qi = qc * a.qchunk + j;                       // query index in the launch
        const long long frame = m.t0 + (long long)qi - npend;   // its new frame (qi >= npend)
        const char* src;
        if (LOOK && qi < npend)   // a waiting q row of this (state, layer)
            src = (const char*)t.ring[si] + a.pend_off + (long long)(m.layer0 + m.l_off + li) * a.pend_layer +
                  ((long long)qi * qrow + (long long)(g * group + gh) * Dio) * E::E;
        else
            src = (const char*)a.q + ((cu * m.n_total + frame) * qrow + (long long)(g * group + gh) * Dio) * E::E;
        if (!kNarrow || 4 * c < Dio) {
            ld4<E>(src + 4 * c * E::E, it.x0);
        } else {
#pragma unroll
            for (int q = 0; q < 4; ++q) it.x0[q] = 0.f;
        }
        if (!kNarrow || H2 + 4 * c < Dio) {
            ld4<E>(src + (H2 + 4 * c) * E::E, it.x1);
        } else {
#pragma unroll
            for (int q = 0; q < 4; ++q) it.x1[q] = 0.f;
        }
        if (APPEND && !LOOK && appender && gh == 0) {
            const long long kv0 = ((cu * m.n_total + frame) * krow + (long long)g * D) * E::E;
            ld4<E>((const char*)a.k + kv0 + 4 * c * E::E, it.k0);
            ld4<E>((const char*)a.k + kv0 + (H2 + 4 * c) * E::E, it.k1);
#pragma unroll
            for (int u = 0; u < L::CPR / CG; ++u)
                it.vch[u] = gld<uint4>((const char*)a.v + kv0 + 16 * (c + u * CG));
        }
    };
    auto finish_item = [&](int x, const Item& it) {
        const int c = x % CG, r = (x / CG) % R, hh = x / (CG * R);
        const int j = r / group, gh = r - j * group;
        const int g = g0 + hh;
        const long long pos = pq0 + j;
        Angle<E> an[4];
        float y0[4], y1[4];
        if constexpr (LOOK) {   // no rotation
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                y0[q] = it.x0[q];
                y1[q] = it.x1[q];
            }
        } else {
#pragma unroll
            for (int q = 0; q < 4; ++q) an[q] = rope_of<E>(pos, a.g.omega[4 * c + q]);
#pragma unroll
            for (int q = 0; q < 4; ++q) rope_pair(it.x0[q], it.x1[q], an[q], &y0[q], &y1[q]);
        }
        char* dst = Qs + (hh * R + r) * L::RB;
        st4<E, false>(dst + 4 * c * E::E, y0);
        st4<E, false>(dst + (H2 + 4 * c) * E::E, y1);
        if (APPEND && !LOOK && appender && gh == 0) {
            char* Kg = layer + (long long)g * a.g.slice_bytes;
            char* Vg = Kg + a.g.v_off;
            const long long slot = MOD ? (pos % a.g.slots) : (long long)(nkv + j);
#pragma unroll
            for (int q = 0; q < 4; ++q) rope_pair(it.k0[q], it.k1[q], an[q], &y0[q], &y1[q]);
            char* kd = Kg + slot * L::RB;
            st4<E, true>(kd + 4 * c * E::E, y0);
            st4<E, true>(kd + (H2 + 4 * c) * E::E, y1);
#pragma unroll
            for (int u = 0; u < L::CPR / CG; ++u)
                gst<uint4>(Vg + slot * L::RB + 16 * (c + u * CG), it.vch[u]);
        }
    };
    Item first;
    const int x0i = threadIdx.x;
    if (x0i < items) load_item(x0i, first);

    // Tiles without new rows may be fetched before the append: every stage is
    // free at the start, so up to NST tiles go out ahead of the prologue (the
    // rest of the first NST follow the prologue's barrier; tiles with new rows
    // are the last ones of a head, so the ones held back always follow the
    // ones issued, and tiles go out in order).
    constexpr int PRE = L::NST;
    bool pre_done[PRE];
    bool held = false;
#pragma unroll
    for (int st = 0; st < PRE; ++st) {
        held = held || !(st < ntt && !has_new(st));
        pre_done[st] = !held;
        if (pre_done[st]) issue(st, st);
    }

    if (x0i < items) finish_item(x0i, first);
    for (int x = x0i + blockDim.x; x < items; x += blockDim.x) {
        Item more;
        load_item(x, more);
        finish_item(x, more);
    }
    // (left, right) windows: the answered queries lag the new frames, so the
    // new K/V rows (copied unrotated, as the separate append writes them) are
    // their own items
    if constexpr (LOOK && APPEND) {
        if (appender) {
            const int nrow = hg * m.n * L::CPR;
            for (int x = threadIdx.x; x < nrow; x += blockDim.x) {
                const int c = x % L::CPR, f = (x / L::CPR) % m.n, hh = x / (L::CPR * m.n);
                const int g = g0 + hh;
                const long long slot = MOD ? ((t.p0[si] + f) % a.g.slots) : (long long)(nkv + f);
                const long long src = ((cu * m.n_total + m.t0 + f) * krow + (long long)g * Dio) * E::E + 16 * c;
                char* kd = layer + (long long)g * a.g.slice_bytes + slot * L::RB + 16 * c;
                const bool in = 16 * c < Dio * E::E;   // past the io row: the ring row's zero padding
                const uint4 kk = in ? gld<uint4>((const char*)a.k + src) : make_uint4(0u, 0u, 0u, 0u);
                const uint4 vv = in ? gld<uint4>((const char*)a.v + src) : make_uint4(0u, 0u, 0u, 0u);
                gst<uint4>(kd, kk);
                gst<uint4>(kd + a.g.v_off, vv);
            }
        }
    }
    // appended rows visible to every thread's later loads; Qs written
    __syncthreads();
    // the next call's waiting q rows, for this group's heads: one 16-byte
    // column per thread, rows in ascending order (a row is written only after
    // every row it is read from, so the copy is safe in place); the prologue
    // has read the old waiting rows before the barrier
    if constexpr (LOOK) {
        if (a.look_keep > 0 && qc == 0) {
            const long long rowb = (long long)a.g.hq * Dio * E::E;
            const int c0 = g0 * group * Dio * E::E / 16, nc = hg * group * Dio * E::E / 16;
            char* pend = (char*)t.ring[si] + a.pend_off + (long long)(m.layer0 + m.l_off + li) * a.pend_layer;
            const int p = a.look_pend, keep = a.look_keep, shift = p + m.n - keep;
            for (int c = threadIdx.x; c < nc; c += blockDim.x)
                for (int r = 0; r < keep; ++r) {
                    const int src = shift + r;
                    const uint4 v =
                        src < p ? gld<uint4>(pend + src * rowb + 16 * (c0 + c))
                                : gld<uint4>((const char*)a.q + (cu * m.n_total + m.t0 + (src - p)) * rowb +
                                             16 * (c0 + c));
                    gst<uint4>(pend + r * rowb + 16 * (c0 + c), v);
                }
        }
    }
#pragma unroll
    for (int st = 0; st < PRE; ++st)
        if (st < ntt && !pre_done[st]) issue(st, st);

    // ---- per-row state.  The softmax denominator is kept per lane (lane =
    // key position mod 64, rescaled by the row's uniform alpha) and summed
    // across lanes once, after the head's last tile.
    float mrow[RPW], lpart[RPW], acc[RPW][DPL];
    int rlo[RPW], rhi[RPW];                  // row bounds relative to tile 0
    const long long T0 = tfirst * kTile;
#pragma unroll
    for (int i = 0; i < RPW; ++i) {
        const long long pq = pq0 + (wave + 4 * i) / group;
        rlo[i] = (int)(max(wlo, pq - W + 1) - T0);
        rhi[i] = (int)(min(whi, pq + fut) - T0);
    }
    uint4 qreg[RPW == 1 ? L::CPR : 1];

    for (int T = 0; T < ntt; ++T) {
        const int hh = T / nt, it = T - hh * nt;
        if (it == 0) {   // head start: reset the rows, load this head's query row
#pragma unroll
            for (int i = 0; i < RPW; ++i) {
                mrow[i] = kSent;
                lpart[i] = 0.f;
#pragma unroll
                for (int k = 0; k < DPL; ++k) acc[i][k] = 0.f;
            }
            if constexpr (RPW == 1) {
                const char* qr = Qs + (hh * R + min(wave, R - 1)) * L::RB;
#pragma unroll
                for (int c = 0; c < L::CPR; ++c) qreg[c] = *(const uint4*)(qr + 16 * c);
            }
        }
        // Outstanding here: tile T and the tiles issued after it, in order:
        // tiles 1 .. NST-1 when T = 0 (the first NST went out before the
        // loop), else tiles T+1 .. T+NST-2 (tile T+NST-1 goes out only after
        // the barrier frees its stage).
        {
            const int after = T == 0 ? min(L::NST - 1, ntt - 1) : min(L::NST - 2, ntt - 1 - T);
            if constexpr (L::NST >= 4) {
                if (after >= 3) wait_vm<3 * L::LPW>();
                else if (after == 2) wait_vm<2 * L::LPW>();
                else if (after == 1) wait_vm<L::LPW>();
                else wait_vm<0>();
            } else if constexpr (L::NST == 3) {
                if (after >= 2) wait_vm<2 * L::LPW>();
                else if (after == 1) wait_vm<L::LPW>();
                else wait_vm<0>();
            } else {
                if (after >= 1) wait_vm<L::LPW>(); else wait_vm<0>();
            }
        }
        __syncthreads();   // every wave's share of T landed; T-1's stage is free
        if (T >= 1 && T + L::NST - 1 < ntt) issue(T + L::NST - 1, (T + L::NST - 1) % L::NST);
        const char* Ks = lds + (T % L::NST) * 2 * L::TILE;
        const char* Vs = Ks + L::TILE;
        const int tb = it * kTile;   // tile start relative to tile 0
#pragma unroll
        for (int i = 0; i < RPW; ++i) {
            const int r = wave + 4 * i;
            if (r >= R) break;
            const int lo = max(-1, min(64, rlo[i] - tb));
            const int hi = max(-1, min(64, rhi[i] - tb));
            if (hi < 0 || lo > 63 || lo > hi) continue;  // no key of this tile for the row
            // scores: lane = key
            float s = 0.f;
            const char* krow_l = Ks + lane * L::RB;
            const char* qr = Qs + (hh * R + r) * L::RB;
#pragma unroll
            for (int c = 0; c < L::CPR; ++c) {
                const uint4 kv = *(const uint4*)(krow_l + 16 * (c ^ ksw<L::CPR>(lane)));
                uint4 qv;
                if constexpr (RPW == 1)
                    qv = qreg[c];
                else
                    qv = *(const uint4*)(qr + 16 * c);
                if constexpr (E::E == 2) {
                    s = dot2bf(kv.x, qv.x, s);
                    s = dot2bf(kv.y, qv.y, s);
                    s = dot2bf(kv.z, qv.z, s);
                    s = dot2bf(kv.w, qv.w, s);
                } else {
                    s = __fmaf_rn(__uint_as_float(kv.x), __uint_as_float(qv.x), s);
                    s = __fmaf_rn(__uint_as_float(kv.y), __uint_as_float(qv.y), s);
                    s = __fmaf_rn(__uint_as_float(kv.z), __uint_as_float(qv.z), s);
                    s = __fmaf_rn(__uint_as_float(kv.w), __uint_as_float(qv.w), s);
                }
            }
            const bool valid = lane >= lo && lane <= hi;
            const float sv = valid ? s * a.scale_log2 : kSent;
            const float mt = wave_max(sv);
            const float mn = fmaxf(mrow[i], mt);
            const float alpha = fast_exp2(mrow[i] - mn);
            const float p = valid ? fast_exp2(sv - mn) : 0.f;
            lpart[i] = __fmaf_rn(lpart[i], alpha, p);
            mrow[i] = mn;
            if constexpr (E::E == 2)
                *(uint16_t*)(Pw + 2 * lane) = (uint16_t)to_bf16(p);
            else
                *(float*)(Pw + 4 * lane) = p;
            __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
            __builtin_amdgcn_wave_barrier();
            __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
            // weights: lane = output dim
#pragma unroll
            for (int h = 0; h < DPL; ++h) {
                float o = acc[i][h] * alpha;
                if constexpr (E::E == 2) {
#pragma unroll
                    for (int kb = 0; kb < 16; ++kb) {
                        // keys 4kb .. 4kb+3 of dim 64h + lane, as two bf16 pairs
                        const int row = 4 * kb + ((lane & 15) >> 2);
                        const int byte = 2 * (64 * h + 16 * (lane >> 4) + 4 * (lane & 3));
                        const int ch = (byte >> 4) ^ vsw<E, L::CPR>(row);
                        const v4i16 r4 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                            (VRT_LDS v4i16*)(__UINTPTR_TYPE__)(Vs + row * L::RB + 16 * ch + (byte & 15)));
                        const uint2 vv = __builtin_bit_cast(uint2, r4);
                        const uint2 pp = *(const uint2*)(Pw + 8 * kb);
                        o = dot2bf(pp.x, vv.x, o);
                        o = dot2bf(pp.y, vv.y, o);
                    }
                } else {
#pragma unroll 4
                    for (int j = 0; j < kTile; j += 4) {
                        const float4 pp = *(const float4*)(Pw + 4 * j);
                        const float* vc = (const float*)(Vs + 4 * (64 * h + lane));
                        o = __fmaf_rn(pp.x, vc[(j + 0) * D], o);
                        o = __fmaf_rn(pp.y, vc[(j + 1) * D], o);
                        o = __fmaf_rn(pp.z, vc[(j + 2) * D], o);
                        o = __fmaf_rn(pp.w, vc[(j + 3) * D], o);
                    }
                }
                acc[i][h] = o;
            }
            __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
            __builtin_amdgcn_wave_barrier();
            __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
        }

        if (it == nt - 1) {   // ---- head epilogue
            const int g = g0 + hh;
#pragma unroll
            for (int i = 0; i < RPW; ++i) {
                const int r = wave + 4 * i;
                if (r >= R) break;
                const float lrow = wave_sum(lpart[i]);
                const int j = r / group, gh = r - j * group;
                if (SPLIT) {
                    float* pr = a.partials +
                                (((cu * a.g.hkv + g) * a.n_splits + split) * group + r) * (long long)(2 + D);
                    if (lane == 0) {
                        gst<float>(pr, mrow[i]);
                        gst<float>(pr + 1, lrow);
                    }
#pragma unroll
                    for (int k = 0; k < DPL; ++k) gst<float>(pr + 2 + lane + 64 * k, acc[i][k]);
                } else {
                    const int hq = g * group + gh;
                    const long long orow = (LOOK ? (long long)a.look_o0 : (long long)m.t0) + (long long)qc * a.qchunk + j;
                    char* dst = (char*)a.out + ((cu * m.n_total + orow) * a.g.hq + hq) * (long long)Dio * E::E;
#pragma unroll
                    for (int k = 0; k < DPL; ++k) {
                        const float o = acc[i][k] / lrow;
                        const int d = lane + 64 * k;
                        if (kNarrow && d >= Dio) continue;   // a padding dim of the ring row
                        if constexpr (E::E == 2)
                            gst<uint16_t>(dst + 2 * d, (uint16_t)to_bf16(o));
                        else
                            gst<float>(dst + 4 * d, o);
                    }
                }
            }
        }
    }
}

// ------------------------------------------------ K4: attention, MFMA ----
// The same windowed-causal attention for large sub-batches (the catch-up
// path): bf16 storage, head_dim 64, one query head per kv head.  One
// workgroup of 4 waves per (unit, head, tile of 128 queries); wave w owns
// queries 32w .. 32w+31 of the tile.  Both products run on the bf16 matrix
// cores (v_mfma_f32_32x32x16_bf16, fp32 accumulation) in transposed form:
//   S^T = K Q^T      (32 keys x 32 queries per block; lane = query, so the
//                    softmax of a query is local to the lane and its partner
//                    lane in the other half of the wave)
//   O^T += V^T P^T   (32 dims x 32 queries; V^T is read from LDS with the
//                    transposing read, P^T is S^T's registers, packed)
// With the MFMA result layout (lane l, register r: key 8(r/4) + 4(l/32) +
// r%4 of the block, query l%32), registers 8c .. 8c+7 of a lane hold the
// eight keys that lane contributes to the k = 16 product of key group c; the
// V^T operand is read with the same key order.
//
// Keys stream through LDS in 64-key tiles aligned to absolute position (the
// same tiles and clamped-row fetch as the VALU kernel); a 32-key half-tile
// outside the band of all 32 queries of a wave is skipped, which is exact:
// such a half-tile would only add zero weights.  The softmax scale is folded
// into the rotated query, so scores come out in log2 units, and the matrix
// cores also subtract a per-query reference maximum (an extra k-step), which
// moves only when a half-tile's scores exceed it by more than 2^8 (then the
// accumulators are rescaled), so most half-tiles need neither a subtraction
// nor a rescale on the vector ALU.  The denominator sums the bf16 weights the products use.
// Every per-query step (the MFMA chains, the reference, the partial sums,
// the rescale) depends only on that query's own window and the absolute tile
// grid, so the result does not depend on how frames were batched.
//
// Queries are rotated in the prologue: the angle p * omega_i is formed and
// reduced by 2 pi in fp64 as for the keys, then sin and cos are taken in fp32
// on the reduced angle (error ~3e-7 rad, far below the bf16 rounding of the
// rotated, scaled query that follows).
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef short v8i16 __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));

struct M4 {
    static constexpr int D = 64;
    static constexpr int RB = 128;                // bytes per K / V row
    static constexpr int CPR = 8;                 // 16-byte chunks per row
    static constexpr int QW = 32;                 // queries per wave
    static constexpr int QT = 4 * QW;             // queries per workgroup
    static constexpr int TILE = kTile * RB;       // 8 KB
    static constexpr int NST = 2;                 // LDS stages (4 workgroups per CU fit)
    static constexpr int IPW = TILE / (4 * 1024); // DMA instructions per wave per K (or V) tile
    static constexpr int LPW = 2 * IPW;
    static constexpr int BYTES = NST * 2 * TILE;
};
static_assert(M4::QT == kQTileMfma, "query tile of the MFMA path");
static_assert(M4::NST == 2, "the tile loop's DMA waits assume two stages");
// A query's reference maximum moves only when a half-tile's scores exceed it
// by more than this (log2 units), so unnormalised weights stay below 2^8.
constexpr float kLazy = 8.0f;

// max(a, b, c); the compiler folds the pair into one v_max3_f32.  Written
// with builtins, not inline asm, on purpose: the operands are often matrix-core
// results, and only compiler-visible reads get the wait states the hardware
// requires between an MFMA writing a register and a VALU reading it.
__device__ __forceinline__ float max3f(float a, float b, float c) {
    return __builtin_fmaxf(__builtin_fmaxf(a, b), c);
}

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
    typedef __bf16 b2 __attribute__((ext_vector_type(2)));
    const b2 v = {(__bf16)lo, (__bf16)hi};   // round to nearest even
    return __builtin_bit_cast(uint32_t, v);
}

// At most 128 VGPRs (four waves per SIMD), so four workgroups share a CU; the
// tile loop works on one 32-key half-tile at a time to stay within them.
__global__ __launch_bounds__(256, 4) void k_attn_mfma(AttnArgs a, StateTable t) {
    using L = M4;
    __shared__ __attribute__((aligned(16))) char lds[L::BYTES];
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int jq = lane & 31;        // query of the lane within the wave
    const int hf = lane >> 5;        // half of the wave

    // Workgroup -> (unit, head, query tile).  Workgroups are dispatched to the
    // 8 XCDs round robin; consecutive logical ids (the query tiles of one
    // (unit, head), which read overlapping key windows) are placed on the same
    // XCD so its L2 serves the overlap.
    int b;
    {
        const int nb = gridDim.x, x = blockIdx.x & 7, s = blockIdx.x >> 3;
        const int base = nb >> 3, rem = nb & 7;
        b = x < rem ? x * (base + 1) + s : rem * (base + 1) + (x - rem) * base + s;
    }
    const int qc = b % a.n_qchunks;
    b /= a.n_qchunks;
    const int g = b % a.g.hkv;
    const int unit = b / a.g.hkv;
    const UnitMap& m = a.m;
    const int si = unit / m.nl, li = unit - si * m.nl;
    const long long cu = (long long)t.call_idx[si] * m.nl_call + m.l_off + li;

    const int W = a.g.window;
    const long long avail = t.p0[si] - t.n_kv[si];
    const long long pq0 = t.p0[si] + (long long)qc * L::QT;
    const int nq = min(L::QT, m.n - qc * L::QT);
    const long long wlo = max(avail, pq0 - W + 1);
    const long long whi = pq0 + nq - 1;
    const long long tfirst = floor_div(wlo, kTile);
    const int ntt = (int)(floor_div(whi, kTile) - tfirst + 1);
    const long long T0 = tfirst * kTile;

    char* layer = (char*)t.ring[si] + (long long)(m.layer0 + m.l_off + li) * a.g.layer_bytes;
    const char* Kg = layer + (long long)g * a.g.slice_bytes;
    const char* Vg = Kg + a.g.v_off;

    // the lane's 16-byte chunk of each DMA instruction: tile row r and its
    // swizzled byte offset; kept for the tiles whose rows are all in range
    unsigned dk[L::IPW], dv[L::IPW];
#pragma unroll
    for (int i = 0; i < L::IPW; ++i) {
        const int q = (wave * L::IPW + i) * 64 + lane;
        const int r = q / L::CPR, pc = q % L::CPR;
        dk[i] = (unsigned)r * L::RB + 16 * (pc ^ ksw<L::CPR>(r));
        dv[i] = (unsigned)r * L::RB + 16 * (pc ^ vsw<BF16T, L::CPR>(r));
    }
    auto issue = [&](int T, int st) {
        const long long TB = T0 + (long long)T * kTile;
        // modulo ring: 0 <= TB < 2^31 and the slot count is a multiple of 64,
        // so a tile is contiguous in the ring and 32-bit arithmetic is exact
        const long long sb = a.g.mod ? (long long)((unsigned)TB % (unsigned)a.g.slots) : TB - avail;
        const int rlo = (int)max(0LL, wlo - TB), rhi = (int)min(63LL, whi - TB);
        char* ks = lds + st * 2 * L::TILE;
        char* vs = ks + L::TILE;
        if (rlo == 0 && rhi == 63) {
#pragma unroll
            for (int i = 0; i < L::IPW; ++i) {
                const int ins = wave * L::IPW + i;
                dma16s(Kg + sb * L::RB, dk[i], ks + ins * 1024);
                dma16s(Vg + sb * L::RB, dv[i], vs + ins * 1024);
            }
            return;
        }
        // an edge tile: rows outside [rlo, rhi] repeat the nearest row in range
#pragma unroll
        for (int i = 0; i < L::IPW; ++i) {
            const int ins = wave * L::IPW + i;
            const int q = ins * 64 + lane_id_v();
            const int r = q / L::CPR, pc = q % L::CPR;
            const int rr = min(max(r, rlo), rhi);
            const unsigned off = (unsigned)rr * L::RB;
            dma16s(Kg + sb * L::RB, off + 16 * (pc ^ ksw<L::CPR>(r)), ks + ins * 1024);
            dma16s(Vg + sb * L::RB, off + 16 * (pc ^ vsw<BF16T, L::CPR>(r)), vs + ins * 1024);
        }
    };

    // ---- this wave's queries; lanes past the last query repeat it
    const int qw0 = wave * L::QW;
    const int nqw = min(L::QW, nq - qw0);   // may be <= 0 for the last tile
    const int jj = max(0, min(jq, nqw - 1));
    const long long pq = pq0 + qw0 + jj;
    const long long frame = m.t0 + (long long)qc * L::QT + qw0 + jj;
    const char* qsrc =
        (const char*)a.q + ((cu * m.n_total + frame) * a.g.hq + g) * (long long)(L::D * 2);
    uint4 qraw[4];
    double om[16];
    if (nqw > 0) {
#pragma unroll
        for (int s = 0; s < 4; ++s) qraw[s] = gld<uint4>(qsrc + 32 * s + 16 * hf);
        const double* wp = a.g.omega + 8 * hf;
#pragma unroll
        for (int s = 0; s < 2; ++s)
#pragma unroll
            for (int e = 0; e < 8; ++e) om[8 * s + e] = wp[16 * s + e];
    }
#pragma unroll
    for (int st = 0; st < L::NST - 1; ++st)
        if (st < ntt) issue(st, st);

    // rotate: the lane holds dims 16s + 8hf + e (s = 0..3, e = 0..7); NEOX
    // pairs (i, i + 32) are chunks s and s + 2 of the same lane.
    bf16x8_t qt[4];
    const float qscale = a.scale_log2;   // scores come out in log2 units
    if (nqw > 0) {
        float cs[16], sn[16];
        const double pd = (double)pq;
        // frequencies 16s + 8hf + e: two contiguous runs of 8 doubles of
        // the argument block per lane, loaded up front
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            const CosSin r = rope_cs(pd * om[i]);
            cs[i] = r.c;
            sn[i] = r.s;
        }
        wait_vm<L::LPW>();   // the query loads (only tile 0 was issued after them)
#pragma unroll
        for (int s = 0; s < 2; ++s) {
            const uint32_t* x0 = (const uint32_t*)&qraw[s];
            const uint32_t* x1 = (const uint32_t*)&qraw[s + 2];
            uint32_t y0[4], y1[4];
#pragma unroll
            for (int w = 0; w < 4; ++w) {
                float a0[2], a1[2], b0[2], b1[2];
                a0[0] = bf_lo(x0[w]); a0[1] = bf_hi(x0[w]);
                a1[0] = bf_lo(x1[w]); a1[1] = bf_hi(x1[w]);
#pragma unroll
                for (int u = 0; u < 2; ++u) {
                    const float c = cs[8 * s + 2 * w + u], sv = sn[8 * s + 2 * w + u];
                    b0[u] = __fmaf_rn(a0[u], c, -(a1[u] * sv)) * qscale;
                    b1[u] = __fmaf_rn(a1[u], c, a0[u] * sv) * qscale;
                }
                y0[w] = pack_bf16x2(b0[0], b0[1]);
                y1[w] = pack_bf16x2(b1[0], b1[1]);
            }
            qt[s] = __builtin_bit_cast(bf16x8_t, make_uint4(y0[0], y0[1], y0[2], y0[3]));
            qt[s + 2] = __builtin_bit_cast(bf16x8_t, make_uint4(y1[0], y1[1], y1[2], y1[3]));
        }
    }

    // ---- bands relative to T0: the lane's query, and the wave's union /
    // intersection (for skipping and for mask-free half-tiles)
    // the lane's own band [max(alo, h - W + 1), h] with h = hq0 + its query
    // index is recomputed on the edge half-tiles that need it
    const int hq0 = (int)(pq0 + qw0 - T0), alo = (int)(avail - T0);
    const long long wq_first = pq0 + qw0, wq_last = pq0 + qw0 + max(nqw, 1) - 1;
    const int blo = (int)(max(avail, wq_first - W + 1) - T0), bhi = (int)(wq_last - T0);
    const int flo = (int)(max(avail, wq_last - W + 1) - T0), fhi = (int)(wq_first - T0);

    f32x16_t o[2];
#pragma unroll
    for (int d = 0; d < 2; ++d)
#pragma unroll
        for (int r = 0; r < 16; ++r) o[d][r] = 0.f;
    // Reference maximum of the lane's query (log2 units), subtracted from the
    // scores by the matrix cores themselves: a fifth k-step per score block
    // multiplies the constant operand kext (ones at k = 0, 1) with qext =
    // (-m_hi, -m_lo), the reference split into two bf16 values, so the block
    // comes out as s - mref with mref = m_hi + m_lo exactly.  mref is 0 until
    // the query's first visible key, then moves only when a half-tile's maximum
    // exceeds it by more than kLazy (weights stay below 2^kLazy); a lane whose
    // reference does not move is rescaled by exactly 1, if at all.
    // lane parts of the LDS addresses (the swizzles depend only on lane
    // bits, so each read is a stage base + one of these + an immediate)
    int koff[4], voff[2];
#pragma unroll
    for (int st = 0; st < 4; ++st) koff[st] = jq * L::RB + 16 * ((2 * st + hf) ^ ksw<L::CPR>(jq));
#pragma unroll
    for (int d = 0; d < 2; ++d) {
        const int row = 4 * hf + ((lane & 15) >> 2);
        const int byte = 2 * (32 * d + 16 * ((lane >> 4) & 1) + 4 * (lane & 3));
        voff[d] = L::TILE + row * L::RB + 16 * ((byte >> 4) ^ vsw<BF16T, L::CPR>(row)) + (byte & 15);
    }
    const uint32_t one_lo = hf == 0 ? 0x3f803f80u : 0u;
    const bf16x8_t kext = __builtin_bit_cast(bf16x8_t, make_uint4(one_lo, 0u, 0u, 0u));
    bf16x8_t qext = __builtin_bit_cast(bf16x8_t, make_uint4(0u, 0u, 0u, 0u));
    float mref = 0.f, lpart = 0.f;
    bool seen = false;
    constexpr uint32_t kOnes = 0x3f803f80u;   // (1, 1) in bf16

    for (int T = 0; T < ntt; ++T) {
        wait_vm<0>();   // two stages: only tile T is in flight here
        __syncthreads();
        if (T + L::NST - 1 < ntt) issue(T + L::NST - 1, (T + L::NST - 1) % L::NST);
        const char* Sb = lds + (T % L::NST) * 2 * L::TILE;   // K tile, then V tile
        const int tb = T * kTile;
        if (nqw <= 0 || tb + 63 < blo || tb > bhi) continue;   // no key of this tile for the wave
        bool rel[2], full[2];
#pragma unroll
        for (int k = 0; k < 2; ++k) {
            const int kb = tb + 32 * k;
            rel[k] = kb + 31 >= blo && kb <= bhi;
            full[k] = kb >= flo && kb + 31 <= fhi;
        }
        // one 32-key half-tile at a time: scores, reference update, weights,
        // then its share of the output
#pragma unroll
        for (int k = 0; k < 2; ++k) {
            if (!rel[k]) continue;
            // scores relative to the reference: S^T = [K | 1] [Q | -mref]^T
            bf16x8_t kv[4];
#pragma unroll
            for (int st = 0; st < 4; ++st)
                kv[st] = __builtin_bit_cast(bf16x8_t, *(const uint4*)(Sb + koff[st] + 32 * k * L::RB));
            f32x16_t s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kext, qext, f32x16_t{}, 0, 0, 0);
#pragma unroll
            for (int st = 0; st < 4; ++st) s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kv[st], qt[st], s, 0, 0, 0);
            // band mask on edge half-tiles (masked scores become the sentinel,
            // whose weight underflows to exactly 0)
            if (!full[k]) {
                const int bhi_v = hq0 + min(lane_id_v() & 31, nqw - 1);
                const int blo_v = max(alo, bhi_v - W + 1);
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int key = tb + 32 * k + 8 * (r >> 2) + 4 * hf + (r & 3);
                    s[r] = (key >= blo_v && key <= bhi_v) ? s[r] : kSent;
                }
            }
            float mt = kSent;
#pragma unroll
            for (int r = 0; r < 16; r += 2) mt = max3f(mt, s[r], s[r + 1]);
            {
                const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(mt), __float_as_uint(mt),
                                                                 false, false);
                mt = max3f(__uint_as_float(sw[0]), __uint_as_float(sw[1]), kSent);
            }
            const bool move = seen ? mt > kLazy : mt > kSent;
            if (__builtin_amdgcn_ballot_w64(move) != 0) {   // a query's first keys, or a jump of 2^kLazy
                float delta = 0.f;
                if (move) {
                    const float mnew = mref + mt;
                    const uint32_t hi = to_bf16(mnew);
                    const float mhi = __uint_as_float(hi << 16);
                    const uint32_t lo = to_bf16(mnew - mhi);
                    const float mt_ref = mhi + __uint_as_float(lo << 16);
                    const float alpha = seen ? fast_exp2(mref - mt_ref) : 0.f;
                    lpart *= alpha;
#pragma unroll
                    for (int d = 0; d < 2; ++d)
#pragma unroll
                        for (int r = 0; r < 16; ++r) o[d][r] *= alpha;
                    delta = mt_ref - mref;
                    mref = mt_ref;
                    seen = true;
                    const uint32_t neg = (hi ^ 0x8000u) | ((lo ^ 0x8000u) << 16);
                    qext = __builtin_bit_cast(bf16x8_t, make_uint4(hf == 0 ? neg : 0u, 0u, 0u, 0u));
                }
#pragma unroll
                for (int r = 0; r < 16; ++r) s[r] -= delta;
            }
            uint32_t pb[8];
#pragma unroll
            for (int w = 0; w < 8; ++w) pb[w] = pack_bf16x2(fast_exp2(s[2 * w]), fast_exp2(s[2 * w + 1]));
            // the denominator sums the same bf16 weights the products use
#pragma unroll
            for (int w = 0; w < 8; ++w) lpart = dot2bf(pb[w], kOnes, lpart);
            // O^T += V^T P^T, key groups in ascending order
#pragma unroll
            for (int c = 0; c < 2; ++c) {
                const bf16x8_t pv = __builtin_bit_cast(
                    bf16x8_t, make_uint4(pb[4 * c], pb[4 * c + 1], pb[4 * c + 2], pb[4 * c + 3]));
#pragma unroll
                for (int d = 0; d < 2; ++d) {
                    v4i16 part[2];
#pragma unroll
                    for (int u = 0; u < 2; ++u)
                        part[u] = __builtin_amdgcn_ds_read_tr16_b64_v4i16((VRT_LDS v4i16*)(__UINTPTR_TYPE__)(
                            Sb + voff[d] + (32 * k + 16 * c + 8 * u) * L::RB));
                    const v8i16 vv = __builtin_shufflevector(part[0], part[1], 0, 1, 2, 3, 4, 5, 6, 7);
                    o[d] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, vv), pv,
                                                                   o[d], 0, 0, 0);
                }
            }
        }
    }

    // ---- epilogue: denominator = lower-half partial + upper-half partial
    if (nqw <= 0) return;
    const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(lpart), __float_as_uint(lpart),
                                                     false, false);
    const float l = __uint_as_float(sw[0]) + __uint_as_float(sw[1]);
    if (jq >= nqw) return;
    // one reciprocal per query instead of 32 divisions (the outputs are
    // rounded to bf16 right after)
    const float rl = 1.0f / l;
    char* dst = (char*)a.out + ((cu * m.n_total + frame) * a.g.hq + g) * (long long)(L::D * 2);
#pragma unroll
    for (int d = 0; d < 2; ++d)
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4) {
            uint2 v;
            v.x = pack_bf16x2(o[d][4 * q4] * rl, o[d][4 * q4 + 1] * rl);
            v.y = pack_bf16x2(o[d][4 * q4 + 2] * rl, o[d][4 * q4 + 3] * rl);
            gst<uint2>(dst + 2 * (32 * d + 8 * q4 + 4 * hf), v);
        }
}

// ------------------------------------------ waiting rows (lookahead) ----
// One thread per 16-byte column of a q row: the last `keep` rows of [the
// waiting rows | this sub-batch's q rows] move to the front of the waiting
// rows.  Source index >= destination index for every row, and a thread
// copies its column's rows in ascending order, so the copy is safe in place.
template <class E, int D>
__global__ __launch_bounds__(64) void k_pend_save(AttnArgs a, StateTable t, int keep) {
    const UnitMap& m = a.m;
    const long long row = (long long)a.g.hq * a.g.Dio * E::E;   // io rows
    const int nch = (int)(row / 16), bpu = (nch + 63) / 64;
    const int unit = blockIdx.x / bpu, c = (blockIdx.x - unit * bpu) * 64 + threadIdx.x;
    if (c >= nch) return;
    const int si = unit / m.nl, li = unit - si * m.nl;
    const long long cu = (long long)t.call_idx[si] * m.nl_call + m.l_off + li;
    char* pend = (char*)t.ring[si] + a.pend_off + (long long)(m.layer0 + m.l_off + li) * a.pend_layer;
    const int p = a.look_pend, shift = p + m.n - keep;
    for (int r = 0; r < keep; ++r) {
        const int src = shift + r;
        uint4 v;
        if (src < p)
            v = gld<uint4>(pend + src * row + 16 * c);
        else
            v = gld<uint4>((const char*)a.q + (cu * m.n_total + m.t0 + (src - p)) * row + 16 * c);
        gst<uint4>(pend + r * row + 16 * c, v);
    }
}

// ---------------------------------------------- K5b: split-K merge ----
// One wave per (unit, q head), lane = output dim.  Splits are merged in
// ascending absolute order; splits past the window were never written.
template <class E, int D>
__global__ __launch_bounds__(64) void k_dec_combine(AttnArgs a, StateTable t) {
    constexpr int DPL = D / 64;
    const int lane = threadIdx.x;
    const int hq = blockIdx.x % a.g.hq;
    const int unit = blockIdx.x / a.g.hq;
    const UnitMap& m = a.m;
    const int si = unit / m.nl, li = unit - si * m.nl;
    const long long cu = (long long)t.call_idx[si] * m.nl_call + m.l_off + li;
    const int g = hq / a.g.group, r = hq - g * a.g.group;  // one position per call
    const long long avail = t.p0[si] - t.n_kv[si];
    const long long pq = t.p0[si];
    const long long wlo = max(avail, pq - a.g.window + 1);
    const int ns = (int)(floor_div(pq, a.split_len) - floor_div(wlo, a.split_len) + 1);
    const int group = a.g.group;
    const float* base = a.partials + ((cu * a.g.hkv + g) * a.n_splits) * group * (long long)(2 + D);
    float M = kSent;
    for (int s = 0; s < ns; ++s) M = fmaxf(M, gld<float>(base + ((long long)s * group + r) * (2 + D)));
    float Lsum = 0.f, o[DPL];
#pragma unroll
    for (int k = 0; k < DPL; ++k) o[k] = 0.f;
    for (int s = 0; s < ns; ++s) {
        const float* pr = base + ((long long)s * group + r) * (2 + D);
        const float w = fast_exp2(gld<float>(pr) - M);
        Lsum = __fmaf_rn(gld<float>(pr + 1), w, Lsum);
#pragma unroll
        for (int k = 0; k < DPL; ++k) o[k] = __fmaf_rn(gld<float>(pr + 2 + lane + 64 * k), w, o[k]);
    }
    char* dst = (char*)a.out + ((cu * m.n_total + m.t0) * a.g.hq + hq) * (long long)D * E::E;
#pragma unroll
    for (int k = 0; k < DPL; ++k) {
        const float v = o[k] / Lsum;
        const int d = lane + 64 * k;
        if constexpr (E::E == 2)
            gst<uint16_t>(dst + 2 * d, (uint16_t)to_bf16(v));
        else
            gst<float>(dst + 4 * d, v);
    }
}

}  // namespace

// ------------------------------------------------ static scratch array ----
// Split-K partials of the allocation-free decode step.  In host code the
// array's name stands for a host-side shadow, not a device address: kernels
// only ever get the address that hipGetSymbolAddress returns for the current
// device (each device holds its own copy at its own address).
static __device__ __align__(256) char scratch[kStaticScratchBytes];

hipError_t static_scratch(void** ptr) {
    constexpr int kDevices = 64;
    static std::mutex mu;
    static void* addr[kDevices] = {};
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kDevices) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(mu);
    if (!addr[dev]) {
        void* p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return e;
        if (!p) return hipErrorInvalidSymbol;
        addr[dev] = p;
    }
    *ptr = addr[dev];
    return hipSuccess;
}

// ------------------------------------------------------------ launchers ----
#define VRT_DISPATCH_ED(dtype, D, BODY)                                        \
    do {                                                                       \
        if ((dtype) == 1 && (D) == 64) { using E_ = BF16T; constexpr int D_ = 64; BODY; } \
        else if ((dtype) == 1 && (D) == 128) { using E_ = BF16T; constexpr int D_ = 128; BODY; } \
        else if ((dtype) == 0 && (D) == 64) { using E_ = F32T; constexpr int D_ = 64; BODY; } \
        else if ((dtype) == 0 && (D) == 128) { using E_ = F32T; constexpr int D_ = 128; BODY; } \
        else return hipErrorInvalidValue;                                      \
    } while (0)

hipError_t launch_rope_append(const AppendArgs& a, const StateTable& t, hipStream_t s) {
    const int nfb = (a.m.n + 3) / 4;
    const dim3 grid((unsigned)(a.m.n_states * a.m.nl * nfb));
    VRT_DISPATCH_ED(a.g.dtype, a.g.D, {
        if (a.g.mod)
            VRT_LAUNCH((k_rope_append<E_, D_, true>), grid, dim3(256), 0, s, a, t);
        else
            VRT_LAUNCH((k_rope_append<E_, D_, false>), grid, dim3(256), 0, s, a, t);
    });
    return hipSuccess;
}

hipError_t launch_attn_valu(const AttnArgs& a, const StateTable& t, hipStream_t s) {
    const long long blocks =
        (long long)a.m.n_states * a.m.nl * (a.g.hkv / a.hg) * a.n_qchunks * a.n_splits;
    const dim3 grid((unsigned)blocks), block(256);
    const bool split = a.n_splits > 1 || a.partials != nullptr;
    const bool app = a.append != 0;
    const int nqs = a.g.rope ? a.m.n : a.look_nout;   // queries per unit in this launch
    const bool one = (long long)std::min(a.qchunk, nqs) * a.g.group <= 4;  // <= 1 row per wave
#define VRT_ATTN(MOD, SPLIT, APP)                                                                   \
    do {                                                                                            \
        if (one)                                                                                    \
            VRT_LAUNCH((k_attn<E_, D_, MOD, SPLIT, APP, 1, false>), grid, block, 0, s, a, t); \
        else                                                                                        \
            VRT_LAUNCH((k_attn<E_, D_, MOD, SPLIT, APP, kRows / 4, false>), grid, block, 0, s, a, t); \
    } while (0)
#define VRT_LOOK(MOD, APP)                                                                          \
    do {                                                                                            \
        if (one)                                                                                    \
            VRT_LAUNCH((k_attn<E_, D_, MOD, false, APP, 1, true>), grid, block, 0, s, a, t); \
        else                                                                                        \
            VRT_LAUNCH((k_attn<E_, D_, MOD, false, APP, kRows / 4, true>), grid, block, 0, s, a, t); \
    } while (0)
    // windows without rotation: no splits; the fused append needs one query chunk
    if (!a.g.rope && (split || (app && a.n_qchunks != 1))) return hipErrorInvalidValue;
    VRT_DISPATCH_ED(a.g.dtype, a.g.D, {
        if (!a.g.rope && a.g.mod && app) VRT_LOOK(true, true);
        else if (!a.g.rope && a.g.mod) VRT_LOOK(true, false);
        else if (!a.g.rope && app) VRT_LOOK(false, true);
        else if (!a.g.rope) VRT_LOOK(false, false);
        else if (a.g.mod && split && app) VRT_ATTN(true, true, true);
        else if (a.g.mod && split) VRT_ATTN(true, true, false);
        else if (a.g.mod && app) VRT_ATTN(true, false, true);
        else if (a.g.mod) VRT_ATTN(true, false, false);
        else if (app) VRT_ATTN(false, false, true);
        else VRT_ATTN(false, false, false);
    });
#undef VRT_ATTN
#undef VRT_LOOK
    return hipSuccess;
}

hipError_t launch_attn_mfma(const AttnArgs& a, const StateTable& t, hipStream_t s) {
    if (a.g.dtype != 1 || a.g.D != 64 || a.g.group != 1 || a.n_splits != 1)
        return hipErrorInvalidValue;
    const long long blocks = (long long)a.m.n_states * a.m.nl * a.g.hkv * a.n_qchunks;
    VRT_LAUNCH(k_attn_mfma, dim3((unsigned)blocks), dim3(256), 0, s, a, t);
    return hipSuccess;
}

hipError_t launch_pend_save(const AttnArgs& a, const StateTable& t, int keep, hipStream_t s) {
    if (keep < 1) return hipSuccess;
    const long long row = (long long)a.g.hq * a.g.Dio * (a.g.dtype == 1 ? 2 : 4);
    const long long bpu = (row / 16 + 63) / 64;
    const dim3 grid((unsigned)((long long)a.m.n_states * a.m.nl * bpu));
    VRT_DISPATCH_ED(a.g.dtype, a.g.D, {
        VRT_LAUNCH((k_pend_save<E_, D_>), grid, dim3(64), 0, s, a, t, keep);
    });
    return hipSuccess;
}

hipError_t launch_dec_combine(const AttnArgs& a, const StateTable& t, hipStream_t s) {
    const dim3 grid((unsigned)(a.m.n_states * a.m.nl * a.g.hq));
    VRT_DISPATCH_ED(a.g.dtype, a.g.D, {
        VRT_LAUNCH((k_dec_combine<E_, D_>), grid, dim3(64), 0, s, a, t);
    });
    return hipSuccess;
}

hipError_t launch_compact(const CompactArgs& a, const CompactTable& t, hipStream_t s) {
    const dim3 grid((unsigned)(a.n_entries * a.g.hkv * 2));
    VRT_DISPATCH_ED(a.g.dtype, a.g.D, {
        VRT_LAUNCH((k_compact<E_, D_>), grid, dim3(256), 0, s, a, t);
    });
    return hipSuccess;
}

}  // namespace vrt
