// gfx950 kernels for streamed windowed-causal attention.
//
//   k_rope_append  NEOX RoPE (theta^(-2i/d) frequencies, angle in fp64) of the
//                  new keys, then the rotated keys and the raw values are
//                  written to their ring slots (Voxtral Realtime streaming-plan
//                  page, "SHIPPED" section: the chunk's K/V go to rows
//                  [n_kv_before, n_kv_total); family doc, Streaming row item 5:
//                  decoder token cur goes to slot cur % n_ctx).
//   k_compact      copies the last `kept` rows of a ring slice to its front
//                  (streaming-plan page, "Unbounded length": compact_enc_ring).
//                  Source and destination may overlap; every chunk is staged
//                  through LDS before any of it is written back.
//   k_attn_valu    windowed-causal attention, fp32 accumulation: a query at
//                  absolute position p sees keys in (p - W, p].  Keys are
//                  visited in 64-key tiles that start at multiples of 64 in
//                  absolute position, in ascending order; keys outside a
//                  query's window get probability exactly 0 and tiles with no
//                  key for a query are exact no-ops for it, so a query's
//                  result does not depend on which other queries share its
//                  workgroup, on ring slots or on compaction: chunked feeding
//                  reproduces the offline pass bit for bit.
//   k_dec_combine  log-sum-exp merge of split-K partials in ascending split
//                  order (decode step).
//
// Numerics: -ffp-contract=off for the whole library; every fused multiply-add
// below is written out.  bf16 storage: q, k, v and the softmax weights enter
// the dot products as bf16 (v_dot2_f32_bf16, fp32 accumulate); fp32 storage
// keeps everything in fp32.
#include <hip/hip_runtime.h>

#include "vrt_internal.h"

namespace vrt {
namespace {

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

struct F32T { static constexpr int E = 4; };
struct BF16T { static constexpr int E = 2; };

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
// omega_i = theta^(-2i/D); angle = pos * omega_i, both in fp64 (a float32
// angle is off by up to ~0.03 rad at positions near 1e6).
__device__ __forceinline__ void rope_angle(long long pos, int i, int D, double theta,
                                           double* c, double* s) {
    const double w = pow(theta, -2.0 * (double)i / (double)D);
    sincos((double)pos * w, s, c);
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

template <class E> __device__ __forceinline__ void ld4(const char* p, float (&x)[4]);
template <> __device__ __forceinline__ void ld4<F32T>(const char* p, float (&x)[4]) {
    const float4 v = *(const float4*)p;
    x[0] = v.x; x[1] = v.y; x[2] = v.z; x[3] = v.w;
}
template <> __device__ __forceinline__ void ld4<BF16T>(const char* p, float (&x)[4]) {
    const uint2 v = *(const uint2*)p;
    x[0] = bf_lo(v.x); x[1] = bf_hi(v.x); x[2] = bf_lo(v.y); x[3] = bf_hi(v.y);
}
template <class E> __device__ __forceinline__ void st4(char* p, const float (&x)[4]);
template <> __device__ __forceinline__ void st4<F32T>(char* p, const float (&x)[4]) {
    *(float4*)p = make_float4(x[0], x[1], x[2], x[3]);
}
template <> __device__ __forceinline__ void st4<BF16T>(char* p, const float (&x)[4]) {
    uint2 v;
    v.x = to_bf16(x[0]) | (to_bf16(x[1]) << 16);
    v.y = to_bf16(x[2]) | (to_bf16(x[3]) << 16);
    *(uint2*)p = v;
}

// ---------------------------------------------------------- K1: append ----
// One workgroup per (unit, group of 4 frames).  Each thread rotates 4 NEOX
// pairs of one (frame, kv head) row; the angles of the workgroup's frames are
// computed once into LDS and shared by all heads.
template <class E, int D, bool MOD>
__global__ __launch_bounds__(256) void k_rope_append(AppendArgs a, StateTable t) {
    constexpr int FR = 4, H2 = D / 2, CG = H2 / 4, VCH = D * E::E / 16;
    __shared__ double cs[FR * H2 * 2];
    const UnitMap& m = a.m;
    const int nfb = (m.n + FR - 1) / FR;
    const int unit = blockIdx.x / nfb, fb = blockIdx.x - unit * nfb;
    const int si = unit / m.nl, li = unit - si * m.nl;
    const long long p0 = t.p0[si];
    const int nkv = t.n_kv[si];
    const int f0 = fb * FR, nf = min(FR, m.n - f0);
    for (int x = threadIdx.x; x < nf * H2; x += blockDim.x) {
        const int f = x / H2, i = x - f * H2;
        double c, s;
        rope_angle(p0 + f0 + f, i, D, a.g.theta, &c, &s);
        cs[2 * x] = c;
        cs[2 * x + 1] = s;
    }
    __syncthreads();
    const int hkv = a.g.hkv;
    const long long cu = (long long)t.call_idx[si] * m.nl_call + m.l_off + li;
    const long long row_elems = (long long)hkv * D;
    const long long in0 = (cu * m.n_total + m.t0 + f0) * row_elems * E::E;
    const char* kin = (const char*)a.k + in0;
    const char* vin = (const char*)a.v + in0;
    char* layer = (char*)t.ring[si] + (long long)(m.layer0 + m.l_off + li) * a.g.layer_bytes;
    for (int x = threadIdx.x; x < nf * hkv * CG; x += blockDim.x) {
        const int c = x % CG, fh = x / CG, h = fh % hkv, f = fh / hkv;
        const long long pos = p0 + f0 + f;
        const long long slot = MOD ? (pos % a.g.slots) : (long long)(nkv + f0 + f);
        const char* src = kin + ((long long)f * row_elems + (long long)h * D) * E::E;
        float x0[4], x1[4], y0[4], y1[4];
        ld4<E>(src + 4 * c * E::E, x0);
        ld4<E>(src + (H2 + 4 * c) * E::E, x1);
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const double* an = cs + 2 * (f * H2 + 4 * c + q);
            rope_rot(x0[q], x1[q], an[0], an[1], &y0[q], &y1[q]);
        }
        char* dst = layer + (long long)h * a.g.slice_bytes + slot * (D * E::E);
        st4<E>(dst + 4 * c * E::E, y0);
        st4<E>(dst + (H2 + 4 * c) * E::E, y1);
    }
    for (int x = threadIdx.x; x < nf * hkv * VCH; x += blockDim.x) {
        const int c = x % VCH, fh = x / VCH, h = fh % hkv, f = fh / hkv;
        const long long pos = p0 + f0 + f;
        const long long slot = MOD ? (pos % a.g.slots) : (long long)(nkv + f0 + f);
        const uint4 val =
            *(const uint4*)(vin + ((long long)f * row_elems + (long long)h * D) * E::E + 16 * c);
        *(uint4*)(layer + a.g.v_off + (long long)h * a.g.slice_bytes + slot * (D * E::E) +
                  16 * c) = val;
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
            stage[x] = *(const uint4*)(src + (long long)r0 * ROWB + 16LL * x);
        __syncthreads();
        for (int x = threadIdx.x; x < n16; x += blockDim.x)
            *(uint4*)(base + (long long)r0 * ROWB + 16LL * x) = stage[x];
        __syncthreads();
    }
}

// ------------------------------------------------------ K3: attention ----
template <class E, int D>
struct Lds {
    static constexpr int ROWDW = D * E::E / 4;           // dwords per K / q row
    static constexpr int KP = ROWDW + 4;                 // padded K row pitch
    static constexpr int VP = kTile * E::E / 4 + 4;      // padded V^T row pitch
    static constexpr int KDW = kTile * KP;
    static constexpr int VDW = D * VP;
    static constexpr int BUF = KDW + VDW;
    static constexpr int QDW = kRows * ROWDW;
    static constexpr int PDW = kTile * E::E / 4;         // one P row per wave
    static constexpr int TOTAL = 2 * BUF + QDW + 4 * PDW;
    static constexpr int CPR = D * E::E / 16;            // 16-byte chunks per row
    static constexpr int IPT = 32 * CPR / 256;           // (row pair, chunk) items per thread
};

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o));
    return v;
}
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v = v + __shfl_xor(v, o);
    return v;
}

// One workgroup (4 waves) per (unit, kv head, query chunk, key split).  Rows
// are (query position j, q head of the kv group): r = j * group + gh.  Wave w
// owns rows w, w + 4, ...; for each tile a row's scores are formed with
// lane = key, its weights with lane = output dim.
//
// APPEND: the call's new frames all belong to this workgroup's query chunk
// (one chunk per unit), so the workgroup whose key range ends at the newest
// frame (chunk 0; in split mode the last split) also rotates and writes the
// new K/V rows of its kv head before it reads the window.  Nothing else reads
// those rows in this launch, so the launch needs no separate append kernel.
template <class E, int D, bool MOD, bool SPLIT, bool APPEND>
__global__ __launch_bounds__(256) void k_attn_valu(AttnArgs a, StateTable t) {
    using L = Lds<E, D>;
    constexpr int H2 = D / 2, CG = H2 / 4;
    __shared__ __attribute__((aligned(16))) uint32_t lds[L::TOTAL];
    uint32_t* Qs = lds + 2 * L::BUF;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    uint32_t* Pw = Qs + L::QDW + wave * L::PDW;

    int b = blockIdx.x;
    const int split = SPLIT ? b % a.n_splits : 0;
    if (SPLIT) b /= a.n_splits;
    const int qc = b % a.n_qchunks;
    b /= a.n_qchunks;
    const int g = b % a.g.hkv;
    const int unit = b / a.g.hkv;
    const UnitMap& m = a.m;
    const int si = unit / m.nl, li = unit - si * m.nl;
    const long long cu = (long long)t.call_idx[si] * m.nl_call + m.l_off + li;

    const int W = a.g.window, group = a.g.group;
    const long long avail = t.p0[si] - t.n_kv[si];           // abs_base / first position
    const long long pq0 = t.p0[si] + (long long)qc * a.qchunk;  // first query of the chunk
    const int nq = min(a.qchunk, m.n - qc * a.qchunk);
    const int R = nq * group;
    long long wlo = max(avail, pq0 - W + 1);
    long long whi = pq0 + nq - 1;
    bool appender = APPEND && qc == 0;
    if (SPLIT) {
        const long long s_abs = floor_div(wlo, a.split_len) + split;
        if (s_abs > floor_div(whi, a.split_len)) return;  // split past the window: nothing
        appender = appender && s_abs == floor_div(whi, a.split_len);
        wlo = max(wlo, s_abs * a.split_len);
        whi = min(whi, s_abs * a.split_len + a.split_len - 1);
    }

    char* layer = (char*)t.ring[si] + (long long)(m.layer0 + m.l_off + li) * a.g.layer_bytes;
    char* Kg = layer + (long long)g * a.g.slice_bytes;
    char* Vg = Kg + a.g.v_off;

    // ---- RoPE angles of the chunk's positions, once, into the second tile
    // buffer (free until the first tile is committed there)
    double* cs = (double*)(lds + L::BUF);
    for (int x = threadIdx.x; x < nq * H2; x += blockDim.x) {
        const int j = x / H2, i = x - j * H2;
        rope_angle(pq0 + j, i, D, a.g.theta, &cs[2 * x], &cs[2 * x + 1]);
    }
    __syncthreads();

    // ---- new K/V rows of kv head g (fused append)
    if (APPEND && appender) {
        constexpr int VCH = D * E::E / 16;
        const long long row_elems = (long long)a.g.hkv * D;
        const long long in0 = (cu * m.n_total + m.t0) * row_elems * E::E;
        const char* kin = (const char*)a.k + in0 + (long long)g * D * E::E;
        const char* vin = (const char*)a.v + in0 + (long long)g * D * E::E;
        const int nkv = t.n_kv[si];
        for (int x = threadIdx.x; x < m.n * CG; x += blockDim.x) {
            const int c = x % CG, f = x / CG;
            const long long pos = t.p0[si] + f;
            const long long slot = MOD ? (pos % a.g.slots) : (long long)(nkv + f);
            const char* src = kin + (long long)f * row_elems * E::E;
            float x0[4], x1[4], y0[4], y1[4];
            ld4<E>(src + 4 * c * E::E, x0);
            ld4<E>(src + (H2 + 4 * c) * E::E, x1);
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const double* an = cs + 2 * (f * H2 + 4 * c + q);
                rope_rot(x0[q], x1[q], an[0], an[1], &y0[q], &y1[q]);
            }
            char* dst = Kg + slot * (D * E::E);
            st4<E>(dst + 4 * c * E::E, y0);
            st4<E>(dst + (H2 + 4 * c) * E::E, y1);
        }
        for (int x = threadIdx.x; x < m.n * VCH; x += blockDim.x) {
            const int c = x % VCH, f = x / VCH;
            const long long pos = t.p0[si] + f;
            const long long slot = MOD ? (pos % a.g.slots) : (long long)(nkv + f);
            *(uint4*)(Vg + slot * (D * E::E) + 16 * c) =
                *(const uint4*)(vin + (long long)f * row_elems * E::E + 16 * c);
        }
    }

    // ---- rotated queries -> LDS (dtype E)
    {
        const long long qrow = (long long)a.g.hq * D;
        for (int x = threadIdx.x; x < R * CG; x += blockDim.x) {
            const int c = x % CG, r = x / CG;
            const int j = r / group, gh = r - j * group;
            const int hq = g * group + gh;
            const char* src = (const char*)a.q +
                              ((cu * m.n_total + m.t0 + (long long)qc * a.qchunk + j) * qrow +
                               (long long)hq * D) * E::E;
            float x0[4], x1[4], y0[4], y1[4];
            ld4<E>(src + 4 * c * E::E, x0);
            ld4<E>(src + (H2 + 4 * c) * E::E, x1);
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const double* an = cs + 2 * (j * H2 + 4 * c + q);
                rope_rot(x0[q], x1[q], an[0], an[1], &y0[q], &y1[q]);
            }
            char* dst = (char*)(Qs + r * L::ROWDW);
            st4<E>(dst + 4 * c * E::E, y0);
            st4<E>(dst + (H2 + 4 * c) * E::E, y1);
        }
    }
    if (APPEND && appender) __threadfence();   // new rows visible before the window is read
    __syncthreads();                           // angles consumed; Qs written

    // ---- per-row state (rows w, w+4, w+8, w+12 of this wave)
    constexpr int RPW = kRows / 4;
    constexpr int DPL = D / 64;  // output dims per lane
    float mrow[RPW], lrow[RPW], acc[RPW][DPL];
    long long rlo[RPW], rhi[RPW];
#pragma unroll
    for (int i = 0; i < RPW; ++i) {
        mrow[i] = kSent;
        lrow[i] = 0.f;
#pragma unroll
        for (int k = 0; k < DPL; ++k) acc[i][k] = 0.f;
        const int r = wave + 4 * i;
        const long long pq = pq0 + r / group;
        rlo[i] = max(wlo, pq - W + 1);
        rhi[i] = min(whi, pq);
    }

    const long long tfirst = floor_div(wlo, kTile);
    const int nt = (int)(floor_div(whi, kTile) - tfirst + 1);

    uint4 pk[L::IPT][2], pv[L::IPT][2];
    auto prefetch = [&](long long tile) {
        const long long TB = tile * kTile;
        const long long sb = MOD ? (TB % a.g.slots) : (TB - avail);
#pragma unroll
        for (int it = 0; it < L::IPT; ++it) {
            const int item = threadIdx.x + it * 256;
            const int jp = item / L::CPR, c = item - jp * L::CPR;
#pragma unroll
            for (int r = 0; r < 2; ++r) {
                const long long pos = TB + 2 * jp + r;
                if (pos >= wlo && pos <= whi) {
                    const long long off = (sb + 2 * jp + r) * (D * E::E) + 16 * c;
                    pk[it][r] = *(const uint4*)(Kg + off);
                    pv[it][r] = *(const uint4*)(Vg + off);
                } else {
                    pk[it][r] = make_uint4(0, 0, 0, 0);
                    pv[it][r] = make_uint4(0, 0, 0, 0);
                }
            }
        }
    };
    auto commit = [&](int buf) {
        uint32_t* Kb = lds + buf * L::BUF;
        uint32_t* Vb = Kb + L::KDW;
#pragma unroll
        for (int it = 0; it < L::IPT; ++it) {
            const int item = threadIdx.x + it * 256;
            const int jp = item / L::CPR, c = item - jp * L::CPR;
            *(uint4*)(Kb + (2 * jp) * L::KP + 4 * c) = pk[it][0];
            *(uint4*)(Kb + (2 * jp + 1) * L::KP + 4 * c) = pk[it][1];
            const uint32_t w0[4] = {pv[it][0].x, pv[it][0].y, pv[it][0].z, pv[it][0].w};
            const uint32_t w1[4] = {pv[it][1].x, pv[it][1].y, pv[it][1].z, pv[it][1].w};
            if constexpr (E::E == 2) {
                // chunk c holds dims 8c .. 8c+7; V^T word (dim, key pair jp)
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    const uint32_t lo = (e & 1) ? (w0[e >> 1] >> 16) : (w0[e >> 1] & 0xffffu);
                    const uint32_t hi = (e & 1) ? (w1[e >> 1] & 0xffff0000u) : (w1[e >> 1] << 16);
                    Vb[(8 * c + e) * L::VP + jp] = lo | hi;
                }
            } else {
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    Vb[(4 * c + e) * L::VP + 2 * jp] = w0[e];
                    Vb[(4 * c + e) * L::VP + 2 * jp + 1] = w1[e];
                }
            }
        }
    };

    prefetch(tfirst);
    commit(0);
    __syncthreads();
    for (int it = 0; it < nt; ++it) {
        if (it + 1 < nt) prefetch(tfirst + it + 1);
        const uint32_t* Kb = lds + (it & 1) * L::BUF;
        const uint32_t* Vb = Kb + L::KDW;
        const long long TB = (tfirst + it) * kTile;
#pragma unroll
        for (int i = 0; i < RPW; ++i) {
            const int r = wave + 4 * i;
            if (r >= R) break;
            const int lo = (int)max(-1LL, min(64LL, rlo[i] - TB));
            const int hi = (int)max(-1LL, min(64LL, rhi[i] - TB));
            if (hi < 0 || lo > 63 || lo > hi) continue;  // no key of this tile for the row
            // scores: lane = key
            float s = 0.f;
            const uint32_t* krow = Kb + lane * L::KP;
            const uint32_t* qrow = Qs + r * L::ROWDW;
#pragma unroll
            for (int c4 = 0; c4 < L::ROWDW / 4; ++c4) {
                const uint4 kv = *(const uint4*)(krow + 4 * c4);
                const uint4 qv = *(const uint4*)(qrow + 4 * c4);
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
            lrow[i] = __fmaf_rn(lrow[i], alpha, wave_sum(p));
            mrow[i] = mn;
            if constexpr (E::E == 2) {
                ((uint16_t*)Pw)[lane] = (uint16_t)to_bf16(p);
            } else {
                ((float*)Pw)[lane] = p;
            }
            __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
            __builtin_amdgcn_wave_barrier();
            __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
            // weights: lane = output dim
#pragma unroll
            for (int k = 0; k < DPL; ++k) {
                const uint32_t* vrow = Vb + (lane + 64 * k) * L::VP;
                float o = acc[i][k] * alpha;
#pragma unroll
                for (int c4 = 0; c4 < kTile * E::E / 16; ++c4) {
                    const uint4 vv = *(const uint4*)(vrow + 4 * c4);
                    const uint4 pp = *(const uint4*)(Pw + 4 * c4);
                    if constexpr (E::E == 2) {
                        o = dot2bf(pp.x, vv.x, o);
                        o = dot2bf(pp.y, vv.y, o);
                        o = dot2bf(pp.z, vv.z, o);
                        o = dot2bf(pp.w, vv.w, o);
                    } else {
                        o = __fmaf_rn(__uint_as_float(pp.x), __uint_as_float(vv.x), o);
                        o = __fmaf_rn(__uint_as_float(pp.y), __uint_as_float(vv.y), o);
                        o = __fmaf_rn(__uint_as_float(pp.z), __uint_as_float(vv.z), o);
                        o = __fmaf_rn(__uint_as_float(pp.w), __uint_as_float(vv.w), o);
                    }
                }
                acc[i][k] = o;
            }
            __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
            __builtin_amdgcn_wave_barrier();
            __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
        }
        if (it + 1 < nt) commit((it + 1) & 1);
        __syncthreads();
    }

    // ---- epilogue
#pragma unroll
    for (int i = 0; i < RPW; ++i) {
        const int r = wave + 4 * i;
        if (r >= R) break;
        const int j = r / group, gh = r - j * group;
        if (SPLIT) {
            float* pr = a.partials +
                        (((cu * a.g.hkv + g) * a.n_splits + split) * group + r) * (long long)(2 + D);
            if (lane == 0) {
                pr[0] = mrow[i];
                pr[1] = lrow[i];
            }
#pragma unroll
            for (int k = 0; k < DPL; ++k) pr[2 + lane + 64 * k] = acc[i][k];
        } else {
            const int hq = g * group + gh;
            char* dst = (char*)a.out +
                        ((cu * m.n_total + m.t0 + (long long)qc * a.qchunk + j) * a.g.hq + hq) *
                            (long long)D * E::E;
#pragma unroll
            for (int k = 0; k < DPL; ++k) {
                const float o = acc[i][k] / lrow[i];
                const int d = lane + 64 * k;
                if constexpr (E::E == 2)
                    ((uint16_t*)dst)[d] = (uint16_t)to_bf16(o);
                else
                    ((float*)dst)[d] = o;
            }
        }
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
    for (int s = 0; s < ns; ++s) M = fmaxf(M, base[((long long)s * group + r) * (2 + D)]);
    float Lsum = 0.f, o[DPL];
#pragma unroll
    for (int k = 0; k < DPL; ++k) o[k] = 0.f;
    for (int s = 0; s < ns; ++s) {
        const float* pr = base + ((long long)s * group + r) * (2 + D);
        const float w = fast_exp2(pr[0] - M);
        Lsum = __fmaf_rn(pr[1], w, Lsum);
#pragma unroll
        for (int k = 0; k < DPL; ++k) o[k] = __fmaf_rn(pr[2 + lane + 64 * k], w, o[k]);
    }
    char* dst = (char*)a.out + ((cu * m.n_total + m.t0) * a.g.hq + hq) * (long long)D * E::E;
#pragma unroll
    for (int k = 0; k < DPL; ++k) {
        const float v = o[k] / Lsum;
        const int d = lane + 64 * k;
        if constexpr (E::E == 2)
            ((uint16_t*)dst)[d] = (uint16_t)to_bf16(v);
        else
            ((float*)dst)[d] = v;
    }
}

}  // namespace

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
            hipLaunchKernelGGL((k_rope_append<E_, D_, true>), grid, dim3(256), 0, s, a, t);
        else
            hipLaunchKernelGGL((k_rope_append<E_, D_, false>), grid, dim3(256), 0, s, a, t);
    });
    return hipGetLastError();
}

hipError_t launch_attn_valu(const AttnArgs& a, const StateTable& t, hipStream_t s) {
    const long long blocks =
        (long long)a.m.n_states * a.m.nl * a.g.hkv * a.n_qchunks * a.n_splits;
    const dim3 grid((unsigned)blocks);
    const bool split = a.n_splits > 1 || a.partials != nullptr;
    const bool app = a.append != 0;
    VRT_DISPATCH_ED(a.g.dtype, a.g.D, {
        if (a.g.mod && split && app)
            hipLaunchKernelGGL((k_attn_valu<E_, D_, true, true, true>), grid, dim3(256), 0, s, a, t);
        else if (a.g.mod && split)
            hipLaunchKernelGGL((k_attn_valu<E_, D_, true, true, false>), grid, dim3(256), 0, s, a, t);
        else if (a.g.mod && app)
            hipLaunchKernelGGL((k_attn_valu<E_, D_, true, false, true>), grid, dim3(256), 0, s, a, t);
        else if (a.g.mod)
            hipLaunchKernelGGL((k_attn_valu<E_, D_, true, false, false>), grid, dim3(256), 0, s, a, t);
        else if (app)
            hipLaunchKernelGGL((k_attn_valu<E_, D_, false, false, true>), grid, dim3(256), 0, s, a, t);
        else
            hipLaunchKernelGGL((k_attn_valu<E_, D_, false, false, false>), grid, dim3(256), 0, s, a, t);
    });
    return hipGetLastError();
}

hipError_t launch_dec_combine(const AttnArgs& a, const StateTable& t, hipStream_t s) {
    const dim3 grid((unsigned)(a.m.n_states * a.m.nl * a.g.hq));
    VRT_DISPATCH_ED(a.g.dtype, a.g.D, {
        hipLaunchKernelGGL((k_dec_combine<E_, D_>), grid, dim3(64), 0, s, a, t);
    });
    return hipGetLastError();
}

hipError_t launch_compact(const CompactArgs& a, const CompactTable& t, hipStream_t s) {
    const dim3 grid((unsigned)(a.n_entries * a.g.hkv * 2));
    VRT_DISPATCH_ED(a.g.dtype, a.g.D, {
        hipLaunchKernelGGL((k_compact<E_, D_>), grid, dim3(256), 0, s, a, t);
    });
    return hipGetLastError();
}

}  // namespace vrt
