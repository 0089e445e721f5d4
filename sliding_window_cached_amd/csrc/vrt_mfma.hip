// gfx950 matrix-core kernel of the windowed-causal attention: the catch-up
// path (sub-batches of 32 or more bf16 frames, head_dim 64, one query head
// per kv head).  The same attention, tile grid and window as the vector
// kernel in vrt_kernels.hip, so chunked feeding still reproduces the
// offline pass bit for bit whenever every sub-batch takes this path.
//
// Numerics: -ffp-contract=off for the whole library; every fused
// multiply-add is written out.
#include <hip/hip_runtime.h>

#include "vrt_device.h"
#include "vrt_internal.h"

namespace vrt {
namespace {

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
// nor a rescale on the vector ALU.  The denominator (the sum of the same bf16
// weights the products use) is a 16x16x32 matrix-core product as well.
// Every per-query step (the MFMA chains, the reference, the partial sums,
// the rescale) depends only on that query's own window and the absolute tile
// grid, so the result does not depend on how frames were batched.
//
// Queries are rotated in the prologue: the angle p * omega_i is formed in
// fp64 in revolutions and reduced to [-1/2, 1/2] there (three roundings of at
// most 2^-53 relative each: below 1.2e-7 revolutions for every position under
// 2^31), then sin and cos are taken in fp32 on the reduced angle (error below
// 1e-6 rad in all, far below the bf16 rounding of the rotated, scaled query
// that follows).
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
            // the angle in revolutions, reduced to [-1/2, 1/2]
            const double x = (pd * om[i]) * 0x1.45f306dc9c883p-3;
            const float r = (float)(x - rint(x));
            cs[i] = __builtin_amdgcn_cosf(r);
            sn[i] = __builtin_amdgcn_sinf(r);
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

    // ---- bands relative to T0: the wave's union / intersection (for
    // skipping and for mask-free half-tiles), and the lane's own band
    // [max(alo, h - W + 1), h] with h the position of its query (lanes past
    // the last query repeat it), for the edge half-tiles
    const int hq0 = (int)(pq0 + qw0 - T0), alo = (int)(avail - T0);
    const long long wq_first = pq0 + qw0, wq_last = pq0 + qw0 + max(nqw, 1) - 1;
    const int blo = (int)(max(avail, wq_first - W + 1) - T0), bhi = (int)(wq_last - T0);
    const int flo = (int)(max(avail, wq_last - W + 1) - T0), fhi = (int)(wq_first - T0);
    const int bhi_v = hq0 + jj;
    const int blo_v = max(alo, bhi_v - W + 1);

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
    // The softmax denominator runs on the matrix cores: a 16x16x32 product
    // takes a PV step's 16-key weight operand as its B operand.  Read that
    // way, lane l's eight weights are k = 8 (l / 16) + i of column l % 16, so
    // with ones in row 0 of A at k in [0, 8) and [16, 24) (lanes 0 and 32) and
    // in row 1 at k in [8, 16) and [24, 32) (lanes 17 and 49), row 0 of the
    // result is the weight sum over the 16 keys of query l % 16 and row 1 that
    // of query 16 + l % 16: registers 0 and 1 of lane l % 16.  The sums are of
    // the same bf16 weights the output products use.
    const uint32_t one16 = (lane == 0 || lane == 32 || lane == 17 || lane == 49) ? 0x3f803f80u : 0u;
    const bf16x8_t ones16 = __builtin_bit_cast(bf16x8_t, make_uint4(one16, one16, one16, one16));
    typedef float f32x4_t __attribute__((ext_vector_type(4)));
    f32x4_t den = {0.f, 0.f, 0.f, 0.f};
    float mref = 0.f;
    float thr = kSent;   // the reference moves when a half-tile's maximum exceeds it

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
                // register r holds key tb + 32k + 4hf + c with c = 8(r/4) + r%4:
                // bit c of vis says whether that key is in the query's band
                const int lo = blo_v - (tb + 32 * k + 4 * hf), hi = bhi_v - (tb + 32 * k + 4 * hf);
                const int lo_c = min(max(lo, 0), 31), hi_c = min(hi + 1, 28);
                const int width = max(hi_c - lo_c, 0);
                const unsigned vis = ((1u << width) - 1u) << lo_c;
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int c = 8 * (r >> 2) + (r & 3);
                    // bit c sign-extended to all ones or zero; an opaque value, so the
                    // select stays one bitfield insert instead of a compare and a select
                    unsigned keep;
                    asm("v_bfe_i32 %0, %1, %2, 1" : "=v"(keep) : "v"(vis), "n"(c));
                    s[r] = __uint_as_float((__float_as_uint(s[r]) & keep) | (__float_as_uint(kSent) & ~keep));
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
            const bool move = mt > thr;
            if (__builtin_amdgcn_ballot_w64(move) != 0) {   // a query's first keys, or a jump of 2^kLazy
                // a lane that had seen keys before rescales its sums; before
                // its first visible key a lane's sums are exactly zero (every
                // weight it added was 0), so a wave whose moving lanes all see
                // their first keys skips the rescale
                const bool jump = move && thr > kSent;
                float delta = 0.f, alpha = 1.f;
                if (move) {
                    const float mnew = mref + mt;
                    const uint32_t hi = to_bf16(mnew);
                    const float mhi = __uint_as_float(hi << 16);
                    const uint32_t lo = to_bf16(mnew - mhi);
                    const float mt_ref = mhi + __uint_as_float(lo << 16);
                    if (jump) alpha = fast_exp2(mref - mt_ref);
                    delta = mt_ref - mref;
                    mref = mt_ref;
                    thr = kLazy;
                    const uint32_t neg = (hi ^ 0x8000u) | ((lo ^ 0x8000u) << 16);
                    qext = __builtin_bit_cast(bf16x8_t, make_uint4(hf == 0 ? neg : 0u, 0u, 0u, 0u));
                }
                if (__builtin_amdgcn_ballot_w64(jump) != 0) {
#pragma unroll
                    for (int d = 0; d < 2; ++d)
#pragma unroll
                        for (int r = 0; r < 16; ++r) o[d][r] *= alpha;
                    // the denominators of queries jq and jq + 16 live in lane
                    // jq % 16 (registers 0 and 1): rescaled with those queries'
                    // alpha, exchanged outside the divergent branch
                    const float a_lo = __shfl(alpha, lane & 15), a_hi = __shfl(alpha, (lane & 15) + 16);
                    den[0] *= a_lo;
                    den[1] *= a_hi;
                }
#pragma unroll
                for (int r = 0; r < 16; ++r) s[r] -= delta;
            }
            uint32_t pb[8];
#pragma unroll
            for (int w = 0; w < 8; ++w) pb[w] = pack_bf16x2(fast_exp2(s[2 * w]), fast_exp2(s[2 * w + 1]));
            // O^T += V^T P^T and the denominators, key groups in ascending order
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
                den = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ones16, pv, den, 0, 0, 0);
            }
        }
    }

    // ---- epilogue: the denominator of query jq, register jq / 16 of lane jq % 16
    const float d0 = __shfl(den[0], jq & 15), d1 = __shfl(den[1], jq & 15);
    const float l = jq < 16 ? d0 : d1;
    // The rows go through LDS (row stride OS: 16-byte aligned, banks spread)
    // and the workgroup writes each 128-byte output row whole, 16 bytes per
    // lane, with the non-temporal hint.  Each lane storing its 8-byte pieces
    // directly cost the catch-up step 2.6 %; with the hint on those pieces,
    // 35 %.
    constexpr int OS = L::RB + 16;
    static_assert(L::QT * OS <= L::BYTES, "output rows fit the stages");
    __syncthreads();   // every wave is done with the last tile's stage
    if (nqw > 0 && jq < nqw) {
        // one reciprocal per query instead of 32 divisions (the outputs are
        // rounded to bf16 right after)
        const float rl = 1.0f / l;
        char* srow = lds + (qw0 + jq) * OS;
#pragma unroll
        for (int d = 0; d < 2; ++d)
#pragma unroll
            for (int q4 = 0; q4 < 4; ++q4) {
                uint2 v;
                v.x = pack_bf16x2(o[d][4 * q4] * rl, o[d][4 * q4 + 1] * rl);
                v.y = pack_bf16x2(o[d][4 * q4 + 2] * rl, o[d][4 * q4 + 3] * rl);
                *(uint2*)(srow + 2 * (32 * d + 8 * q4 + 4 * hf)) = v;
            }
    }
    __syncthreads();
    // row x of the tile is query qc * QT + x, frame m.t0 + qc * QT + x
    for (int x = threadIdx.x; x < nq * L::CPR; x += blockDim.x) {
        const int row = x / L::CPR, c = x % L::CPR;
        const long long fr = m.t0 + (long long)qc * L::QT + row;
        char* dst = (char*)a.out + ((cu * m.n_total + fr) * a.g.hq + g) * (long long)L::RB + 16 * c;
        gst_nt<uint4>(dst, *(const uint4*)(lds + row * OS + 16 * c));
    }
}

}  // namespace

hipError_t launch_attn_mfma(const AttnArgs& a, const StateTable& t, hipStream_t s) {
    if (a.g.dtype != 1 || a.g.D != 64 || a.g.group != 1 || a.n_splits != 1)
        return hipErrorInvalidValue;
    const long long blocks = (long long)a.m.n_states * a.m.nl * a.g.hkv * a.n_qchunks;
    VRT_LAUNCH(k_attn_mfma, dim3((unsigned)blocks), dim3(256), 0, s, a, t);
    return hipSuccess;
}

}  // namespace vrt
