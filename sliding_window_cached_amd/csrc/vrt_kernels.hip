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
//   k_attn_mfma    (vrt_mfma.hip) the same attention for sub-batches of 32 or
//                  more bf16 frames (the catch-up path), with both products
//                  on the matrix cores and the same absolute tile grid.
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

#include "vrt_device.h"
#include "vrt_internal.h"

namespace vrt {
namespace {

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
    static constexpr int QCAP = attn_qs_bytes(RB);   // rotated query rows of the head group
    static constexpr int BYTES = NST * 2 * TILE + QCAP + 4 * PRB;
};
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
    // split mode: (m, l) of every row of the group's heads, written out as one
    // 128-byte line per head after the last head
    __shared__ float mls[SPLIT ? 2 * (L::QCAP / L::RB) : 1];
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
            // the new rows go out with the non-temporal hint (st4_ring, gst_nt)
            char* Kg = layer + (long long)g * a.g.slice_bytes;
            char* Vg = Kg + a.g.v_off;
            const long long slot = MOD ? (pos % a.g.slots) : (long long)(nkv + j);
#pragma unroll
            for (int q = 0; q < 4; ++q) rope_pair(it.k0[q], it.k1[q], an[q], &y0[q], &y1[q]);
            char* kd = Kg + slot * L::RB;
            st4_ring<E>(kd + 4 * c * E::E, y0);
            st4_ring<E>(kd + (H2 + 4 * c) * E::E, y1);
#pragma unroll
            for (int u = 0; u < L::CPR / CG; ++u)
                gst_nt<uint4>(Vg + slot * L::RB + 16 * (c + u * CG), it.vch[u]);
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
                    float* rec = a.partials + ((cu * a.g.hkv + g) * a.n_splits + split) * dec_record_floats(group, D);
                    if (lane == 0) {
                        mls[(hh * R + r) * 2] = mrow[i];
                        mls[(hh * R + r) * 2 + 1] = lrow;
                    }
#pragma unroll
                    for (int k = 0; k < DPL; ++k) gst_nt<float>(rec + kMlFloats + r * D + lane + 64 * k, acc[i][k]);
                } else if constexpr (!LOOK) {
                    // the output row goes to this wave's own query row of the
                    // head, which nothing reads any more; the workgroup writes
                    // all of them after the last head
                    char* srow = Qs + (hh * R + r) * L::RB;
#pragma unroll
                    for (int k = 0; k < DPL; ++k) {
                        const float o = acc[i][k] / lrow;
                        const int d = lane + 64 * k;
                        if constexpr (E::E == 2)
                            *(uint16_t*)(srow + 2 * d) = (uint16_t)to_bf16(o);
                        else
                            *(float*)(srow + 4 * d) = o;
                    }
                } else {
                    const int hq = g * group + gh;
                    const long long orow = (long long)a.look_o0 + (long long)qc * a.qchunk + j;
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

    // ---- split mode: the (m, l) line of each head's partial record, 2 R
    // values then zeros, written whole
    if constexpr (SPLIT) {
        __syncthreads();   // every wave's (m, l) are in mls
        for (int x = threadIdx.x; x < hg * kMlFloats; x += blockDim.x) {
            const int hh = x / kMlFloats, f = x - hh * kMlFloats;
            float* rec = a.partials + ((cu * a.g.hkv + g0 + hh) * a.n_splits + split) * dec_record_floats(group, D);
            gst_nt<float>(rec + f, f < 2 * R ? mls[hh * 2 * R + f] : 0.f);
        }
    }
    // ---- outputs: 16-byte stores of the staged rows.  The rows of query j
    // for the group's heads are adjacent in `out` (q heads g0 * group onwards),
    // so consecutive threads write consecutive bytes.  Written once at the end
    // instead of one 2- or 4-byte element per lane at each head's end: on the
    // 256-stream serving step that made the launch 2 % faster.
    if constexpr (!SPLIT && !LOOK) {
        __syncthreads();   // every wave's output rows are in Qs
        const long long orow0 = (long long)m.t0 + (long long)qc * a.qchunk;
        for (int x = threadIdx.x; x < hg * R * L::CPR; x += blockDim.x) {
            const int c = x % L::CPR, rest = x / L::CPR;
            const int gh = rest % group, hh = (rest / group) % hg, j = rest / (group * hg);
            const uint4 v = *(const uint4*)(Qs + (hh * R + j * group + gh) * L::RB + 16 * c);
            char* dst = (char*)a.out +
                        ((cu * m.n_total + orow0 + j) * a.g.hq + (long long)(g0 + hh) * group + gh) * (long long)L::RB;
            gst<uint4>(dst + 16 * c, v);
        }
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
    const long long rec = dec_record_floats(group, D);
    const float* base = a.partials + ((cu * a.g.hkv + g) * a.n_splits) * rec;
    float M = kSent;
    for (int s = 0; s < ns; ++s) M = fmaxf(M, gld<float>(base + s * rec + 2 * r));
    float Lsum = 0.f, o[DPL];
#pragma unroll
    for (int k = 0; k < DPL; ++k) o[k] = 0.f;
    for (int s = 0; s < ns; ++s) {
        const float* pr = base + s * rec;
        const float w = fast_exp2(gld<float>(pr + 2 * r) - M);
        Lsum = __fmaf_rn(gld<float>(pr + 2 * r + 1), w, Lsum);
#pragma unroll
        for (int k = 0; k < DPL; ++k) o[k] = __fmaf_rn(gld<float>(pr + kMlFloats + r * D + lane + 64 * k), w, o[k]);
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
