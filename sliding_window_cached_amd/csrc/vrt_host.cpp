// C-ABI host side: argument checks, the host mirror of every ring, sub-batch
// splitting, compaction decisions and launch planning.  Device work is only
// enqueued after every check has passed; the mirrors advance as it is
// enqueued, so no call ever reads anything back from the GPU.
#include <algorithm>
#include <atomic>
#include <climits>
#include <cmath>
#include <cstdio>
#include <cstring>
#include <new>
#include <vector>

#include "vrt.h"
#include "vrt_internal.h"

struct vrt_stream_state {
    vrt_cache_desc d;
    char* dev;
    size_t bytes;
    std::vector<int64_t> abs_base;  // per layer: position held in slot 0 (decoder: first position)
    std::vector<int32_t> n_kv;      // per layer: rows held (decoder: tokens written)
    bool poisoned;
};

namespace {

// Testing hook (vrt_test_launch_hook): the launch that fails (1-based count
// since the hook was set; 0 none), whether launches are skipped (dry run),
// and the launches that reached the gate since the hook was last set.
thread_local int32_t g_fail_at = 0;
thread_local int32_t g_dry = 0;
thread_local int64_t g_launches = 0;

// Compute units and LDS bytes per CU of each device, read once.
constexpr int kMaxDevices = 64;
std::atomic<int> g_cus[kMaxDevices];
std::atomic<int> g_lds[kMaxDevices];

void device_props(int* cus, int* lds) {
    *cus = 256;
    *lds = 160 * 1024;
    int dev = 0;
    if (g_dry || hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return;
    int c = g_cus[dev].load(std::memory_order_relaxed), l = g_lds[dev].load(std::memory_order_relaxed);
    if (c <= 0 || l <= 0) {
        if (hipDeviceGetAttribute(&c, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || c <= 0)
            c = 256;
        if (hipDeviceGetAttribute(&l, hipDeviceAttributeMaxSharedMemoryPerMultiprocessor, dev) !=
                hipSuccess ||
            l <= 0)
            l = 160 * 1024;
        g_cus[dev].store(c, std::memory_order_relaxed);
        g_lds[dev].store(l, std::memory_order_relaxed);
    }
    *cus = c;
    *lds = l;
}

}  // namespace

namespace vrt {

int launch_gate(hipError_t* e) {
    ++g_launches;
    if (g_fail_at > 0 && g_launches == g_fail_at) {
        *e = hipErrorLaunchFailure;
        return 0;
    }
    if (g_dry) {
        *e = hipSuccess;
        return 0;
    }
    return 1;
}

int device_cus() {
    int c, l;
    device_props(&c, &l);
    return c;
}

int device_lds() {
    int c, l;
    device_props(&c, &l);
    return l;
}

}  // namespace vrt

namespace {

using namespace vrt;

// Absolute positions stay below 2^31 (about 1.4 years of 50 Hz encoder
// frames); the query rotation of the matrix path reduces its angles exactly
// up to this bound.
constexpr int64_t kPosLimit = (int64_t)1 << 31;

// Text of the last HIP error a launch on this thread reported (diagnostics
// only; read through vrt_last_device_error).
thread_local char g_last_error[256] = "";

hipError_t note(hipError_t e) {
    if (e != hipSuccess) {
        std::snprintf(g_last_error, sizeof g_last_error, "%s (%d)", hipGetErrorString(e), (int)e);
    }
    return e;
}

// Optional timing events recorded around attention launches
// (vrt_set_attn_events); null when off.
thread_local hipEvent_t g_ev_start = nullptr;
thread_local hipEvent_t g_ev_stop = nullptr;

hipError_t record_start(hipStream_t s) {
    return g_ev_start && !g_dry ? hipEventRecord(g_ev_start, s) : hipSuccess;
}
hipError_t record_stop(hipStream_t s) {
    return g_ev_stop && !g_dry ? hipEventRecord(g_ev_stop, s) : hipSuccess;
}

// A HIP error code is sticky per thread: an earlier failed runtime call made
// by someone else would otherwise be reported after our own launch.  Clear it
// once before a call enqueues anything.
void clear_sticky_error() {
    if (!g_dry) (void)hipGetLastError();
}

int elem_bytes(const vrt_cache_desc& d) { return d.dtype == VRT_BF16 ? 2 : 4; }

bool same_desc(const vrt_cache_desc& a, const vrt_cache_desc& b) {
    return a.kind == b.kind && a.dtype == b.dtype && a.n_layers == b.n_layers &&
           a.lookahead == b.lookahead &&
           a.n_heads_q == b.n_heads_q && a.n_heads_kv == b.n_heads_kv &&
           a.head_dim == b.head_dim && a.window == b.window && a.ring_slots == b.ring_slots &&
           a.max_batch == b.max_batch && a.rope_theta == b.rope_theta;
}

vrt_status check_desc(const vrt_cache_desc* d) {
    if (!d) return VRT_ERR_INVALID;
    if (d->kind != VRT_ENC_RING && d->kind != VRT_DEC_MODRING && d->kind != VRT_ENC_MODRING &&
        d->kind != VRT_ENC_LOOKAHEAD)
        return VRT_ERR_UNSUPPORTED;
    const bool look = d->kind == VRT_ENC_LOOKAHEAD;
    if (look ? (d->lookahead < 0 || d->lookahead > (1 << 16)) : d->lookahead != 0) return VRT_ERR_INVALID;
    if (d->dtype != VRT_F32 && d->dtype != VRT_BF16) return VRT_ERR_UNSUPPORTED;
    if (d->n_layers < 1 || d->n_heads_q < 1 || d->n_heads_kv < 1 || d->window < 1 ||
        d->ring_slots < 1 || d->max_batch < 1)
        return VRT_ERR_INVALID;
    if (d->n_heads_q % d->n_heads_kv != 0) return VRT_ERR_INVALID;
    if (look ? d->rope_theta != 0.0 : (!(d->rope_theta > 1.0) || !std::isfinite(d->rope_theta)))
        return VRT_ERR_INVALID;
    // head_dim 64 or 128; the lookahead kind (no rotation) also takes any
    // multiple of 8 below 64, its ring rows padded to 64 elements
    if (d->head_dim != 64 && d->head_dim != 128 &&
        !(look && d->head_dim >= 8 && d->head_dim < 64 && d->head_dim % 8 == 0))
        return VRT_ERR_UNSUPPORTED;
    const int group = d->n_heads_q / d->n_heads_kv;
    if (group > kRows) return VRT_ERR_UNSUPPORTED;
    if (d->ring_slots > (1 << 24) || d->window > (1 << 24) || d->max_batch > (1 << 20))
        return VRT_ERR_UNSUPPORTED;
    if (d->kind == VRT_ENC_RING) {
        if ((int64_t)d->ring_slots < (int64_t)d->window + d->max_batch) return VRT_ERR_UNSUPPORTED;
    } else if (look) {
        // the oldest key a sub-batch's first answered query reads lies
        // window - 1 + F frames before the sub-batch's newest frame
        const int64_t f = std::max(d->lookahead - 1, 0);
        if ((int64_t)d->ring_slots < (int64_t)d->window + f + d->max_batch - 1 ||
            d->ring_slots % kTile != 0)
            return VRT_ERR_UNSUPPORTED;
    } else if (d->kind == VRT_ENC_MODRING) {
        // a sub-batch of max_batch frames, written before its attention, must
        // not overwrite the oldest key (window - 1 back) its first query reads
        if ((int64_t)d->ring_slots < (int64_t)d->window - 1 + d->max_batch ||
            d->ring_slots % kTile != 0)
            return VRT_ERR_UNSUPPORTED;
    } else {
        if (d->ring_slots < d->window || d->ring_slots % kTile != 0) return VRT_ERR_UNSUPPORTED;
    }
    return VRT_OK;
}

bool is_encoder(const vrt_cache_desc& d) {
    return d.kind == VRT_ENC_RING || d.kind == VRT_ENC_MODRING || d.kind == VRT_ENC_LOOKAHEAD;
}
// future frames a query of a lookahead cache waits for (0 for other kinds)
int look_f(const vrt_cache_desc& d) {
    return d.kind == VRT_ENC_LOOKAHEAD ? std::max(d.lookahead - 1, 0) : 0;
}
size_t pend_layer_bytes(const vrt_cache_desc& d) {
    return (size_t)look_f(d) * d.n_heads_q * d.head_dim * (d.dtype == VRT_BF16 ? 2 : 4);
}

// elements per ring row: head_dim, or 64 for a lookahead head_dim below 64
// (rows padded with zeros, so the kernels see a 64-element head)
int ring_dim(const vrt_cache_desc& d) { return d.head_dim < 64 ? 64 : d.head_dim; }

size_t slice_bytes(const vrt_cache_desc& d) {
    return (size_t)d.ring_slots * ring_dim(d) * elem_bytes(d);
}
size_t layer_bytes(const vrt_cache_desc& d) { return 2 * (size_t)d.n_heads_kv * slice_bytes(d); }

Geom make_geom(const vrt_cache_desc& d) {
    Geom g;
    g.dtype = d.dtype;
    g.D = ring_dim(d);
    g.Dio = d.head_dim;
    g.hq = d.n_heads_q;
    g.hkv = d.n_heads_kv;
    g.group = d.n_heads_q / d.n_heads_kv;
    g.slots = d.ring_slots;
    g.window = d.window;
    g.mod = d.kind == VRT_ENC_RING ? 0 : 1;
    g.rope = d.kind == VRT_ENC_LOOKAHEAD ? 0 : 1;
    g.slice_bytes = (long long)slice_bytes(d);
    g.v_off = (long long)d.n_heads_kv * g.slice_bytes;
    g.layer_bytes = 2 * g.v_off;
    for (int i = 0; i < 64; ++i)
        g.omega[i] = (g.rope && i < d.head_dim / 2) ? std::pow(d.rope_theta, -2.0 * i / d.head_dim) : 0.0;
    return g;
}

// log2(e) / sqrt(head_dim): the softmax scale of the head as given (40 for a
// 40-wide head stored in 64-element rows)
float scale_log2(int D) { return (float)(1.4426950408889634 / std::sqrt((double)D)); }


// kv heads per attention workgroup: the largest divisor of hkv whose rotated
// query rows fit the workgroup's LDS budget and that still leaves a full
// round of workgroups (as many per CU as the kernel's LDS allows, at most 4),
// so each workgroup streams a long run of tiles through one pipeline.
int pick_hg(const Geom& g, long long units, int rows_per_head, long long qchunks, long long splits) {
    int cus, lds;
    device_props(&cus, &lds);
    const int elem = g.dtype == 1 ? 2 : 4;
    const int qs = attn_qs_bytes(g.D * elem);
    const long long wg_lds = (long long)attn_stages(g.dtype, g.D, splits > 1) * 2 * kTile * g.D * elem + qs +
                             4 * kTile * elem;
    const long long per_cu = std::max(1LL, std::min(4LL, lds / wg_lds));
    const long long target = per_cu * cus;
    int best = 1;
    for (int h = 2; h <= g.hkv; ++h) {
        if (g.hkv % h) continue;
        if ((long long)h * rows_per_head * g.D * elem > qs) break;
        if (units * (g.hkv / h) * qchunks * splits < target) break;
        best = h;
    }
    return best;
}

// Arithmetic path of one sub-batch of n frames: a pure function of the cache
// description and n, so two feeds that split a sequence differently but take
// the same path produce bit-identical outputs.
bool use_mfma(const vrt_cache_desc& d, int n) {
    return is_encoder(d) && d.kind != VRT_ENC_LOOKAHEAD && d.dtype == VRT_BF16 && d.head_dim == 64 &&
           d.n_heads_q == d.n_heads_kv && n >= kMfmaMinFrames;
}

// Attention launch parameters of a sub-batch of n frames over `units` units.
void attn_shape(const Geom& g, bool mfma, long long units, int n, AttnArgs* at) {
    at->partials = nullptr;
    at->n_splits = 1;
    at->split_len = kSplitLen;
    at->scale_log2 = scale_log2(g.Dio);
    if (mfma) {
        at->qchunk = kQTileMfma;
        at->n_qchunks = (n + kQTileMfma - 1) / kQTileMfma;
        at->append = 0;
        at->hg = 1;
        return;
    }
    at->qchunk = kRows / g.group;
    at->n_qchunks = (n + at->qchunk - 1) / at->qchunk;
    // one query chunk per unit: the attention launch appends the new rows
    // itself; otherwise a separate append launch runs first
    at->append = at->n_qchunks == 1 ? 1 : 0;
    at->hg = pick_hg(g, units, std::min(at->qchunk, n) * g.group, at->n_qchunks, 1);
}

// Attention launch parameters of a decoder sub-batch of m tokens over
// `units` units: a single token is split over keys (split-K, merged after),
// a prefill is not.
void dec_shape(const Geom& g, long long units, int m, AttnArgs* at) {
    at->split_len = kSplitLen;
    at->scale_log2 = scale_log2(g.Dio);
    if (m == 1) {
        at->qchunk = 1;
        at->n_qchunks = 1;
        at->n_splits = (g.window + kSplitLen - 2) / kSplitLen + 1;
    } else {
        at->partials = nullptr;
        at->qchunk = kRows / g.group;
        at->n_qchunks = (m + at->qchunk - 1) / at->qchunk;
        at->n_splits = 1;
    }
    at->append = at->n_qchunks == 1 ? 1 : 0;
    at->hg = pick_hg(g, units, std::min(at->qchunk, m) * g.group, at->n_qchunks, at->n_splits);
}

hipError_t launch_attn(const AttnArgs& at, bool mfma, const StateTable& t, hipStream_t s) {
    hipError_t e = record_start(s);
    if (e == hipSuccess) e = mfma ? launch_attn_mfma(at, t, s) : launch_attn_valu(at, t, s);
    if (e == hipSuccess) e = record_stop(s);
    return e;
}

// Common checks for the batched calls.  Pure: touches nothing.
vrt_status check_batch(vrt_stream_state* const* st, int n_states, int layer0, int n_layers,
                       int kind) {
    if (!st || n_states < 1 || !st[0]) return VRT_ERR_INVALID;
    const vrt_cache_desc& d = st[0]->d;
    if (d.kind != kind) return VRT_ERR_INVALID;
    if (layer0 < 0 || n_layers < 1 || layer0 > d.n_layers - n_layers) return VRT_ERR_INVALID;
    std::vector<const vrt_stream_state*> seen;
    seen.reserve(n_states);
    for (int i = 0; i < n_states; ++i) {
        if (!st[i]) return VRT_ERR_INVALID;
        if (!same_desc(st[i]->d, d)) return VRT_ERR_INVALID;
        seen.push_back(st[i]);
    }
    std::sort(seen.begin(), seen.end());
    if (std::adjacent_find(seen.begin(), seen.end()) != seen.end()) return VRT_ERR_INVALID;
    for (int i = 0; i < n_states; ++i)
        if (st[i]->poisoned) return VRT_ERR_POISONED;
    return VRT_OK;
}

std::vector<int> split_feed(int n, int max_batch) {
    std::vector<int> out;
    for (int t = 0; t < n; t += max_batch) out.push_back(std::min(max_batch, n - t));
    return out;
}

// One kernel launch's worth of units: a list of states (by call index) and a
// layer range relative to the call's layer0.  All layers of a state in one
// launch share (abs_base, n_kv).
struct Plan {
    std::vector<int> states;
    int l_off, nl;
};

// Group the call's units into launches.  A state whose layers all hold the
// same (abs_base, n_kv) goes into an all-layer launch; a state whose layers
// differ is launched layer by layer.
std::vector<Plan> plan_launches(vrt_stream_state* const* st, int n_states, int layer0,
                                int n_layers) {
    std::vector<Plan> plans;
    std::vector<int> uniform, ragged;
    for (int i = 0; i < n_states; ++i) {
        bool u = true;
        for (int l = 1; l < n_layers && u; ++l)
            u = st[i]->abs_base[layer0 + l] == st[i]->abs_base[layer0] &&
                st[i]->n_kv[layer0 + l] == st[i]->n_kv[layer0];
        (u ? uniform : ragged).push_back(i);
    }
    for (size_t b = 0; b < uniform.size(); b += kMaxStates) {
        Plan p;
        p.states.assign(uniform.begin() + b,
                        uniform.begin() + std::min(uniform.size(), b + (size_t)kMaxStates));
        p.l_off = 0;
        p.nl = n_layers;
        plans.push_back(p);
    }
    for (int l = 0; l < n_layers && !ragged.empty(); ++l)
        for (size_t b = 0; b < ragged.size(); b += kMaxStates) {
            Plan p;
            p.states.assign(ragged.begin() + b,
                            ragged.begin() + std::min(ragged.size(), b + (size_t)kMaxStates));
            p.l_off = l;
            p.nl = 1;
            plans.push_back(p);
        }
    return plans;
}

void fill_table(const Plan& p, vrt_stream_state* const* st, int layer, StateTable* t) {
    for (size_t i = 0; i < p.states.size(); ++i) {
        const vrt_stream_state* s = st[p.states[i]];
        t->ring[i] = (unsigned long long)(uintptr_t)s->dev;
        t->p0[i] = s->abs_base[layer] + s->n_kv[layer];
        t->n_kv[i] = s->n_kv[layer];
        t->call_idx[i] = p.states[i];
    }
}

void poison(vrt_stream_state* const* st, int n) {
    for (int i = 0; i < n; ++i) st[i]->poisoned = true;
}

// Enqueue compaction of the given (state, layer) rings and advance their
// mirrors.  `which` lists (call index, layer) pairs with n_kv > window.
hipError_t run_compactions(vrt_stream_state* const* st,
                           const std::vector<std::pair<int, int>>& which, hipStream_t stream) {
    if (which.empty()) return hipSuccess;
    const vrt_cache_desc& d = st[which[0].first]->d;
    CompactArgs a;
    a.g = make_geom(d);
    a.kept = d.window;
    CompactTable t;
    for (size_t b = 0; b < which.size(); b += kMaxCompact) {
        const size_t e = std::min(which.size(), b + (size_t)kMaxCompact);
        a.n_entries = (int)(e - b);
        for (size_t i = b; i < e; ++i) {
            vrt_stream_state* s = st[which[i].first];
            const int l = which[i].second;
            t.layer_ring[i - b] =
                (unsigned long long)(uintptr_t)(s->dev + (size_t)l * layer_bytes(d));
            t.shift[i - b] = s->n_kv[l] - d.window;
        }
        const hipError_t err = note(launch_compact(a, t, stream));
        if (err != hipSuccess) return err;
    }
    for (const auto& w : which) {
        vrt_stream_state* s = st[w.first];
        const int l = w.second;
        s->abs_base[l] += s->n_kv[l] - d.window;
        s->n_kv[l] = d.window;
    }
    return hipSuccess;
}

UnitMap make_map(const Plan& p, int layer0, int n_layers, int n_total, int t0, int n) {
    UnitMap m;
    m.n_states = (int)p.states.size();
    m.nl = p.nl;
    m.l_off = p.l_off;
    m.nl_call = n_layers;
    m.layer0 = layer0;
    m.n_total = n_total;
    m.t0 = t0;
    m.n = n;
    return m;
}

}  // namespace

extern "C" {

const char* vrt_status_str(vrt_status s) {
    switch (s) {
        case VRT_OK: return "ok";
        case VRT_ERR_INVALID: return "invalid argument";
        case VRT_ERR_UNSUPPORTED: return "unsupported configuration";
        case VRT_ERR_CAPACITY: return "insufficient capacity";
        case VRT_ERR_DEVICE: return "device error";
        case VRT_ERR_POISONED: return "state poisoned by an earlier device error";
    }
    return "unknown status";
}

const char* vrt_version(void) { return "vrt 0.1 gfx950"; }

const char* vrt_last_device_error(void) { return g_last_error; }

vrt_status vrt_desc_check(const vrt_cache_desc* desc) { return check_desc(desc); }

size_t vrt_state_device_bytes(const vrt_cache_desc* desc) {
    if (check_desc(desc) != VRT_OK) return 0;
    return (size_t)desc->n_layers * (layer_bytes(*desc) + pend_layer_bytes(*desc));
}

size_t vrt_ring_offset(const vrt_cache_desc* desc, int layer, int which, int kv_head) {
    if (check_desc(desc) != VRT_OK || layer < 0 || layer >= desc->n_layers || which < 0 ||
        which > 1 || kv_head < 0 || kv_head >= desc->n_heads_kv)
        return (size_t)-1;
    return (size_t)layer * layer_bytes(*desc) +
           ((size_t)which * desc->n_heads_kv + kv_head) * slice_bytes(*desc);
}

vrt_status vrt_stream_state_create(const vrt_cache_desc* desc, void* dev_mem, size_t bytes,
                                   int64_t start_pos, vrt_stream_state** out) {
    const vrt_status s = check_desc(desc);
    if (s != VRT_OK) return s;
    if (!out || !dev_mem || ((uintptr_t)dev_mem & 255) != 0) return VRT_ERR_INVALID;
    if (start_pos < 0 || start_pos >= kPosLimit) return VRT_ERR_INVALID;
    if (bytes < vrt_state_device_bytes(desc)) return VRT_ERR_CAPACITY;
    vrt_stream_state* st = new (std::nothrow) vrt_stream_state;
    if (!st) return VRT_ERR_CAPACITY;
    st->d = *desc;
    st->dev = (char*)dev_mem;
    st->bytes = bytes;
    st->abs_base.assign(desc->n_layers, start_pos);
    st->n_kv.assign(desc->n_layers, 0);
    st->poisoned = false;
    *out = st;
    return VRT_OK;
}

vrt_status vrt_stream_state_reset(vrt_stream_state* st, int64_t start_pos) {
    if (!st || start_pos < 0 || start_pos >= kPosLimit) return VRT_ERR_INVALID;
    std::fill(st->abs_base.begin(), st->abs_base.end(), start_pos);
    std::fill(st->n_kv.begin(), st->n_kv.end(), 0);
    st->poisoned = false;
    return VRT_OK;
}

void vrt_stream_state_destroy(vrt_stream_state* st) { delete st; }

vrt_status vrt_stream_state_query(const vrt_stream_state* st, int layer, int64_t* abs_base,
                                  int32_t* n_kv) {
    if (!st || layer < 0 || layer >= st->d.n_layers) return VRT_ERR_INVALID;
    if (abs_base) *abs_base = st->abs_base[layer];
    if (n_kv) *n_kv = st->n_kv[layer];
    return st->poisoned ? VRT_ERR_POISONED : VRT_OK;
}

vrt_status vrt_ring_advance(const vrt_cache_desc* desc, int64_t* abs_base, int32_t* n_kv,
                            int n_new, int32_t* n_compactions) {
    const vrt_status s = check_desc(desc);
    if (s != VRT_OK) return s;
    if (!is_encoder(*desc) || !abs_base || !n_kv || n_new < 0) return VRT_ERR_INVALID;
    if (desc->kind != VRT_ENC_RING) {   // modulo rings: n_kv counts every frame
        if (*n_kv < 0 || *abs_base < 0 || *abs_base + *n_kv > kPosLimit - n_new)
            return VRT_ERR_INVALID;
        *n_kv += n_new;
        if (n_compactions) *n_compactions = 0;
        return VRT_OK;
    }
    if (*n_kv < 0 || *n_kv > desc->ring_slots) return VRT_ERR_INVALID;
    int64_t base = *abs_base;
    int32_t nkv = *n_kv, nc = 0;
    for (int m : split_feed(n_new, desc->max_batch)) {
        if (nkv + m > desc->ring_slots) {
            base += nkv - desc->window;
            nkv = desc->window;
            ++nc;
        }
        nkv += m;
    }
    *abs_base = base;
    *n_kv = nkv;
    if (n_compactions) *n_compactions = nc;
    return VRT_OK;
}

int vrt_attn_out_frames(const vrt_cache_desc* desc, int32_t n_kv, int n_new) {
    if (check_desc(desc) != VRT_OK || !is_encoder(*desc) || n_kv < 0 || n_new < 0) return -1;
    const int f = look_f(*desc);
    return (int)(std::max<int64_t>(0, (int64_t)n_kv + n_new - f) - std::max<int64_t>(0, (int64_t)n_kv - f));
}

int vrt_attn_path(const vrt_cache_desc* desc, int n) {
    if (check_desc(desc) != VRT_OK || n < 1) return -1;
    return use_mfma(*desc, n) ? 1 : 0;
}

vrt_status vrt_attn_plan(const vrt_cache_desc* desc, int64_t units, int n, int32_t* heads_per_group,
                         int32_t* n_splits, int32_t* n_qchunks) {
    const vrt_status s = check_desc(desc);
    if (s != VRT_OK) return s;
    if (units < 1 || units > ((int64_t)1 << 40) || n < 1 || !heads_per_group || !n_splits || !n_qchunks)
        return VRT_ERR_INVALID;
    const Geom g = make_geom(*desc);
    AttnArgs at{};
    if (desc->kind == VRT_DEC_MODRING)
        dec_shape(g, (long long)units, n, &at);
    else
        attn_shape(g, use_mfma(*desc, n), (long long)units, n, &at);
    *heads_per_group = at.hg;
    *n_splits = at.n_splits;
    *n_qchunks = at.n_qchunks;
    return VRT_OK;
}

void vrt_test_launch_hook(int32_t fail_at, int32_t dry_run) {
    g_fail_at = fail_at > 0 ? fail_at : 0;
    g_dry = dry_run ? 1 : 0;
    g_launches = 0;
}

int64_t vrt_test_launch_count(void) { return g_launches; }

size_t vrt_offline_scratch_bytes(const vrt_cache_desc* desc, int T) {
    if (check_desc(desc) != VRT_OK || T < 1) return 0;
    return 2 * (size_t)desc->n_heads_kv * (size_t)T * ring_dim(*desc) * elem_bytes(*desc);
}

vrt_status vrt_enc_attn_offline(const vrt_cache_desc* desc, const void* q, const void* k,
                                const void* v, int T, int64_t start_pos, void* out,
                                void* scratch, size_t scratch_bytes, hipStream_t stream) {
    const vrt_status s = check_desc(desc);
    if (s != VRT_OK) return s;
    if (!is_encoder(*desc)) return VRT_ERR_INVALID;
    if (!q || !k || !v || !out || !scratch || T < 1) return VRT_ERR_INVALID;
    if (start_pos < 0 || start_pos > kPosLimit - T) return VRT_ERR_INVALID;
    if (scratch_bytes < vrt_offline_scratch_bytes(desc, T)) return VRT_ERR_CAPACITY;

    // The whole sequence is one linear "ring" of T slots in the scratch.
    Geom g = make_geom(*desc);
    g.slots = T;
    g.mod = 0;
    g.slice_bytes = (long long)T * ring_dim(*desc) * elem_bytes(*desc);
    g.v_off = (long long)desc->n_heads_kv * g.slice_bytes;
    g.layer_bytes = 2 * g.v_off;
    StateTable t;
    t.ring[0] = (unsigned long long)(uintptr_t)scratch;
    t.p0[0] = start_pos;
    t.n_kv[0] = 0;
    t.call_idx[0] = 0;
    Plan p;
    p.states = {0};
    p.l_off = 0;
    p.nl = 1;
    const UnitMap m = make_map(p, 0, 1, T, 0, T);

    AppendArgs aa;
    aa.g = g;
    aa.m = m;
    aa.k = k;
    aa.v = v;
    clear_sticky_error();
    if (note(launch_rope_append(aa, t, stream)) != hipSuccess) return VRT_ERR_DEVICE;

    AttnArgs at{};
    at.g = g;
    at.m = m;
    at.q = q;
    at.k = k;
    at.v = v;
    at.out = out;
    const bool mfma = use_mfma(*desc, T);
    attn_shape(g, mfma, 1, T, &at);
    at.append = 0;   // the append above already wrote every row
    at.look_f = look_f(*desc);   // lookahead: every frame answered, the last ones see the end
    at.look_nout = T;
    if (note(launch_attn(at, mfma, t, stream)) != hipSuccess) return VRT_ERR_DEVICE;
    return VRT_OK;
}

vrt_status vrt_enc_attn_feed(vrt_stream_state* const* st, int n_states, int layer0,
                             int n_layers, const void* q, const void* k, const void* v,
                             int n_new, void* out, hipStream_t stream) {
    if (!st || n_states < 1 || !st[0] || !is_encoder(st[0]->d)) return VRT_ERR_INVALID;
    vrt_status s = check_batch(st, n_states, layer0, n_layers, st[0]->d.kind);
    if (s != VRT_OK) return s;
    if (!q || !k || !v || !out || n_new < 1) return VRT_ERR_INVALID;
    for (int i = 0; i < n_states; ++i)
        for (int l = layer0; l < layer0 + n_layers; ++l)
            if (st[i]->abs_base[l] + st[i]->n_kv[l] > kPosLimit - n_new) return VRT_ERR_INVALID;

    const vrt_cache_desc& d = st[0]->d;
    const Geom g = make_geom(d);
    // lookahead: every (state, layer) of the call holds the same number of
    // waiting queries, so one launch answers the same count for all
    const int F = look_f(d);
    const int wait0 = (int)std::min<int64_t>(st[0]->n_kv[layer0], F);
    for (int i = 0; i < n_states; ++i)
        for (int l = layer0; l < layer0 + n_layers; ++l)
            if (std::min<int64_t>(st[i]->n_kv[l], F) != wait0) return VRT_ERR_INVALID;
    clear_sticky_error();
    int t0 = 0, o_written = 0;
    for (int m : split_feed(n_new, d.max_batch)) {
        int n_out_sb = m;
        std::vector<std::pair<int, int>> comp;
        if (d.kind == VRT_ENC_RING)
            for (int i = 0; i < n_states; ++i)
                for (int l = layer0; l < layer0 + n_layers; ++l)
                    if (st[i]->n_kv[l] + m > d.ring_slots) comp.emplace_back(i, l);
        if (run_compactions(st, comp, stream) != hipSuccess) {
            poison(st, n_states);
            return VRT_ERR_DEVICE;
        }
        for (const Plan& p : plan_launches(st, n_states, layer0, n_layers)) {
            StateTable t;
            fill_table(p, st, layer0 + p.l_off, &t);
            const UnitMap um = make_map(p, layer0, n_layers, n_new, t0, m);
            AppendArgs aa;
            aa.g = g;
            aa.m = um;
            aa.k = k;
            aa.v = v;
            AttnArgs at{};
            at.g = g;
            at.m = um;
            at.q = q;
            at.k = k;
            at.v = v;
            at.out = out;
            if (d.kind == VRT_ENC_LOOKAHEAD) {
                // append (no rotation), answer the queries whose last future
                // frame now exists, keep the rest waiting
                const int pw = (int)std::min<int64_t>(st[p.states[0]]->n_kv[layer0 + p.l_off], F);
                n_out_sb = pw == F ? m : std::max(0, pw + m - F);
                const int keep = pw == F ? F : std::min(pw + m, F);
                at.look_f = F;
                at.look_pend = pw;
                at.look_nout = n_out_sb;
                at.look_o0 = o_written;
                at.pend_off = (long long)d.n_layers * (long long)layer_bytes(d);
                at.pend_layer = (long long)pend_layer_bytes(d);
                at.partials = nullptr;
                at.n_splits = 1;
                at.split_len = kSplitLen;
                at.scale_log2 = scale_log2(g.Dio);
                at.qchunk = kRows / g.group;
                at.n_qchunks = (n_out_sb + at.qchunk - 1) / at.qchunk;
                // with one query chunk the attention launch appends the new
                // rows itself; otherwise (or with no query to answer) a
                // separate append runs first
                at.append = at.n_qchunks == 1 ? 1 : 0;
                at.look_keep = at.append ? keep : 0;   // and saves the waiting rows
                at.hg = n_out_sb > 0 ? pick_hg(g, (long long)um.n_states * um.nl,
                                               std::min(at.qchunk, n_out_sb) * g.group, at.n_qchunks, 1)
                                     : 1;
                if ((!at.append && note(launch_rope_append(aa, t, stream)) != hipSuccess) ||
                    (n_out_sb > 0 && note(launch_attn(at, false, t, stream)) != hipSuccess) ||
                    (!at.append && note(launch_pend_save(at, t, keep, stream)) != hipSuccess)) {
                    poison(st, n_states);
                    return VRT_ERR_DEVICE;
                }
                continue;
            }
            const bool mfma = use_mfma(d, m);
            attn_shape(g, mfma, (long long)um.n_states * um.nl, m, &at);
            if ((!at.append && note(launch_rope_append(aa, t, stream)) != hipSuccess) ||
                note(launch_attn(at, mfma, t, stream)) != hipSuccess) {
                poison(st, n_states);
                return VRT_ERR_DEVICE;
            }
        }
        for (int i = 0; i < n_states; ++i)
            for (int l = layer0; l < layer0 + n_layers; ++l) st[i]->n_kv[l] += m;
        t0 += m;
        o_written += n_out_sb;
    }
    return VRT_OK;
}

vrt_status vrt_ring_compact(vrt_stream_state* const* st, int n_states, int layer0, int n_layers,
                            hipStream_t stream) {
    if (!st || n_states < 1 || !st[0] || !is_encoder(st[0]->d)) return VRT_ERR_INVALID;
    const vrt_status s = check_batch(st, n_states, layer0, n_layers, st[0]->d.kind);
    if (s != VRT_OK) return s;
    if (st[0]->d.kind == VRT_ENC_MODRING) return VRT_OK;   // a modulo ring is never compacted
    std::vector<std::pair<int, int>> comp;
    for (int i = 0; i < n_states; ++i)
        for (int l = layer0; l < layer0 + n_layers; ++l)
            if (st[i]->n_kv[l] > st[i]->d.window) comp.emplace_back(i, l);
    clear_sticky_error();
    if (run_compactions(st, comp, stream) != hipSuccess) {
        poison(st, n_states);
        return VRT_ERR_DEVICE;
    }
    return VRT_OK;
}

size_t vrt_dec_workspace_bytes(const vrt_cache_desc* desc, int n_states, int n_layers,
                               int n_tok) {
    if (check_desc(desc) != VRT_OK || n_states < 1 || n_layers < 1 || n_tok < 1) return 0;
    if (n_tok > 1) return 0;  // prefill needs no workspace
    const size_t n_splits = (size_t)(desc->window + kSplitLen - 2) / kSplitLen + 1;
    const size_t group = desc->n_heads_q / desc->n_heads_kv;
    return (size_t)n_states * n_layers * desc->n_heads_kv * n_splits *
           (size_t)dec_record_floats((int)group, desc->head_dim) * sizeof(float);
}

vrt_status vrt_dec_attn_step(vrt_stream_state* const* st, int n_states, int layer0,
                             int n_layers, const void* q, const void* k, const void* v,
                             int n_tok, void* out, void* workspace, size_t ws_bytes,
                             hipStream_t stream) {
    vrt_status s = check_batch(st, n_states, layer0, n_layers, VRT_DEC_MODRING);
    if (s != VRT_OK) return s;
    if (!q || !k || !v || !out || n_tok < 1) return VRT_ERR_INVALID;
    const vrt_cache_desc& d = st[0]->d;
    if (n_tok == 1) {
        if (!workspace || ((uintptr_t)workspace & 15)) return VRT_ERR_INVALID;
        if (ws_bytes < vrt_dec_workspace_bytes(&d, n_states, n_layers, 1)) return VRT_ERR_CAPACITY;
    }
    // positions in range, and no sub-batch of a prefill overwrites a slot that
    // one of its own queries still reads
    const std::vector<int> subs = split_feed(n_tok, d.max_batch);
    for (int i = 0; i < n_states; ++i)
        for (int l = layer0; l < layer0 + n_layers; ++l) {
            const int64_t start = st[i]->abs_base[l];
            int64_t next = start + st[i]->n_kv[l];
            if (next > kPosLimit - n_tok || (int64_t)st[i]->n_kv[l] + n_tok > INT_MAX)
                return VRT_ERR_INVALID;
            for (int m : subs) {
                const int64_t evicted_max = next + m - 1 - d.ring_slots;
                const int64_t needed_min = std::max(start, next - d.window + 1);
                if (m > 1 && evicted_max >= needed_min) return VRT_ERR_INVALID;
                next += m;
            }
        }

    const Geom g = make_geom(d);
    clear_sticky_error();
    int t0 = 0;
    for (int m : subs) {
        for (const Plan& p : plan_launches(st, n_states, layer0, n_layers)) {
            StateTable t;
            fill_table(p, st, layer0 + p.l_off, &t);
            const UnitMap um = make_map(p, layer0, n_layers, n_tok, t0, m);
            AppendArgs aa;
            aa.g = g;
            aa.m = um;
            aa.k = k;
            aa.v = v;
            AttnArgs at{};
            at.g = g;
            at.m = um;
            at.q = q;
            at.k = k;
            at.v = v;
            at.out = out;
            at.partials = m == 1 ? (float*)workspace : nullptr;
            dec_shape(g, (long long)um.n_states * um.nl, m, &at);
            hipError_t err = hipSuccess;
            if (!at.append) err = note(launch_rope_append(aa, t, stream));
            if (err == hipSuccess) err = note(record_start(stream));
            if (err == hipSuccess) err = note(launch_attn_valu(at, t, stream));
            if (err == hipSuccess && m == 1) err = note(launch_dec_combine(at, t, stream));
            if (err == hipSuccess) err = note(record_stop(stream));
            if (err != hipSuccess) {
                poison(st, n_states);
                return VRT_ERR_DEVICE;
            }
        }
        for (int i = 0; i < n_states; ++i)
            for (int l = layer0; l < layer0 + n_layers; ++l) st[i]->n_kv[l] += m;
        t0 += m;
    }
    return VRT_OK;
}

vrt_status vrt_dec_attn_step_static(vrt_stream_state* const* st, int n_states, int layer0,
                                    int n_layers, const void* q, const void* k, const void* v,
                                    int n_tok, void* out, hipStream_t stream) {
    const vrt_status s = check_batch(st, n_states, layer0, n_layers, VRT_DEC_MODRING);
    if (s != VRT_OK) return s;
    if (!q || !k || !v || !out || n_tok < 1) return VRT_ERR_INVALID;
    if (n_tok > 1)   // a prefill has no partials
        return vrt_dec_attn_step(st, n_states, layer0, n_layers, q, k, v, n_tok, out, nullptr, 0, stream);
    const size_t need = vrt_dec_workspace_bytes(&st[0]->d, n_states, n_layers, 1);
    if (need > kStaticScratchBytes) return VRT_ERR_CAPACITY;
    void* ws = nullptr;
    if (g_dry) {
        ws = (void*)(uintptr_t)256;   // dry run: nothing is launched, nothing is read
    } else {
        clear_sticky_error();
        if (note(static_scratch(&ws)) != hipSuccess) return VRT_ERR_DEVICE;
    }
    return vrt_dec_attn_step(st, n_states, layer0, n_layers, q, k, v, 1, out, ws, need, stream);
}

vrt_status vrt_set_attn_events(hipEvent_t start, hipEvent_t stop) {
    if ((start == nullptr) != (stop == nullptr)) return VRT_ERR_INVALID;
    if (start) {
        for (hipEvent_t e : {start, stop}) {
            const hipError_t q = hipEventQuery(e);
            if (q != hipSuccess && q != hipErrorNotReady) {
                note(q);
                clear_sticky_error();
                return VRT_ERR_INVALID;
            }
        }
    }
    g_ev_start = start;
    g_ev_stop = stop;
    return VRT_OK;
}


// ---- encoder attention block around the path

static bool aligned16(const void* p) { return ((uintptr_t)p & 15) == 0; }

vrt_status vrt_rmsnorm(const void* x, int rows, int dim, const void* w, float eps, void* y,
                       hipStream_t stream) {
    if (!x || !w || !y || rows < 1 || dim < 8 || dim % 8 != 0 || dim > 2048) return VRT_ERR_INVALID;
    if (!(eps >= 0.f) || !std::isfinite(eps)) return VRT_ERR_INVALID;
    if (!aligned16(x) || !aligned16(w) || !aligned16(y)) return VRT_ERR_INVALID;
    NormArgs a{x, dim, w, y, dim, rows, dim, eps};
    clear_sticky_error();
    return note(launch_rmsnorm(a, stream)) == hipSuccess ? VRT_OK : VRT_ERR_DEVICE;
}

vrt_status vrt_linear(const void* A, int M, int K, const void* W, int N, const void* bias,
                      const void* residual, void* out, hipStream_t stream) {
    if (!A || !W || !out || M < 1 || K < 1 || N < 1) return VRT_ERR_INVALID;
    if (K % 64 != 0 || N % 128 != 0) return VRT_ERR_UNSUPPORTED;
    if (!aligned16(A) || !aligned16(W) || ((uintptr_t)out & 1) || ((uintptr_t)bias & 1) ||
        ((uintptr_t)residual & 1))
        return VRT_ERR_INVALID;
    GemmArgs g{};
    g.A = A;
    g.lda = K;
    g.W = W;
    g.ldw = K;
    g.R = residual;
    g.ldr = N;
    g.M = M;
    g.N = N;
    g.K = K;
    gemm_plain(&g);
    g.seg_w = N;
    g.n_seg = 1;
    g.seg[0] = GemmSeg{out, bias, N};
    clear_sticky_error();
    return note(launch_gemm(g, stream)) == hipSuccess ? VRT_OK : VRT_ERR_DEVICE;
}

static size_t block_buf_bytes(int n_rows, int dim) {
    return ((size_t)n_rows * dim * 2 + 255) / 256 * 256;
}

size_t vrt_block_workspace_bytes(const vrt_cache_desc* desc, int n_rows) {
    if (check_desc(desc) != VRT_OK || n_rows < 1) return 0;
    return 5 * block_buf_bytes(n_rows, desc->n_heads_q * desc->head_dim);
}

vrt_status vrt_enc_block_feed(vrt_stream_state* const* st, int n_states, int layer, const void* x,
                              int n_new, const vrt_block_weights* w, void* out, void* workspace,
                              size_t ws_bytes, hipStream_t stream) {
    if (!st || n_states < 1 || !st[0] || !is_encoder(st[0]->d)) return VRT_ERR_INVALID;
    vrt_status s = check_batch(st, n_states, layer, 1, st[0]->d.kind);
    if (s != VRT_OK) return s;
    const vrt_cache_desc& d = st[0]->d;
    if (!x || !out || !w || !workspace || n_new < 1) return VRT_ERR_INVALID;
    if (!w->norm_w || !w->w_qkv || !w->w_o || w->reserved != 0) return VRT_ERR_INVALID;
    if (!(w->eps >= 0.f) || !std::isfinite(w->eps)) return VRT_ERR_INVALID;
    // (left, right) windows answer other frames' queries than the rows fed,
    // so the residual rows would not line up: the block takes the rings only
    if (d.kind == VRT_ENC_LOOKAHEAD) return VRT_ERR_UNSUPPORTED;
    if (d.dtype != VRT_BF16 || d.n_heads_q != d.n_heads_kv) return VRT_ERR_UNSUPPORTED;
    const int dim = d.n_heads_q * d.head_dim;
    if (dim % 128 != 0 || dim > 2048) return VRT_ERR_UNSUPPORTED;
    if (!aligned16(x) || !aligned16(out) || !aligned16(workspace) || !aligned16(w->norm_w) ||
        !aligned16(w->w_qkv) || !aligned16(w->w_o) || ((uintptr_t)w->b_q & 1) ||
        ((uintptr_t)w->b_v & 1) || ((uintptr_t)w->b_o & 1))
        return VRT_ERR_INVALID;
    if ((long long)n_states * n_new > INT_MAX / 4) return VRT_ERR_INVALID;
    const int M = n_states * n_new;
    if (ws_bytes < vrt_block_workspace_bytes(&d, M)) return VRT_ERR_CAPACITY;
    // the checks vrt_enc_attn_feed makes, before anything is enqueued
    for (int i = 0; i < n_states; ++i)
        if (st[i]->abs_base[layer] + st[i]->n_kv[layer] > kPosLimit - n_new) return VRT_ERR_INVALID;

    const size_t bb = block_buf_bytes(M, dim);
    char* ws = (char*)workspace;
    char *y = ws, *q = ws + bb, *k = ws + 2 * bb, *v = ws + 3 * bb, *a = ws + 4 * bb;
    clear_sticky_error();
    NormArgs na{x, dim, w->norm_w, y, dim, M, dim, w->eps};
    if (note(launch_rmsnorm(na, stream)) != hipSuccess) {
        poison(st, n_states);
        return VRT_ERR_DEVICE;
    }
    GemmArgs g{};
    g.A = y;
    g.lda = dim;
    g.W = w->w_qkv;
    g.ldw = dim;
    g.M = M;
    g.N = 3 * dim;
    g.K = dim;
    gemm_plain(&g);
    g.seg_w = dim;
    g.n_seg = 3;
    g.seg[0] = GemmSeg{q, w->b_q, dim};
    g.seg[1] = GemmSeg{k, nullptr, dim};
    g.seg[2] = GemmSeg{v, w->b_v, dim};
    if (note(launch_gemm(g, stream)) != hipSuccess) {
        poison(st, n_states);
        return VRT_ERR_DEVICE;
    }
    // every check of the feed was made above, so it can only fail on a
    // launch, and then it has poisoned the states itself
    s = vrt_enc_attn_feed(st, n_states, layer, 1, q, k, v, n_new, a, stream);
    if (s != VRT_OK) return s;
    GemmArgs o{};
    o.A = a;
    o.lda = dim;
    o.W = w->w_o;
    o.ldw = dim;
    o.R = x;
    o.ldr = dim;
    o.M = M;
    o.N = dim;
    o.K = dim;
    gemm_plain(&o);
    o.seg_w = dim;
    o.n_seg = 1;
    o.seg[0] = GemmSeg{out, w->b_o, dim};
    if (note(launch_gemm(o, stream)) != hipSuccess) {
        // the rings already hold this feed's rows: a retry would append them twice
        poison(st, n_states);
        return VRT_ERR_DEVICE;
    }
    return VRT_OK;
}


// ---- causal conv stem ahead of the encoder

}  // extern "C"

struct vrt_conv_stem {
    int n_mel, d_model;
    char* dev;          // mel cache [2][n_mel], then conv0 pending rows [2][d_model] (bf16)
    size_t pend_off;
    int pending;        // conv0 frames carried for conv1 (1 or 2)
    bool fresh;         // caches hold nothing yet (they read as zeros)
    int64_t frames_in;  // mel frames fed since the last reset
};

namespace {

constexpr int kConvPad0 = 2;   // (kernel 3 - 1) + 1 - stride 1
constexpr int kConvPad1 = 1;   // (kernel 3 - 1) + 1 - stride 2

bool conv_dims_ok(int n_mel, int d_model) {
    return n_mel >= 64 && n_mel % 64 == 0 && n_mel <= 4096 && d_model >= 128 && d_model % 128 == 0 &&
           d_model <= 8192;
}
size_t pad256(size_t b) { return (b + 255) / 256 * 256; }
// conv1 outputs of a feed whose staged conv0 rows number L (pending + new)
int conv1_outputs(int L) { return L >= 3 ? (L - 1) / 2 : 0; }

}  // namespace

extern "C" {

size_t vrt_conv_stem_device_bytes(int n_mel, int d_model) {
    if (!conv_dims_ok(n_mel, d_model)) return 0;
    return pad256((size_t)kConvPad0 * n_mel * 2) + pad256((size_t)2 * d_model * 2);
}

vrt_status vrt_conv_stem_create(int n_mel, int d_model, void* dev_mem, size_t bytes,
                                vrt_conv_stem** out) {
    if (!out || !dev_mem || ((uintptr_t)dev_mem & 255) != 0) return VRT_ERR_INVALID;
    if (!conv_dims_ok(n_mel, d_model)) return VRT_ERR_UNSUPPORTED;
    if (bytes < vrt_conv_stem_device_bytes(n_mel, d_model)) return VRT_ERR_CAPACITY;
    vrt_conv_stem* c = new (std::nothrow) vrt_conv_stem;
    if (!c) return VRT_ERR_CAPACITY;
    c->n_mel = n_mel;
    c->d_model = d_model;
    c->dev = (char*)dev_mem;
    c->pend_off = pad256((size_t)kConvPad0 * n_mel * 2);
    c->pending = kConvPad1;
    c->fresh = true;
    c->frames_in = 0;
    *out = c;
    return VRT_OK;
}

vrt_status vrt_conv_stem_reset(vrt_conv_stem* c) {
    if (!c) return VRT_ERR_INVALID;
    c->pending = kConvPad1;
    c->fresh = true;
    c->frames_in = 0;
    return VRT_OK;
}

void vrt_conv_stem_destroy(vrt_conv_stem* c) { delete c; }

vrt_status vrt_conv_stem_query(const vrt_conv_stem* c, int64_t* frames_in, int32_t* pending) {
    if (!c) return VRT_ERR_INVALID;
    if (frames_in) *frames_in = c->frames_in;
    if (pending) *pending = c->pending;
    return VRT_OK;
}

int vrt_conv_out_frames(const vrt_conv_stem* c, int n_frames) {
    if (!c || n_frames < 0) return -1;
    return conv1_outputs(c->pending + n_frames);
}

// conv1 runs as kConv1Split k parts (one per tap) and an ordered reduce
constexpr int kConv1Split = 3;

size_t vrt_conv_workspace_bytes(int n_mel, int d_model, int n_stems, int n_frames) {
    if (!conv_dims_ok(n_mel, d_model) || n_stems < 1 || n_frames < 1) return 0;
    return pad256((size_t)n_stems * (n_frames + kConvPad0) * n_mel * 2) +
           pad256((size_t)n_stems * (n_frames + 2) * d_model * 2) +
           (size_t)kConv1Split * n_stems * ((n_frames + 2) / 2) * d_model * 4;   // conv1's fp32 parts
}

vrt_status vrt_conv_stem_feed(vrt_conv_stem* const* stems, int n_stems, const void* mel,
                              int n_frames, const vrt_conv_weights* w, void* out, int32_t* n_out,
                              void* workspace, size_t ws_bytes, hipStream_t stream) {
    if (!stems || n_stems < 1 || n_stems > kMaxStems || !stems[0] || !mel || !w || !out || !n_out ||
        !workspace || n_frames < 1)
        return VRT_ERR_INVALID;
    if (!w->w0 || !w->w1) return VRT_ERR_INVALID;
    const int n_mel = stems[0]->n_mel, d = stems[0]->d_model, p = stems[0]->pending;
    std::vector<const vrt_conv_stem*> seen;
    for (int i = 0; i < n_stems; ++i) {
        const vrt_conv_stem* c = stems[i];
        if (!c || c->n_mel != n_mel || c->d_model != d || c->pending != p ||
            c->pend_off != stems[0]->pend_off)
            return VRT_ERR_INVALID;
        seen.push_back(c);
    }
    std::sort(seen.begin(), seen.end());
    if (std::adjacent_find(seen.begin(), seen.end()) != seen.end()) return VRT_ERR_INVALID;
    if ((long long)n_stems * (n_frames + kConvPad0) > INT_MAX / 2) return VRT_ERR_INVALID;
    if (!aligned16(mel) || !aligned16(out) || !aligned16(workspace) || !aligned16(w->w0) ||
        !aligned16(w->w1) || ((uintptr_t)w->b0 & 1) || ((uintptr_t)w->b1 & 1))
        return VRT_ERR_INVALID;
    if (ws_bytes < vrt_conv_workspace_bytes(n_mel, d, n_stems, n_frames)) return VRT_ERR_CAPACITY;

    const int L = p + n_frames, o = conv1_outputs(L), keep = L - 2 * o;   // keep: 1 or 2
    char* st0 = (char*)workspace;                       // [stem][n_frames + 2][n_mel]
    char* st1 = st0 + pad256((size_t)n_stems * (n_frames + kConvPad0) * n_mel * 2);  // [stem][n_frames + 2][d]
    RowCopyTable t;
    for (int i = 0; i < n_stems; ++i) {
        t.cache[i] = (unsigned long long)(uintptr_t)stems[i]->dev;
        t.fresh[i] = stems[i]->fresh ? 1 : 0;
    }
    const long long pend_off = (long long)stems[0]->pend_off;
    clear_sticky_error();
    // staging, in one launch: [mel cache | new mel] and [pending conv0 rows | conv0 output]
    {
        RowCopyArgs a{};
        a.n_groups = n_stems;
        a.n_seg = 3;
        a.seg[0] = RowCopySeg{kConvPad0, n_mel * 2, 0, st0, n_frames + kConvPad0, 0, 0, nullptr, 0, 1};
        a.seg[1] = RowCopySeg{p, d * 2, 0, st1, L, 0, pend_off, nullptr, 0, 1};
        a.seg[2] = RowCopySeg{n_frames, n_mel * 2, 0, st0, n_frames + kConvPad0, kConvPad0, 0,
                              (const char*)mel, n_frames, 0};
        if (note(launch_row_copy(a, t, stream)) != hipSuccess) return VRT_ERR_DEVICE;
    }
    GemmArgs g0{};
    g0.A = st0;
    g0.lda = n_mel;
    g0.W = w->w0;
    g0.ldw = 3 * n_mel;
    g0.M = n_stems * n_frames;
    g0.N = d;
    g0.K = 3 * n_mel;
    gemm_plain(&g0);
    g0.a_grp = n_frames;
    g0.a_gstride = n_frames + kConvPad0;
    g0.a_stride = 1;
    g0.a_cols = n_mel;
    g0.o_grp = n_frames;
    g0.o_gstride = L;
    g0.o_off = p;
    g0.act = 1;
    g0.seg_w = d;
    g0.n_seg = 1;
    g0.seg[0] = GemmSeg{st1, w->b0, d};
    if (note(launch_gemm(g0, stream)) != hipSuccess) return VRT_ERR_DEVICE;
    // new caches: the last two staged mel rows; the conv0 rows from 2 o on.  They
    // read only staging rows that conv0 has written, so when conv1 runs they ride
    // on its reduce launch, else they are one launch of their own.
    RowCopyArgs cout{};
    cout.n_groups = n_stems;
    cout.n_seg = 2;
    cout.seg[0] = RowCopySeg{kConvPad0, n_mel * 2, 1, st0, n_frames + kConvPad0, n_frames, 0, nullptr, 0, 0};
    cout.seg[1] = RowCopySeg{keep, d * 2, 1, st1, L, 2LL * o, pend_off, nullptr, 0, 0};
    if (o > 0) {
        GemmArgs g1{};
        g1.A = st1;
        g1.lda = d;
        g1.W = w->w1;
        g1.ldw = 3 * d;
        g1.M = n_stems * o;
        g1.N = d;
        g1.K = 3 * d;
        gemm_plain(&g1);
        g1.a_grp = o;
        g1.a_gstride = L;
        g1.a_stride = 2;
        g1.a_cols = d;
        g1.act = 1;
        g1.seg_w = d;
        g1.n_seg = 1;
        g1.seg[0] = GemmSeg{out, w->b1, d};
        // one k part per tap: three times the workgroups of a 3 d-deep product
        g1.ksplit = kConv1Split;
        g1.part = (float*)(st1 + pad256((size_t)n_stems * (n_frames + 2) * d * 2));
        if (note(launch_gemm(g1, stream, &cout, &t)) != hipSuccess) return VRT_ERR_DEVICE;
    }
    if (o == 0 && note(launch_row_copy(cout, t, stream)) != hipSuccess) return VRT_ERR_DEVICE;
    for (int i = 0; i < n_stems; ++i) {
        stems[i]->pending = keep;
        stems[i]->fresh = false;
        stems[i]->frames_in += n_frames;
    }
    *n_out = o;
    return VRT_OK;
}

vrt_status vrt_read_probe(const void* buf, size_t bytes, void* sink, hipStream_t stream) {
    if (!buf || !sink || bytes < 16 || !aligned16(buf) || ((uintptr_t)sink & 3)) return VRT_ERR_INVALID;
    clear_sticky_error();
    return note(launch_read_probe(buf, bytes, (unsigned*)sink, stream)) == hipSuccess ? VRT_OK : VRT_ERR_DEVICE;
}

vrt_status vrt_tile_stream_probe(const void* buf, size_t bytes, int n_wg, int heads, int tiles, int n_regions,
                                 size_t region_stride, size_t kv_off, int passes, int first_row, int last_row,
                                 int flags, void* sink, hipStream_t stream) {
    if (!buf || !sink || !aligned16(buf) || ((uintptr_t)sink & 3) || n_wg < 1 || heads < 1 || tiles < 1 ||
        n_regions < 1 || passes < 1 || region_stride % 16 || kv_off % 16 || (flags & ~1))
        return VRT_ERR_INVALID;
    if (first_row < 0 || first_row >= kTile || last_row < 0 || last_row >= kTile ||
        (tiles == 1 && first_row > last_row))
        return VRT_ERR_INVALID;
    // the last byte read: region n_regions - 1, its V half, the end of tile `tiles` - 1
    const long double last = (long double)(n_regions - 1) * region_stride + kv_off + (long double)tiles * 8192;
    if ((long long)heads * tiles > (1LL << 30) || last > (long double)bytes || last > 9.0e18L)
        return VRT_ERR_INVALID;
    clear_sticky_error();
    return note(launch_tile_probe((const char*)buf, (long long)region_stride, (long long)kv_off, n_regions, n_wg,
                                  heads, tiles, passes, first_row, last_row, (flags & 1) != 0, (unsigned*)sink,
                                  stream)) == hipSuccess
               ? VRT_OK
               : VRT_ERR_DEVICE;
}

}  // extern "C"
