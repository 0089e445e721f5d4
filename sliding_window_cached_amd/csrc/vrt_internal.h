// Internal launch interface between the C-ABI host code (vrt_host.cpp) and the
// gfx950 kernels (vrt_kernels.hip).  Not part of the public ABI.
#pragma once

#include <stdint.h>
#include <hip/hip_runtime.h>

namespace vrt {

// Every kernel launch of the library goes through this gate first.  It
// returns 1 to go ahead; 0 to skip the launch with *e as its result: the
// launch the testing hook (vrt_test_launch_hook) marks to fail gets a launch
// error, and in the hook's dry-run mode every other launch is skipped and
// reported successful (host logic without a GPU).
int launch_gate(hipError_t* e);
// Compute units and LDS bytes per compute unit of the current device, read
// once per device (256 and 160 KB, MI355X's, when no device answers).
int device_cus();
int device_lds();
#define VRT_LAUNCH(KERNEL, ...)                                      \
    do {                                                             \
        hipError_t gate_e_;                                          \
        if (::vrt::launch_gate(&gate_e_)) {                          \
            hipLaunchKernelGGL(KERNEL, __VA_ARGS__);                 \
            gate_e_ = hipGetLastError();                             \
        }                                                            \
        if (gate_e_ != hipSuccess) return gate_e_;                   \
    } while (0)

// States per launch.  The per-state table travels in the kernel arguments
// (no device-side table to upload, nothing for the library to allocate);
// 256 entries (one launch for 256 streams) make a 6 KB argument block;
// kernel arguments of this size are passed intact on gfx950.
constexpr int kMaxStates = 256;
// Compaction entries per launch (one entry = one (state, layer) ring).
constexpr int kMaxCompact = 256;
// Keys per tile; tiles start at multiples of 64 in absolute position.
constexpr int kTile = 64;
// Query rows (q head x position) of one kv head in one attention workgroup.
constexpr int kRows = 16;
// LDS bytes for the rotated query rows of a workgroup's kv-head group: 6 KB,
// or more when kRows rows of one head are wider than that (fp32 rows of
// head_dim 128, 16 x 512 bytes).  The attention kernel also stages its output
// rows there.
constexpr int kQsBytes = 6144;
constexpr int attn_qs_bytes(int row_bytes) { return kRows * row_bytes > kQsBytes ? kRows * row_bytes : kQsBytes; }
// Sub-batches of at least this many frames take the matrix-core path (bf16,
// head_dim 64, one query head per kv head); smaller ones the VALU path.
constexpr int kMfmaMinFrames = 32;
// Queries per workgroup of the matrix-core path.
constexpr int kQTileMfma = 128;
// Keys per split of the decode step; splits start at multiples of this in
// absolute position and are merged in ascending order.  At window 8192 that is
// 5 splits: the 32-stream x 26-layer step writes about half the partials
// 1024-key splits did and ran 1.3 % faster, with 8 320 workgroups still in
// the launch.
constexpr int kSplitLen = 2048;
// Split-K partials: one record per (call unit, kv head, split).  Its first
// 128 bytes hold (m, l) of each of the split's `group` query rows (2 floats per
// row, zeros after them; group <= kRows = 16 fills at most the line), then the
// rows' D accumulators follow.  Records and accumulator rows are whole 128-byte
// lines, so the decode step writes whole lines.
constexpr int kMlFloats = 32;
constexpr long long dec_record_floats(int group, int D) { return kMlFloats + (long long)group * D; }
// Sentinel for "no key seen yet" in the running maximum (finite on purpose:
// exp2(SENT - SENT) = 1 keeps fully masked tiles exact no-ops).
constexpr float kSent = -1.0e30f;

// LDS tile stages of the vector-path attention kernel per (storage dtype,
// head_dim, split mode); the host sizes its workgroups-per-CU target by it.
// Two everywhere: three or four stages (fewer workgroups per CU, more bytes
// in flight per CU) measured the same on the serving and decoder workloads,
// which already stream near the part's read ceiling.
constexpr int attn_stages(int dtype, int D, bool split) {
    return 2 + 0 * (dtype + D + (split ? 1 : 0));
}

// Geometry of one cache kind, shared by every state of a launch.
struct Geom {
    int dtype;          // 0 f32, 1 bf16
    int D;              // elements per ring row and per head in the kernels (64 or 128)
    int Dio;            // head_dim of the inputs and outputs (= D, or below 64 for lookahead
                        // windows: ring rows zero-padded from Dio to D elements)
    int hq, hkv, group; // query heads, kv heads, hq / hkv
    int slots;          // ring slots per (layer, kv head)
    int window;         // W
    int mod;            // 1: slot = pos % slots; 0: slot = pos - abs_base
    int rope;           // 1: q and k are rotated at their positions; 0: no rotation
    long long layer_bytes;  // bytes per layer inside a state (K ring + V ring)
    long long slice_bytes;  // bytes per kv-head slice = slots * D * elem
    long long v_off;        // byte offset of the V ring inside a layer
    double omega[64];       // RoPE frequencies theta^(-2i/D), i < D/2, fp64
};

// Per-state entries of one launch.  p0 = absolute position of the first new
// frame of this sub-batch; n_kv = rows (tokens, for the decoder) the ring held
// before this sub-batch was appended, so abs_base = p0 - n_kv.
struct StateTable {
    unsigned long long ring[kMaxStates];
    long long p0[kMaxStates];
    int n_kv[kMaxStates];
    int call_idx[kMaxStates];   // index of the state within the call's arrays
};

// How a launch's units map to the call's input/output arrays.
//   unit (si, li) of the launch  ->  call unit call_idx[si] * nl_call + l_off + li
//   state layer index            ->  layer0 + l_off + li
//   element offset of frame f    ->  (call_unit * n_total + t0 + f) * heads * D
struct UnitMap {
    int n_states;   // states in this launch (<= kMaxStates)
    int nl;         // layers in this launch
    int l_off;      // first layer of the launch, relative to the call's layer0
    int nl_call;    // layers in the call
    int layer0;     // state layer index of the call's first layer
    int n_total;    // frames per unit in the caller's arrays (n_new / n_tok)
    int t0;         // first frame of this sub-batch inside those arrays
    int n;          // frames in this sub-batch
};

struct AppendArgs {
    Geom g;
    UnitMap m;
    const void* k;
    const void* v;
};

struct AttnArgs {
    Geom g;
    UnitMap m;
    const void* q;
    const void* k;      // new keys / values (fused append only)
    const void* v;
    void* out;          // [call unit][frame][hq][D]  (non-split)
    float* partials;    // split mode: [call unit][hkv][split] records, dec_record_floats each
    int qchunk;         // positions per workgroup
    int n_qchunks;
    int n_splits;       // 1 = no split
    int split_len;
    float scale_log2;   // log2(e) / sqrt(D)
    int append;         // 1: the attention launch also appends the new K/V rows
    int hg;             // kv heads per workgroup (divides hkv)
    // (left, right) windows: query i of this launch (0 <= i < look_nout) sits
    // at p0 - look_pend + i, sees keys up to look_f frames past itself (up to
    // the newest frame written), and takes its q row from the state's waiting
    // rows when i < look_pend, else from new frame i - look_pend; its output
    // goes to row look_o0 + i of the call's output
    int look_f, look_pend, look_nout, look_o0;
    // > 0: the launch (one query chunk) also leaves the last look_keep rows of
    // [waiting rows | new q rows] as the next call's waiting rows
    int look_keep;
    long long pend_off;       // byte offset, in a state, of layer 0's waiting q rows
    long long pend_layer;     // bytes of one layer's waiting rows (look_f rows)
};

// Waiting q rows after a sub-batch of a lookahead cache: the last `keep`
// rows of [the `pend` waiting rows | the sub-batch's q rows] (a forward copy
// in place: every row moves to a lower or equal index)
hipError_t launch_pend_save(const AttnArgs& a, const StateTable& t, int keep, hipStream_t s);

struct CompactTable {
    unsigned long long layer_ring[kMaxCompact];  // base of the (state, layer) K ring
    int shift[kMaxCompact];                      // rows dropped from the front
};

struct CompactArgs {
    Geom g;
    int n_entries;
    int kept;           // rows kept (= window)
};

// ---- encoder attention block around the path (vrt_block.hip)
struct NormArgs {
    const void* x;      // [rows][ldx] bf16
    long long ldx;
    const void* w;      // [dim] bf16 gain
    void* y;            // [rows][ldy] bf16
    long long ldy;
    int rows, dim;
    float eps;
};

constexpr int kMaxGemmSeg = 4;
struct GemmSeg {
    void* out;          // [M][ld] bf16: columns [s * seg_w, (s + 1) * seg_w) of the product
    const void* bias;   // [seg_w] bf16 or null
    long long ld;
};
struct GemmArgs {
    const void* A;      // bf16 rows of lda elements (see the row addressing below)
    long long lda;
    const void* W;      // [N][ldw] bf16, one row per output column
    long long ldw;
    const void* R;      // [M][ldr] bf16 residual (indexed by product row), or null
    long long ldr;
    int M, N, K;
    int seg_w, n_seg;
    GemmSeg seg[kMaxGemmSeg];
    // A row addressing (an implicit im2col for convolutions): product row m
    // of group g = m / a_grp, i = m % a_grp, reads for k in
    // [t a_cols, (t + 1) a_cols) the source row g a_gstride + i a_stride + t.
    // A plain product: a_grp = M, a_gstride = 0, a_stride = 1, a_cols = K.
    int a_grp, a_stride, a_cols;
    long long a_gstride;
    // output rows: product row m is stored at row (m / o_grp) o_gstride +
    // m % o_grp + o_off of its segment.  Plain: o_grp = M, o_gstride = 0, o_off = 0.
    int o_grp, o_off;
    long long o_gstride;
    int act;            // 0: none; 1: GELU (exact, erf form) after bias and residual
    // ksplit > 1: the k range is cut into ksplit equal parts (each a multiple
    // of 64 and of a_cols); workgroup part s writes its fp32 sums to
    // part[s][m][n], and an ordered reduce then forms the output as above
    // from ((part 0 + part 1) + part 2) + ...
    int ksplit;
    float* part;
};
inline void gemm_plain(GemmArgs* g) {
    g->a_grp = g->M;
    g->a_stride = 1;
    g->a_cols = g->K;
    g->a_gstride = 0;
    g->o_grp = g->M;
    g->o_off = 0;
    g->o_gstride = 0;
    g->act = 0;
    g->ksplit = 1;
    g->part = nullptr;
}

// ---- causal conv stem (vrt_block.hip): row copies between each stem's
// caches (device memory of its own, given by a table), the new input rows and
// the staging rows; up to kMaxCopySeg segments in one launch
constexpr int kMaxStems = 256;
constexpr int kMaxCopySeg = 3;
struct RowCopySeg {
    int rows;                   // rows per group (0: the segment is empty)
    int row_bytes;              // multiple of 16
    int to_cache;               // 0: cache (or src) -> staging; 1: staging -> cache
    char* stage;                // group g row r at stage + (g gstride + off + r) row_bytes
    long long gstride, off;
    long long cache_off;        // byte offset of the segment's rows in each stem's memory
    const char* src;            // to_cache = 0 and non-null: group g row r read from
    long long src_gstride;      //   src + (g src_gstride + r) row_bytes instead of a cache
    int zero_fresh;             // cache -> staging: zeros for the stems marked fresh
};
struct RowCopyArgs {
    int n_groups, n_seg;
    RowCopySeg seg[kMaxCopySeg];
};
struct RowCopyTable {
    unsigned long long cache[kMaxStems];   // base of each stem's memory
    int fresh[kMaxStems];
};
hipError_t launch_row_copy(const RowCopyArgs& a, const RowCopyTable& t, hipStream_t s);
// A product; with ksplit > 1 the ordered reduce follows, and `tail` (with its
// table), an independent row copy, rides on the reduce launch as extra
// workgroups; with ksplit = 1 it is launched after the product.
hipError_t launch_gemm(const GemmArgs& a, hipStream_t s, const RowCopyArgs* tail = nullptr,
                       const RowCopyTable* tail_t = nullptr);
hipError_t launch_read_probe(const void* buf, size_t bytes, unsigned* sink, hipStream_t s);
hipError_t launch_tile_probe(const char* buf, long long region_stride, long long kv_off, int n_regions, int n_wg,
                             int heads, int tiles, int passes, int row_lo, int row_hi, bool nt, unsigned* sink,
                             hipStream_t s);

hipError_t launch_rmsnorm(const NormArgs& a, hipStream_t s);


// Bytes of the library's static device scratch array (one per device, held
// until the process ends), and its device address on the current device:
// looked up once per device with hipGetSymbolAddress, then reused.
constexpr size_t kStaticScratchBytes = (size_t)128 << 20;
hipError_t static_scratch(void** ptr);

hipError_t launch_rope_append(const AppendArgs& a, const StateTable& t, hipStream_t s);
hipError_t launch_attn_valu(const AttnArgs& a, const StateTable& t, hipStream_t s);
hipError_t launch_attn_mfma(const AttnArgs& a, const StateTable& t, hipStream_t s);
hipError_t launch_dec_combine(const AttnArgs& a, const StateTable& t, hipStream_t s);
hipError_t launch_compact(const CompactArgs& a, const CompactTable& t, hipStream_t s);

}  // namespace vrt
