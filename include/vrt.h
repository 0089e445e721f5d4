/*
 * vrt.h - streamed windowed-causal attention for MI355X (gfx950), C ABI.
 *
 * What the library computes
 * -------------------------
 * The hot path of a streaming audio encoder (Voxtral Realtime family doc,
 * "Architecture (summary)" and the Capability Validation table, Streaming
 * row): each feed of new encoder frames is rotated with NEOX RoPE
 * (theta 1e6, head_dim 64) at absolute positions, its K/V are appended to a
 * per-layer 1536-slot ring, the ring is compacted to its last 750 frames when
 * it would overflow, and every new query attends only to keys whose absolute
 * position p' satisfies p - 750 < p' <= p (streaming-plan page, "SHIPPED"
 * section, "Mechanism" and "Unbounded length" paragraphs).  The decoder's
 * one-token step (GQA 32 query / 8 kv heads, head_dim 128, window 8192,
 * modulo ring) runs on the same kernels (family doc, Decoder bullet;
 * Streaming row item 5).
 *
 * State is injected (bunsen book, "Stateless modules and streaming
 * contexts", "The principle: state is injected" and "The pattern"): the
 * caller owns every byte of device memory, creates one state per stream (one
 * state holds all layers of that stream, like a multi-layer KV cache), and
 * passes the states back on every call.  One call may carry many states
 * (streams are written one at a time and read together: same chapter, "The
 * write_read fold").
 *
 * Conventions for every entry point
 * ---------------------------------
 * - All device pointers are caller-owned; the library never allocates or
 *   frees device memory (the one exception is the static 128 MiB partials
 *   array of vrt_dec_attn_step_static, part of the loaded library on each
 *   device it runs on) and holds no state between calls apart from the
 *   optional per-thread timing events of vrt_set_attn_events, the testing
 *   hook of vrt_test_launch_hook, each device's compute-unit count and LDS
 *   size, read once, and that array's address per device.  All device work
 *   is enqueued on the caller's `stream` and is asynchronous.
 * - Arguments are checked before anything is enqueued.  On any error nothing
 *   is enqueued and no state changes (streaming-plan page, "Per-hook
 *   behavior": validate is pure).
 * - Host metadata (abs_base, n_kv per layer) advances when work is enqueued;
 *   it is a deterministic function of the calls, so no device-to-host sync is
 *   ever needed.
 * - If a kernel launch reports an error, VRT_ERR_DEVICE is returned and every
 *   state in the call is marked poisoned; poisoned states refuse every call
 *   (VRT_ERR_POISONED) until vrt_stream_state_reset.
 * - Absolute positions are int64 and must stay in [0, 2^31): a call whose
 *   frames would reach 2^31 fails with VRT_ERR_INVALID.
 * - Tensors are contiguous, row-major, in the state's dtype (float32 or
 *   bfloat16 bit patterns), 256-byte aligned device pointers.
 */
#ifndef VRT_H
#define VRT_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    VRT_OK = 0,
    VRT_ERR_INVALID = 1,      /* bad argument: null pointer, size, range, mixed descs */
    VRT_ERR_UNSUPPORTED = 2,  /* a configuration the library does not build */
    VRT_ERR_CAPACITY = 3,     /* memory or size too small for the request */
    VRT_ERR_DEVICE = 4,       /* a HIP launch failed; involved states are poisoned */
    VRT_ERR_POISONED = 5      /* state was poisoned by an earlier device error */
} vrt_status;

typedef enum { VRT_F32 = 0, VRT_BF16 = 1 } vrt_dtype;

typedef enum {
    VRT_ENC_RING = 0,     /* encoder: contiguous ring + compaction */
    VRT_DEC_MODRING = 1,  /* decoder: slot = position % ring_slots */
    VRT_ENC_MODRING = 2,  /* encoder: slot = position % ring_slots, no compaction */
    VRT_ENC_LOOKAHEAD = 3 /* encoder with (left, right) windows and no RoPE, modulo ring */
} vrt_cache_kind;

/* Everything about a cache is fixed when its states are created
 * (bunsen book, "Known gaps": invalid configurations fail at construction).
 * Encoder on the pages: kind ENC_RING, 20 heads (q = kv), head_dim 64,
 * window 750, ring_slots 1536, max_batch 512, rope_theta 1e6, 32 layers.
 * Decoder: kind DEC_MODRING, 32 q / 8 kv heads, head_dim 128,
 * window = ring_slots = 8192, rope_theta 1e6, 26 layers.
 * ENC_MODRING is the encoder cache stored the decoder's way (family doc,
 * Streaming row item 5: slot = position % ring_slots, positions stay
 * absolute): the same feeds, masks and arithmetic as ENC_RING without the
 * compaction copies, so its outputs are bit-identical to ENC_RING's (the
 * pages validate their decoder ring the same way, by an A/B against a buffer
 * that never wraps).  It needs ring_slots >= window - 1 + max_batch (a
 * sub-batch never overwrites a row one of its own queries reads), a multiple
 * of 64 (a 64-key tile never wraps); 1280 for the encoder above.
 * ENC_LOOKAHEAD is the moonshine streaming encoder's attention (moonshine
 * forward map, "Per-layer sliding-window mask" and "Encoder attention": no
 * RoPE, per-layer (left, right) windows): a query at t sees the keys u with
 * t - u in [0, window) or u - t in (0, lookahead), so lookahead - 1 future
 * frames.  A query is answered once its last future frame has been fed; the
 * queries still waiting keep their q rows in the state.  rope_theta must be
 * 0; ring_slots >= window + F + max_batch - 1 (F = future frames), a
 * multiple of 64.  Layers with different windows use different descs.
 * Its head_dim may also be a multiple of 8 below 64 (the streaming-tiny
 * model's 8 heads of 40, moonshine forward map, "Variant Notes"): inputs,
 * outputs and waiting q rows keep head_dim elements per head, the ring rows
 * are stored padded with zeros to 64 elements, and the softmax scale is
 * 1/sqrt(head_dim). */
typedef struct {
    int32_t kind;        /* vrt_cache_kind */
    int32_t dtype;       /* vrt_dtype: storage and I/O type; accumulation is fp32 */
    int32_t n_layers;    /* layers held by one state (>= 1) */
    int32_t n_heads_q;   /* query heads (multiple of n_heads_kv) */
    int32_t n_heads_kv;  /* key/value heads */
    int32_t head_dim;    /* 64 or 128; ENC_LOOKAHEAD also a multiple of 8 below 64 */
    int32_t window;      /* W: a query at p sees keys in (p - W, p] */
    int32_t ring_slots;  /* ENC_RING: >= window + max_batch; DEC_MODRING: >= window,
                            multiple of 64; ENC_MODRING: >= window - 1 + max_batch,
                            multiple of 64 */
    int32_t max_batch;   /* encoder kinds: largest sub-batch per append (feeds are split) */
    int32_t lookahead;   /* ENC_LOOKAHEAD: the right bound R above; 0 for every other kind */
    double rope_theta;   /* NEOX RoPE base; omega_i = theta^(-2i/head_dim) */
} vrt_cache_desc;

/* Opaque host object: desc, per-layer abs_base / n_kv, the device memory it
 * was given.  It owns no device memory. */
typedef struct vrt_stream_state vrt_stream_state;

const char* vrt_status_str(vrt_status s);
const char* vrt_version(void);

/* Text of the last HIP error that a launch made by this library reported on
 * the calling thread ("" if none).  Diagnostics only; the pointer stays valid
 * until the next failing launch on the same thread. */
const char* vrt_last_device_error(void);

/* Check a descriptor without creating anything.  VRT_ERR_INVALID for
 * non-positive sizes, a nonzero lookahead outside ENC_LOOKAHEAD, or a
 * nonzero rope_theta inside it; VRT_ERR_UNSUPPORTED for a
 * head_dim other than 64/128 (or, for ENC_LOOKAHEAD, a multiple of 8 below
 * 64), an unknown dtype/kind, an ENC_RING ring smaller
 * than window + max_batch (streaming-plan page, "Unbounded length": batches
 * of at most 512 frames so one feed can never overflow the 1536-slot ring),
 * a decoder ring smaller than the window or not a multiple of 64, an
 * ENC_MODRING ring smaller than window - 1 + max_batch or not a multiple
 * of 64, or an ENC_LOOKAHEAD ring smaller than window + F + max_batch - 1 or
 * not a multiple of 64. */
vrt_status vrt_desc_check(const vrt_cache_desc* desc);

/* Device bytes one state needs: for each layer a K ring and a V ring, each
 * [n_heads_kv][ring_slots][row] elements, row = head_dim (64 for a
 * lookahead head_dim below 64); for ENC_LOOKAHEAD then, per layer, F rows of
 * n_heads_q * head_dim elements of waiting queries.  0 if the desc is
 * invalid. */
size_t vrt_state_device_bytes(const vrt_cache_desc* desc);

/* Byte offset, inside a state's device memory, of row 0 of the ring slice
 * (layer, which = 0 for K / 1 for V, kv head).  Rows are head_dim elements
 * (64, zero-padded, for a lookahead head_dim below 64); slot s of that slice
 * starts at offset + s * row * elem_size.  K rows
 * hold RoPE-rotated keys, V rows the values as given.  (size_t)-1 on bad
 * arguments. */
size_t vrt_ring_offset(const vrt_cache_desc* desc, int layer, int which, int kv_head);

/* Create a state over caller memory `dev_mem` of `bytes` (>= the value of
 * vrt_state_device_bytes; 256-byte aligned).  Every layer starts empty with
 * abs_base = start_pos (the absolute position of the first frame that will
 * be fed).  Nothing is written to dev_mem.  VRT_ERR_CAPACITY if bytes is too
 * small.  The state must be destroyed with vrt_stream_state_destroy. */
vrt_status vrt_stream_state_create(const vrt_cache_desc* desc, void* dev_mem, size_t bytes,
                                   int64_t start_pos, vrt_stream_state** out);

/* Clear the stream (every layer: n_kv = 0, abs_base = start_pos), keep the
 * memory, clear the poisoned flag (streaming-plan page, "Per-hook behavior":
 * reset clears streaming state and keeps allocations).  Host-only. */
vrt_status vrt_stream_state_reset(vrt_stream_state* st, int64_t start_pos);

void vrt_stream_state_destroy(vrt_stream_state* st);

/* Host mirror of one layer's ring: abs_base = absolute position held in slot
 * 0 (streaming-plan page, "Unbounded length": stream_enc_abs_base), n_kv =
 * rows held.  For a modulo-ring state (DEC_MODRING, ENC_MODRING) abs_base is
 * the stream's first position and n_kv counts every token written (slot of
 * position p is p % ring_slots). */
vrt_status vrt_stream_state_query(const vrt_stream_state* st, int layer, int64_t* abs_base,
                                  int32_t* n_kv);

/* Pure host planning of one encoder append, the rule every feed applies per
 * (state, layer) before each sub-batch (streaming-plan page, "Unbounded
 * length": contiguous writes, compaction keeping the last `window` frames
 * when the ring would overflow, feeds split into <= max_batch sub-batches).
 * Applies a feed of n_new frames to (*abs_base, *n_kv) in place and returns
 * in *n_compactions how many compactions it implies.  For ENC_MODRING it
 * only adds n_new to *n_kv (no compaction).  No device work.
 * VRT_ERR_INVALID for a decoder desc. */
vrt_status vrt_ring_advance(const vrt_cache_desc* desc, int64_t* abs_base, int32_t* n_kv,
                            int n_new, int32_t* n_compactions);

/* Which attention path a sub-batch of n frames takes: 0 = vector-ALU kernel
 * (fp32 dot products), 1 = matrix-core kernel (bf16 MFMA products, fp32
 * accumulation).  A pure function of the desc and n: 1 exactly for encoder
 * descs (either kind) with bf16 storage, head_dim 64, n_heads_q == n_heads_kv
 * and n >= 32;
 * 0 otherwise; -1 for an invalid desc or n < 1.  A feed is split into
 * sub-batches of at most max_batch frames and each takes its own path; the
 * offline call is one sub-batch of T frames.  Outputs are bit-identical
 * under any chunking whose sub-batches all take the same path; the two paths
 * agree within bf16 rounding. */
int vrt_attn_path(const vrt_cache_desc* desc, int n);

/* Launch plan of the attention kernel for one sub-batch of n frames (for a
 * decoder desc: n tokens, 1 = the split decode step) over `units`
 * (state, layer) caches in one launch: the kv heads each workgroup streams
 * (*heads_per_group), the key splits per (unit, head group) (*n_splits, 1
 * except for the decode step) and the query chunks per unit (*n_qchunks).
 * The plan follows the unit count and the current device's compute units
 * and LDS size (256 and 160 KB when no device answers); outputs are
 * bit-identical under every plan, since each query's arithmetic depends
 * only on its own window and the absolute tile grid.  Host-only.
 * VRT_ERR_INVALID on null outputs, units < 1 or n < 1. */
vrt_status vrt_attn_plan(const vrt_cache_desc* desc, int64_t units, int n, int32_t* heads_per_group,
                         int32_t* n_splits, int32_t* n_qchunks);

/* Outputs a feed of n_new frames produces per (state, layer) when that layer
 * has been fed n_kv frames before: n_new for ENC_RING and ENC_MODRING;
 * max(0, n_kv + n_new - F) - max(0, n_kv - F) for ENC_LOOKAHEAD (a query is
 * answered once F frames past it exist).  -1 for invalid arguments. */
int vrt_attn_out_frames(const vrt_cache_desc* desc, int32_t n_kv, int n_new);

/* Offline windowed attention over one whole sequence (streaming-plan page,
 * "Why offline == streaming" and the bounded-window re-encode section: the
 * whole-clip encoder under the 750-frame windowed-causal mask).
 * q [T][n_heads_q][head_dim], k/v [T][n_heads_kv][head_dim], out like q;
 * positions are start_pos + t.  `scratch` (device, caller-owned, at least
 * vrt_offline_scratch_bytes) receives the rotated keys and the values in
 * head-major order.  Same kernels and arithmetic as the streamed path, so a
 * streamed run on the same path is bit-identical to this call.
 * Encoder descs only (VRT_ERR_INVALID otherwise). */
size_t vrt_offline_scratch_bytes(const vrt_cache_desc* desc, int T);
vrt_status vrt_enc_attn_offline(const vrt_cache_desc* desc, const void* q, const void* k,
                                const void* v, int T, int64_t start_pos, void* out,
                                void* scratch, size_t scratch_bytes, hipStream_t stream);

/* One feed of n_new frames to layers [layer0, layer0 + n_layers) of each of
 * n_states encoder states (streaming-plan page, "Mechanism": the chunk's K/V
 * are written at rows [n_kv_before, n_kv_total) and the queries then read
 * rows [0, n_kv_total) under the windowed mask).  Per (state, layer) and per
 * sub-batch of <= max_batch frames: compaction if needed (ENC_RING only),
 * RoPE + append, then attention of the sub-batch's queries (each new query
 * also sees the earlier new frames of its feed).
 * q/out: [n_states][n_layers][n_new][n_heads_q][head_dim];
 * k/v:   [n_states][n_layers][n_new][n_heads_kv][head_dim].
 * For ENC_LOOKAHEAD the answered queries are written, oldest first, to the
 * first vrt_attn_out_frames rows of each (state, layer) in out; every
 * (state, layer) of the call must hold the same number of waiting queries.
 * All states must share one desc (field-wise equal) and be distinct.
 * VRT_ERR_INVALID on null pointers, n_new < 1, bad layer range, mixed descs,
 * a repeated state, or a decoder state. */
vrt_status vrt_enc_attn_feed(vrt_stream_state* const* states, int n_states, int layer0,
                             int n_layers, const void* q, const void* k, const void* v,
                             int n_new, void* out, hipStream_t stream);

/* Compact layers [layer0, layer0 + n_layers) of each state now: keep the last
 * `window` rows at the front (streaming-plan page, "Unbounded length": copy
 * the last 750 frames to the front).  A no-op for a layer with
 * n_kv <= window, and for ENC_MODRING states (nothing is ever compacted).
 * Encoder states only. */
vrt_status vrt_ring_compact(vrt_stream_state* const* states, int n_states, int layer0,
                            int n_layers, hipStream_t stream);

/* Decoder attention for n_tok tokens per (state, layer) (family doc,
 * Streaming row item 5: token cur is written to slot cur % ring_slots, RoPE
 * positions stay absolute, the step reveals [cur - window + 1, cur]; GQA:
 * query head h reads kv head h / (n_heads_q / n_heads_kv)).  n_tok = 1 is
 * the decode step (split over keys, then a log-sum-exp merge in ascending
 * key order); n_tok > 1 is a prefill (family doc: the 39-token prompt) and
 * may not overwrite a slot that one of its own queries still needs
 * (VRT_ERR_INVALID).
 * q/out: [n_states][n_layers][n_tok][n_heads_q][head_dim]; k/v as for feed.
 * `workspace` (device, caller-owned, 16-byte aligned; 128-byte alignment puts
 * every split's partial record on whole cache lines) must hold
 * vrt_dec_workspace_bytes; VRT_ERR_INVALID if it is null or misaligned. */
size_t vrt_dec_workspace_bytes(const vrt_cache_desc* desc, int n_states, int n_layers,
                               int n_tok);
vrt_status vrt_dec_attn_step(vrt_stream_state* const* states, int n_states, int layer0,
                             int n_layers, const void* q, const void* k, const void* v,
                             int n_tok, void* out, void* workspace, size_t ws_bytes,
                             hipStream_t stream);

/* The decode step of vrt_dec_attn_step without a workspace argument, for
 * callers that cannot allocate device memory (code under HIP graph capture,
 * tight serving loops, harnesses that forbid allocation): the split-K
 * partials go to a static device array inside the library, 128 MiB on each
 * device it runs on, held until the process ends; this call itself
 * allocates nothing (its first call on a device looks the array's address
 * up).  The same kernels and arithmetic as vrt_dec_attn_step, so the outputs
 * are bit-identical.  n_tok = 1 needs vrt_dec_workspace_bytes(desc,
 * n_states, n_layers, 1) <= 128 MiB (VRT_ERR_CAPACITY otherwise; the
 * 32-stream x 26-layer step at window 8192 needs 69.1 MiB); n_tok > 1 (a
 * prefill) uses no partials.  Nothing in the array has to start at zero:
 * the merge reads only the splits the same call wrote.  Every call on one
 * device shares that device's array and it keeps the last call's contents,
 * so calls that overlap on one device (different host threads or streams
 * without ordering between them) race and must not be made. */
vrt_status vrt_dec_attn_step_static(vrt_stream_state* const* states, int n_states, int layer0,
                                    int n_layers, const void* q, const void* k, const void* v,
                                    int n_tok, void* out, hipStream_t stream);

/* ---- The attention half of an encoder block around the path (family doc,
 * "Architecture (summary)", Encoder bullet: pre-norm RMSNorm blocks, NEOX
 * RoPE, the causal 750-frame sliding window, biases on q, v and o and none on
 * k).  bf16 storage throughout, fp32 accumulation; every intermediate is
 * rounded to bf16 once, where it is stored. */

/* y[r] = x[r] / sqrt(mean(x[r]^2) + eps) * w, row by row: x, y [rows][dim],
 * w [dim], bf16, 16-byte aligned; dim a multiple of 8 and at most 2048.
 * Computed in fp32 with one rounding.  VRT_ERR_INVALID on bad sizes,
 * pointers, alignment or eps (negative or not finite). */
vrt_status vrt_rmsnorm(const void* x, int rows, int dim, const void* w, float eps, void* y,
                       hipStream_t stream);

/* out = A W^T (+ bias) (+ residual): A [M][K], W [N][K] (one row per output
 * column, a projection matrix as stored), bias [N] or null, residual [M][N]
 * or null, out [M][N]; bf16, fp32 accumulation on the matrix cores, one
 * rounding.  A and W 16-byte aligned.  VRT_ERR_UNSUPPORTED unless K is a
 * multiple of 64 and N a multiple of 128; VRT_ERR_INVALID on null or
 * misaligned pointers or M < 1.  out must not overlap A, W or residual. */
vrt_status vrt_linear(const void* A, int M, int K, const void* W, int N, const void* bias,
                      const void* residual, void* out, hipStream_t stream);

/* Weights of one block's attention half, device pointers, bf16, with
 * dim = n_heads * head_dim features in head-major order. */
typedef struct {
    const void* norm_w;  /* [dim] RMSNorm gain */
    const void* w_qkv;   /* [3 * dim][dim]: the rows of Wq, then Wk, then Wv */
    const void* b_q;     /* [dim] or null */
    const void* b_v;     /* [dim] or null (k has no bias) */
    const void* w_o;     /* [dim][dim] */
    const void* b_o;     /* [dim] or null */
    float eps;           /* RMSNorm epsilon (the pages print none; 1e-5 is usual) */
    int32_t reserved;    /* must be 0 */
} vrt_block_weights;

/* Workspace of vrt_enc_block_feed for n_rows = n_states * n_new rows: the
 * normed rows, q, k, v and the attention output, bf16, each 256-byte
 * aligned.  0 for an invalid desc or n_rows < 1. */
size_t vrt_block_workspace_bytes(const vrt_cache_desc* desc, int n_rows);

/* One feed through the attention half of layer `layer` of each state:
 *   y = RMSNorm(x); q = y Wq^T + b_q; k = y Wk^T; v = y Wv^T + b_v;
 *   a = the cached path (vrt_enc_attn_feed with q, k, v, one layer);
 *   out = x + a Wo^T + b_o.
 * x/out: [n_states][n_new][dim].  Encoder ring states (ENC_RING or
 * ENC_MODRING) with bf16 storage and n_heads_q == n_heads_kv; dim a multiple
 * of 128 and at most 2048.  ENC_LOOKAHEAD states are refused
 * (VRT_ERR_UNSUPPORTED): their answered queries lag the rows fed, so the
 * residual rows would not line up.  Every check of vrt_enc_attn_feed is made
 * before anything is enqueued, plus VRT_ERR_INVALID for null or misaligned
 * (16-byte) pointers, a nonzero reserved field or eps < 0, VRT_ERR_CAPACITY
 * for a short workspace, VRT_ERR_UNSUPPORTED for other storage or head
 * layouts.  The states advance exactly as under vrt_enc_attn_feed; a failed
 * launch at any point poisons them. */
vrt_status vrt_enc_block_feed(vrt_stream_state* const* states, int n_states, int layer,
                              const void* x, int n_new, const vrt_block_weights* w, void* out,
                              void* workspace, size_t ws_bytes, hipStream_t stream);

/* ---- The causal conv stem ahead of the encoder (family doc, "Architecture
 * (summary)", Encoder bullet: n_mel -> d_model with kernel 3 and stride 1,
 * then d_model -> d_model with kernel 3 and stride 2, each with bias and
 * GELU; streaming-plan page, "Chunk alignment": left padding 2 and 1, kept
 * across chunks as padding caches, so a streamed stem equals the offline
 * one).  bf16 storage, fp32 accumulation on the matrix cores; the conv0
 * output is rounded to bf16 where it is stored; GELU is the exact erf form.
 *
 * A stem object holds one stream's caches in caller-owned device memory: the
 * last 2 mel frames, and the 1 or 2 conv0 frames that conv1's next stride-2
 * window still needs.  Before the first feed both read as zeros (the causal
 * padding); nothing is written at creation. */
typedef struct vrt_conv_stem vrt_conv_stem;

/* Device bytes of one stem (n_mel a multiple of 64, d_model of 128; 0 if
 * not). */
size_t vrt_conv_stem_device_bytes(int n_mel, int d_model);
/* dev_mem: 256-byte aligned, at least vrt_conv_stem_device_bytes.
 * VRT_ERR_UNSUPPORTED for other sizes, VRT_ERR_CAPACITY for short memory. */
vrt_status vrt_conv_stem_create(int n_mel, int d_model, void* dev_mem, size_t bytes,
                                vrt_conv_stem** out);
/* Host-only: the caches read as zeros again, as before the first feed. */
vrt_status vrt_conv_stem_reset(vrt_conv_stem* c);
void vrt_conv_stem_destroy(vrt_conv_stem* c);
/* Mel frames fed since the last reset, and conv0 frames pending (1 or 2). */
vrt_status vrt_conv_stem_query(const vrt_conv_stem* c, int64_t* frames_in, int32_t* pending);
/* Stem outputs a feed of n_frames mel frames would give: (pending + n - 1) / 2
 * when pending + n >= 3, else 0 (8 frames after an 8-frame feed give 4).
 * -1 on bad arguments.  Pure host planning. */
int vrt_conv_out_frames(const vrt_conv_stem* c, int n_frames);

/* Conv weights, device pointers, bf16, tap-major: w0[o][k * n_mel + c] is
 * conv0's weight[o][c][k] (k = 0 the oldest frame), w1[o][k * d_model + c]
 * conv1's; biases [d_model] or null. */
typedef struct {
    const void* w0;
    const void* b0;
    const void* w1;
    const void* b1;
} vrt_conv_weights;

size_t vrt_conv_workspace_bytes(int n_mel, int d_model, int n_stems, int n_frames);

/* Feed n_frames new mel frames to each of n_stems stems: mel
 * [n_stems][n_frames][n_mel]; out [n_stems][*n_out][d_model] receives the
 * stem outputs that became computable (*n_out = vrt_conv_out_frames).  All
 * stems must have the same dimensions and the same pending count, and be
 * distinct (VRT_ERR_INVALID otherwise); at most 256 per call.  mel, out,
 * workspace, w0 and w1 16-byte aligned.  The caches advance as the work is
 * enqueued.  On VRT_ERR_DEVICE the stems are left as they were (host state
 * and caches): the caches are written only by the call's last launch, so
 * the feed can be made again. */
vrt_status vrt_conv_stem_feed(vrt_conv_stem* const* stems, int n_stems, const void* mel,
                              int n_frames, const vrt_conv_weights* w, void* out, int32_t* n_out,
                              void* workspace, size_t ws_bytes, hipStream_t stream);

/* Measurement only: one pass that reads bytes / 16 16-byte chunks of buf
 * (16-byte aligned) as fast as the part allows and writes nothing but,
 * never in practice, one word to sink (4-byte aligned).  Timing it gives the
 * practical streaming-read ceiling beside the nominal HBM bandwidth (the
 * survey's advice: confirm the constants with measured kernels). */
vrt_status vrt_read_probe(const void* buf, size_t bytes, void* sink, hipStream_t stream);

/* Measurement only: the vector attention kernel's tile stream with none of
 * its arithmetic, to set its HBM rate beside vrt_read_probe's ceiling
 * (flags 1: the non-temporal loads that kernel uses; flags 0: plain loads,
 * as the GEMMs use, e.g. for a stream kept in L2).  Other flag bits are
 * invalid.
 * n_wg workgroups; workgroup w reads regions (w * heads + h) mod n_regions,
 * h < heads, region r starting at buf + r * region_stride: from each,
 * `tiles` consecutive 8 KB K tiles and the 8 KB tiles kv_off bytes further
 * on (its V rows), a 16 KB tile at a time through two LDS stages with one
 * workgroup barrier per tile, `passes` times over.  The first tile of each
 * region is read from its row first_row on, the last up to its row last_row
 * (rows are 128 bytes, 64 to a tile); rows outside fetch the nearest row read,
 * as the attention kernel's tiles at a window's edges do (0 and 63: whole
 * tiles).  Writes nothing but, never in practice, one word to sink (4-byte
 * aligned).  buf 16-byte aligned, region_stride and kv_off multiples of 16,
 * every byte read below buf + bytes, all counts >= 1, 0 <= first_row,
 * last_row <= 63 and, for one tile, first_row <= last_row; else
 * VRT_ERR_INVALID.  A small n_regions keeps the stream in L2. */
vrt_status vrt_tile_stream_probe(const void* buf, size_t bytes, int n_wg, int heads, int tiles, int n_regions,
                                 size_t region_stride, size_t kv_off, int passes, int first_row, int last_row,
                                 int flags, void* sink, hipStream_t stream);

/* Per-component timing (the pages time each stage of a streamed feed on its
 * own: family doc, Capability Validation table, Streaming row, items 7 and
 * 8).  While both events are non-null, every later call on this thread
 * records `start` on its stream just before each attention launch (after the
 * compaction and append launches of the same sub-batch) and `stop` just
 * after it (for the decode step, after the merge launch), so
 * hipEventElapsedTime(start, stop) covers the attention kernels alone; a
 * call with several attention launches leaves the pair on its last one.
 * Events are caller-owned hipEvent_t handles created with timing enabled;
 * passing two nulls turns recording off.  This per-thread pair is the only
 * setting the library keeps.  VRT_ERR_INVALID if exactly one is null or a
 * handle is not a valid event. */
vrt_status vrt_set_attn_events(hipEvent_t start, hipEvent_t stop);

/* Testing only: exercises the error paths and the host planning without
 * faulting a GPU.  From this call on, on the calling thread, the fail_at-th
 * kernel launch the library makes (counting from 1; 0 = none) reports a
 * launch error without launching anything, as a failed launch would; with
 * dry_run = 1 no kernel is launched at all (every other launch is skipped
 * and reported successful, and no HIP call is made to enqueue work), so the
 * metadata, poisoning and "nothing enqueued" rules can be checked on a host
 * without a GPU.  Device memory is never touched in dry-run mode, but the
 * state metadata advances as if the work had run.  Setting the hook restarts
 * the launch count; vrt_test_launch_hook(0, 0) turns it off.
 * vrt_test_launch_count returns the launches (made, failed or skipped) that
 * reached the library's launch gate on this thread since the hook was last
 * set. */
void vrt_test_launch_hook(int32_t fail_at, int32_t dry_run);
int64_t vrt_test_launch_count(void);

#ifdef __cplusplus
}
#endif

#endif /* VRT_H */
