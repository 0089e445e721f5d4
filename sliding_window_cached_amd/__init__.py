"""Python binding of libvrt (the C ABI declared in include/vrt.h).

Argument marshalling only: every step of the path runs in the HIP library.
Device buffers are passed as raw pointers; anything with a ``data_ptr()``
method (a torch tensor on the GPU) or a plain int is accepted.  Streams are
``hipStream_t`` handles as ints (``torch.cuda.current_stream().cuda_stream``),
0 for the null stream.

Importing this module loads ``libvrt.so`` from this directory and raises if
it is missing: there is no fallback path.
"""
from __future__ import annotations

import ctypes
import os
from ctypes import POINTER, Structure, byref, c_char_p, c_double, c_int, c_int32, c_int64, \
    c_size_t, c_void_p

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libvrt.so")

F32, BF16 = 0, 1
ENC_RING, DEC_MODRING, ENC_MODRING, ENC_LOOKAHEAD = 0, 1, 2, 3
OK, ERR_INVALID, ERR_UNSUPPORTED, ERR_CAPACITY, ERR_DEVICE, ERR_POISONED = range(6)

EXPORTS = (
    "vrt_status_str", "vrt_version", "vrt_last_device_error", "vrt_desc_check", "vrt_state_device_bytes",
    "vrt_ring_offset", "vrt_stream_state_create", "vrt_stream_state_reset",
    "vrt_stream_state_destroy", "vrt_stream_state_query", "vrt_ring_advance", "vrt_attn_path",
    "vrt_attn_out_frames",
    "vrt_offline_scratch_bytes", "vrt_enc_attn_offline", "vrt_enc_attn_feed",
    "vrt_ring_compact", "vrt_dec_workspace_bytes", "vrt_dec_attn_step", "vrt_set_attn_events",
    "vrt_rmsnorm", "vrt_linear", "vrt_block_workspace_bytes", "vrt_enc_block_feed",
    "vrt_conv_stem_device_bytes", "vrt_conv_stem_create", "vrt_conv_stem_reset",
    "vrt_conv_stem_destroy", "vrt_conv_stem_query", "vrt_conv_out_frames",
    "vrt_conv_workspace_bytes", "vrt_conv_stem_feed", "vrt_read_probe", "vrt_tile_stream_probe", "vrt_attn_plan",
    "vrt_test_launch_hook", "vrt_test_launch_count", "vrt_dec_attn_step_static",
)


class BlockWeights(Structure):
    """vrt_block_weights: device pointers of one block's attention half."""
    _fields_ = [("norm_w", ctypes.c_void_p), ("w_qkv", ctypes.c_void_p), ("b_q", ctypes.c_void_p),
                ("b_v", ctypes.c_void_p), ("w_o", ctypes.c_void_p), ("b_o", ctypes.c_void_p),
                ("eps", ctypes.c_float), ("reserved", c_int32)]


class ConvWeights(Structure):
    """vrt_conv_weights: tap-major conv weights and biases (device pointers)."""
    _fields_ = [("w0", ctypes.c_void_p), ("b0", ctypes.c_void_p), ("w1", ctypes.c_void_p),
                ("b1", ctypes.c_void_p)]


class CacheDesc(Structure):
    _fields_ = [
        ("kind", c_int32), ("dtype", c_int32), ("n_layers", c_int32),
        ("n_heads_q", c_int32), ("n_heads_kv", c_int32), ("head_dim", c_int32),
        ("window", c_int32), ("ring_slots", c_int32), ("max_batch", c_int32),
        ("lookahead", c_int32), ("rope_theta", c_double),
    ]


def enc_desc(dtype=BF16, n_layers=1, heads=20, head_dim=64, window=750, ring_slots=None,
             max_batch=512, theta=1.0e6, kind=ENC_RING) -> CacheDesc:
    """Encoder cache as on the pages: 20 heads x 64, window 750, 1536 slots
    (kind ENC_RING, compaction).  kind=ENC_MODRING stores the same cache as a
    modulo ring (slot = position % ring_slots, no compaction); its default
    ring is window - 1 + max_batch rounded up to a multiple of 64 (1280)."""
    if ring_slots is None:
        ring_slots = 1536 if kind == ENC_RING else -(-(window - 1 + max_batch) // 64) * 64
    return CacheDesc(kind, dtype, n_layers, heads, heads, head_dim, window, ring_slots,
                     max_batch, 0, theta)


def lookahead_desc(left, right, dtype=BF16, n_layers=1, heads=8, head_dim=64, max_batch=512,
                   ring_slots=None) -> CacheDesc:
    """(left, right) windows without RoPE (the moonshine streaming encoder's
    per-layer masks): keys u with t - u in [0, left) or u - t in (0, right)."""
    f = max(right - 1, 0)
    if ring_slots is None:
        ring_slots = -(-(left + f + max_batch - 1) // 64) * 64
    return CacheDesc(ENC_LOOKAHEAD, dtype, n_layers, heads, heads, head_dim, left, ring_slots,
                     max_batch, right, 0.0)


def dec_desc(dtype=BF16, n_layers=1, heads_q=32, heads_kv=8, head_dim=128, window=8192,
             ring_slots=8192, max_batch=512, theta=1.0e6) -> CacheDesc:
    """Decoder cache as on the pages: GQA 32/8, 128, window = ring = 8192."""
    return CacheDesc(DEC_MODRING, dtype, n_layers, heads_q, heads_kv, head_dim, window,
                     ring_slots, max_batch, 0, theta)


class VrtError(RuntimeError):
    def __init__(self, status: int, what: str):
        self.status = status
        msg = f"{what}: {status_str(status)} ({status})"
        if status == ERR_DEVICE:
            msg += f": {last_device_error()}"
        super().__init__(msg)


def _preload_hip_runtime():
    """Use the HIP runtime PyTorch ships, when PyTorch is installed.

    Two HIP runtimes in one process cannot share the GPU: the second one to
    start sees no device.  PyTorch's ROCm wheel carries its own
    libamdhip64.so (soname libamdhip64.so.7, the one libvrt.so needs), so
    mapping that copy first makes both libraries bind to a single runtime,
    whichever of them the program imports first.  PyTorch itself is not
    imported here."""
    import importlib.util
    spec = importlib.util.find_spec("torch")
    if spec is None or not spec.origin:
        return None
    path = os.path.join(os.path.dirname(spec.origin), "lib", "libamdhip64.so")
    if os.path.exists(path):
        ctypes.CDLL(path, mode=ctypes.RTLD_GLOBAL)
        return path
    return None


HIP_RUNTIME = None


def _load():
    global HIP_RUNTIME
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is missing: build it with __graft_entry__.build() "
                          "(there is no fallback path)")
    HIP_RUNTIME = _preload_hip_runtime()
    lib = ctypes.CDLL(LIB_PATH)
    P = c_void_p
    sig = {
        "vrt_status_str": (c_char_p, [c_int]),
        "vrt_version": (c_char_p, []),
        "vrt_last_device_error": (c_char_p, []),
        "vrt_desc_check": (c_int, [POINTER(CacheDesc)]),
        "vrt_state_device_bytes": (c_size_t, [POINTER(CacheDesc)]),
        "vrt_ring_offset": (c_size_t, [POINTER(CacheDesc), c_int, c_int, c_int]),
        "vrt_stream_state_create": (c_int, [POINTER(CacheDesc), P, c_size_t, c_int64, POINTER(P)]),
        "vrt_stream_state_reset": (c_int, [P, c_int64]),
        "vrt_stream_state_destroy": (None, [P]),
        "vrt_stream_state_query": (c_int, [P, c_int, POINTER(c_int64), POINTER(c_int32)]),
        "vrt_ring_advance": (c_int, [POINTER(CacheDesc), POINTER(c_int64), POINTER(c_int32), c_int,
                                     POINTER(c_int32)]),
        "vrt_attn_path": (c_int, [POINTER(CacheDesc), c_int]),
        "vrt_attn_out_frames": (c_int, [POINTER(CacheDesc), c_int32, c_int]),
        "vrt_offline_scratch_bytes": (c_size_t, [POINTER(CacheDesc), c_int]),
        "vrt_enc_attn_offline": (c_int, [POINTER(CacheDesc), P, P, P, c_int, c_int64, P, P,
                                         c_size_t, P]),
        "vrt_enc_attn_feed": (c_int, [POINTER(P), c_int, c_int, c_int, P, P, P, c_int, P, P]),
        "vrt_ring_compact": (c_int, [POINTER(P), c_int, c_int, c_int, P]),
        "vrt_dec_workspace_bytes": (c_size_t, [POINTER(CacheDesc), c_int, c_int, c_int]),
        "vrt_dec_attn_step": (c_int, [POINTER(P), c_int, c_int, c_int, P, P, P, c_int, P, P,
                                      c_size_t, P]),
        "vrt_set_attn_events": (c_int, [P, P]),
        "vrt_dec_attn_step_static": (c_int, [POINTER(P), c_int, c_int, c_int, P, P, P, c_int, P, P]),
        "vrt_rmsnorm": (c_int, [P, c_int, c_int, P, ctypes.c_float, P, P]),
        "vrt_linear": (c_int, [P, c_int, c_int, P, c_int, P, P, P, P]),
        "vrt_block_workspace_bytes": (c_size_t, [POINTER(CacheDesc), c_int]),
        "vrt_enc_block_feed": (c_int, [POINTER(P), c_int, c_int, P, c_int, POINTER(BlockWeights), P,
                                       P, c_size_t, P]),
        "vrt_conv_stem_device_bytes": (c_size_t, [c_int, c_int]),
        "vrt_conv_stem_create": (c_int, [c_int, c_int, P, c_size_t, POINTER(P)]),
        "vrt_conv_stem_reset": (c_int, [P]),
        "vrt_conv_stem_destroy": (None, [P]),
        "vrt_conv_stem_query": (c_int, [P, POINTER(c_int64), POINTER(c_int32)]),
        "vrt_conv_out_frames": (c_int, [P, c_int]),
        "vrt_conv_workspace_bytes": (c_size_t, [c_int, c_int, c_int, c_int]),
        "vrt_read_probe": (c_int, [P, c_size_t, P, P]),
        "vrt_tile_stream_probe": (c_int, [P, c_size_t, c_int, c_int, c_int, c_int, c_size_t, c_size_t, c_int, c_int,
                                          c_int, c_int, P, P]),
        "vrt_attn_plan": (c_int, [POINTER(CacheDesc), c_int64, c_int, POINTER(c_int32),
                                  POINTER(c_int32), POINTER(c_int32)]),
        "vrt_test_launch_hook": (None, [c_int32, c_int32]),
        "vrt_test_launch_count": (c_int64, []),
        "vrt_conv_stem_feed": (c_int, [POINTER(P), c_int, P, c_int, POINTER(ConvWeights), P,
                                       POINTER(c_int32), P, c_size_t, P]),
    }
    for name, (res, args) in sig.items():
        f = getattr(lib, name)
        f.restype = res
        f.argtypes = args
    return lib


lib = _load()


def status_str(s: int) -> str:
    return lib.vrt_status_str(s).decode()


def version() -> str:
    return lib.vrt_version().decode()


def last_device_error() -> str:
    return lib.vrt_last_device_error().decode()


def _ptr(x) -> int | None:
    if x is None:
        return None
    if isinstance(x, int):
        return x
    return x.data_ptr()


def _check(s: int, what: str) -> None:
    if s != OK:
        raise VrtError(s, what)


def desc_check(desc: CacheDesc) -> int:
    return lib.vrt_desc_check(byref(desc))


def state_device_bytes(desc: CacheDesc) -> int:
    return lib.vrt_state_device_bytes(byref(desc))


def ring_offset(desc: CacheDesc, layer: int, which: int, kv_head: int) -> int:
    return lib.vrt_ring_offset(byref(desc), layer, which, kv_head)


def attn_out_frames(desc: CacheDesc, n_kv: int, n_new: int) -> int:
    return lib.vrt_attn_out_frames(byref(desc), n_kv, n_new)


def attn_path(desc: CacheDesc, n: int) -> int:
    return lib.vrt_attn_path(byref(desc), n)


def attn_plan(desc: CacheDesc, units: int, n: int):
    """(kv heads per workgroup, key splits, query chunks per unit) of the
    attention launch for a sub-batch of n frames over `units` caches."""
    hg, sp, qc = c_int32(), c_int32(), c_int32()
    _check(lib.vrt_attn_plan(byref(desc), units, n, byref(hg), byref(sp), byref(qc)), "attn_plan")
    return hg.value, sp.value, qc.value


def test_launch_hook(fail_at: int = 0, dry_run: bool = False) -> None:
    """Testing only: make the fail_at-th next launch fail (0: none); with
    dry_run, skip every launch (host logic without a GPU)."""
    lib.vrt_test_launch_hook(fail_at, 1 if dry_run else 0)


def test_launch_count() -> int:
    return lib.vrt_test_launch_count()


def ring_advance(desc: CacheDesc, abs_base: int, n_kv: int, n_new: int):
    """Pure host planning of one encoder feed: (abs_base, n_kv, n_compactions)."""
    b, k, c = c_int64(abs_base), c_int32(n_kv), c_int32(0)
    _check(lib.vrt_ring_advance(byref(desc), byref(b), byref(k), n_new, byref(c)), "ring_advance")
    return b.value, k.value, c.value


class StreamState:
    """One stream's multi-layer cache over caller-owned device memory."""

    def __init__(self, desc: CacheDesc, dev_mem, nbytes: int, start_pos: int = 0):
        self.desc = desc
        self.mem = dev_mem          # keep the owner (e.g. a torch tensor) alive
        h = c_void_p()
        _check(lib.vrt_stream_state_create(byref(desc), _ptr(dev_mem), nbytes, start_pos,
                                           byref(h)), "stream_state_create")
        self.handle = h.value

    def reset(self, start_pos: int) -> None:
        _check(lib.vrt_stream_state_reset(self.handle, start_pos), "stream_state_reset")

    def query(self, layer: int):
        b, k = c_int64(), c_int32()
        s = lib.vrt_stream_state_query(self.handle, layer, byref(b), byref(k))
        if s not in (OK, ERR_POISONED):
            _check(s, "stream_state_query")
        return b.value, k.value

    def status(self) -> int:
        """OK, or ERR_POISONED after a failed launch (until reset)."""
        return lib.vrt_stream_state_query(self.handle, 0, None, None)

    def close(self) -> None:
        if self.handle:
            lib.vrt_stream_state_destroy(self.handle)
            self.handle = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


def _handles(states):
    arr = (c_void_p * len(states))(*[s.handle for s in states])
    return arr


def offline_scratch_bytes(desc: CacheDesc, T: int) -> int:
    return lib.vrt_offline_scratch_bytes(byref(desc), T)


def enc_attn_offline(desc, q, k, v, T, start_pos, out, scratch, scratch_bytes, stream=0):
    _check(lib.vrt_enc_attn_offline(byref(desc), _ptr(q), _ptr(k), _ptr(v), T, start_pos,
                                    _ptr(out), _ptr(scratch), scratch_bytes, stream),
           "enc_attn_offline")


def enc_attn_feed(states, layer0, n_layers, q, k, v, n_new, out, stream=0, check=True):
    s = lib.vrt_enc_attn_feed(_handles(states), len(states), layer0, n_layers, _ptr(q), _ptr(k),
                              _ptr(v), n_new, _ptr(out), stream)
    if check:
        _check(s, "enc_attn_feed")
    return s


def ring_compact(states, layer0, n_layers, stream=0):
    _check(ring_compact_status(states, layer0, n_layers, stream), "ring_compact")


def ring_compact_status(states, layer0, n_layers, stream=0) -> int:
    return lib.vrt_ring_compact(_handles(states), len(states), layer0, n_layers, stream)


def dec_workspace_bytes(desc, n_states, n_layers, n_tok) -> int:
    return lib.vrt_dec_workspace_bytes(byref(desc), n_states, n_layers, n_tok)


def dec_attn_step(states, layer0, n_layers, q, k, v, n_tok, out, workspace=None, ws_bytes=0,
                  stream=0, check=True):
    s = lib.vrt_dec_attn_step(_handles(states), len(states), layer0, n_layers, _ptr(q), _ptr(k),
                              _ptr(v), n_tok, _ptr(out), _ptr(workspace), ws_bytes, stream)
    if check:
        _check(s, "dec_attn_step")
    return s


def dec_attn_step_static(states, layer0, n_layers, q, k, v, n_tok, out, stream=0, check=True):
    """The decode step with its partials in the library's static device array
    (allocates nothing; calls that overlap on one device race)."""
    s = lib.vrt_dec_attn_step_static(_handles(states), len(states), layer0, n_layers, _ptr(q), _ptr(k),
                                     _ptr(v), n_tok, _ptr(out), stream)
    if check:
        _check(s, "dec_attn_step_static")
    return s


def rmsnorm(x, rows, dim, w, eps, y, stream=0, check=True):
    s = lib.vrt_rmsnorm(_ptr(x), rows, dim, _ptr(w), eps, _ptr(y), stream)
    if check:
        _check(s, "rmsnorm")
    return s


def linear(A, M, K, W, N, bias, residual, out, stream=0, check=True):
    s = lib.vrt_linear(_ptr(A), M, K, _ptr(W), N, _ptr(bias), _ptr(residual), _ptr(out), stream)
    if check:
        _check(s, "linear")
    return s


def block_weights(norm_w, w_qkv, b_q, b_v, w_o, b_o, eps=1.0e-5) -> BlockWeights:
    """Keep the owners (e.g. torch tensors) alive while the struct is used."""
    return BlockWeights(_ptr(norm_w), _ptr(w_qkv), _ptr(b_q), _ptr(b_v), _ptr(w_o), _ptr(b_o),
                        eps, 0)


def block_workspace_bytes(desc, n_rows) -> int:
    return lib.vrt_block_workspace_bytes(byref(desc), n_rows)


def enc_block_feed(states, layer, x, n_new, weights: BlockWeights, out, workspace, ws_bytes,
                   stream=0, check=True):
    s = lib.vrt_enc_block_feed(_handles(states), len(states), layer, _ptr(x), n_new, byref(weights),
                               _ptr(out), _ptr(workspace), ws_bytes, stream)
    if check:
        _check(s, "enc_block_feed")
    return s


class ConvStem:
    """One stream's conv stem caches over caller-owned device memory."""

    def __init__(self, n_mel: int, d_model: int, dev_mem, nbytes: int):
        self.mem = dev_mem          # keep the owner alive
        h = c_void_p()
        _check(lib.vrt_conv_stem_create(n_mel, d_model, _ptr(dev_mem), nbytes, byref(h)),
               "conv_stem_create")
        self.h = h

    def reset(self):
        _check(lib.vrt_conv_stem_reset(self.h), "conv_stem_reset")

    def query(self):
        f, p = c_int64(), c_int32()
        _check(lib.vrt_conv_stem_query(self.h, byref(f), byref(p)), "conv_stem_query")
        return f.value, p.value

    def out_frames(self, n: int) -> int:
        return lib.vrt_conv_out_frames(self.h, n)

    def close(self):
        if self.h:
            lib.vrt_conv_stem_destroy(self.h)
            self.h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


def conv_stem_device_bytes(n_mel, d_model) -> int:
    return lib.vrt_conv_stem_device_bytes(n_mel, d_model)


def conv_workspace_bytes(n_mel, d_model, n_stems, n_frames) -> int:
    return lib.vrt_conv_workspace_bytes(n_mel, d_model, n_stems, n_frames)


def conv_weights(w0, b0, w1, b1) -> ConvWeights:
    """Keep the owners alive while the struct is used."""
    return ConvWeights(_ptr(w0), _ptr(b0), _ptr(w1), _ptr(b1))


def conv_stem_feed(stems, mel, n_frames, weights: ConvWeights, out, workspace, ws_bytes, stream=0,
                   check=True):
    """Returns the number of stem outputs written per stem (or the status
    when check is False and the call fails)."""
    arr = (c_void_p * len(stems))(*[s.h for s in stems])
    n_out = c_int32(0)
    s = lib.vrt_conv_stem_feed(arr, len(stems), _ptr(mel), n_frames, byref(weights), _ptr(out),
                               byref(n_out), _ptr(workspace), ws_bytes, stream)
    if check:
        _check(s, "conv_stem_feed")
        return n_out.value
    return s if s != OK else n_out.value


def read_probe(buf, nbytes, sink, stream=0):
    _check(lib.vrt_read_probe(_ptr(buf), nbytes, _ptr(sink), stream), "read_probe")


def tile_stream_probe(buf, nbytes, n_wg, heads, tiles, n_regions, region_stride, kv_off, passes, sink, stream=0,
                      nontemporal=True, first_row=0, last_row=63):
    _check(lib.vrt_tile_stream_probe(_ptr(buf), nbytes, n_wg, heads, tiles, n_regions, region_stride, kv_off,
                                     passes, first_row, last_row, 1 if nontemporal else 0, _ptr(sink), stream),
           "tile_stream_probe")


def set_attn_events(start=None, stop=None):
    """Record `start` / `stop` around every later attention launch of this
    thread (torch.cuda.Event objects that have been recorded once, or raw
    hipEvent_t ints); no arguments turns recording off."""
    def h(e):
        if e is None:
            return None
        return e if isinstance(e, int) else e.cuda_event
    _check(lib.vrt_set_attn_events(h(start), h(stop)), "set_attn_events")
