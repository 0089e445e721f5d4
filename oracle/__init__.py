"""Plain, slow, fp64 CPU oracle for streamed windowed-causal attention.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path may import, call or
execute anything in this package; only ``tests/``, ``__graft_entry__.smoke()``
and the ``cpu_baseline`` leg of ``bench.py`` use it.  It shares no code with
the HIP library (no kernels, headers, tables or constant generators) and
imports nothing from it; the one shared module is ``synth`` (seeded inputs).

What it computes (sources are the four pages this method is described on):

* ``rope``      - NEOX rotary embedding at absolute positions, theta 1e6, as a
                  materialised d x d block rotation (Voxtral Realtime family
                  doc, "Architecture (summary)": NEOX RoPE theta=1e6 hd 64 for
                  the encoder, hd 128 for the decoder; the pairing (i, i+d/2)
                  is the NEOX layout that the moonshine forward map contrasts
                  with GPT-J's interleaved 0::2 / 1::2 slices, "Decoder block
                  pattern").
* ``attention`` - windowed-causal attention over a whole sequence: a query at
                  absolute position p sees keys with positions in (p-W, p]
                  (streaming-plan page, bounded-window re-encode section:
                  frame i attends to [i-749, i]; family doc Streaming row
                  item 5: the decoder step reveals [cur-8191, cur]).  GQA maps
                  query head h to kv head h // (Hq/Hkv) (family doc, Decoder
                  bullet: GQA 32q/8kv).
* ``ring``      - the integer ring model: 1536-slot encoder ring with
                  contiguous writes, compaction to the last 750 frames when a
                  sub-batch would overflow it, feeds split into <=512-frame
                  sub-batches, slot 0's absolute position tracked (streaming-
                  plan page, "SHIPPED" section, "Unbounded length"
                  paragraph); decoder modulo ring, slot = pos % 8192 (family
                  doc, Streaming row, item 5).
* ``block``     - the attention half of an encoder block around the path:
                  RMSNorm, q/k/v projections with q and v biases, the
                  windowed attention, the output projection with bias and the
                  residual (family doc, "Architecture (summary)", Encoder
                  bullet).
* ``conv``      - the causal conv stem ahead of the encoder (kernel 3, strides
                  1 and 2, left padding 2 and 1, GELU), offline and streamed
                  with padding caches (family doc, Encoder bullet;
                  streaming-plan page, "Chunk alignment").
* ``stream``    - the same attention driven incrementally through the ring
                  model with explicit fp64 ring buffers, feed by feed.  The
                  pages state the streamed result equals the offline pass
                  (streaming-plan page, "Verification" item 1; bunsen
                  streaming chapter, "Chunking must not be observable").

Pins (tests/test_oracle_*.py, all run with ``-m "not gpu"``): brute force with
an explicit mask matrix on tiny inputs; reduction to plain causal attention
(torch SDPA, float64) when W >= T; closed forms W=1 (out = v) and q=0
(out = window mean of v); window-edge perturbation; RoPE norm preservation,
identity at p=0, composition, relative-position invariance, the d=2 closed
form and the NEOX pairing; bit-identical chunked vs one-shot results; ring
compaction counts in closed form; GQA = MHA with repeated kv heads; decoder
modulo ring = linear buffer.  No output value of this oracle is "parity
unpinned".
"""
from . import rope, attention, ring, stream, block, conv  # noqa: F401
