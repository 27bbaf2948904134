"""CPU oracle for the FP4 KV-cache chunk-attention path.

TEST INFRASTRUCTURE ONLY.  This package is a plain, slow, obviously correct
NumPy statement of what the path computes.  Only the test suite, the smoke
check and the benchmark's CPU-baseline leg may import it.  The product path
(the HIP library and its Python binding) never imports, calls or links
anything here, and nothing here imports the product path.

Sources (web pages about LongLive 2.0, cited by host and section):
  * aiany.app, "LongLive 2.0: An NVFP4 Parallel Infrastructure for Long Video
    Generation", sections "What Sets It Apart" and "How It Works (brief)".
  * hysenlabs.com, "NVlabs/LongLive 2.0: NVFP4 parallel infrastructure for
    long video generation", section "NVFP4, sequence parallel and the async
    decode path".
  * heatdrop.ai, "Nvidia's recipe for 45 FPS long-video generation",
    sections "What it does" and "The interesting bit".
  * refft.com, "NVlabs/LongLive" core analysis, question "How do KV-cache
    relative RoPE and TriAttention work together ...".
  * evermx.com, "LongLive ... long video generation", sections "NVFP4
    Quantization End-to-End" and "Multi-Shot Generation".

The pages name the mechanisms (an NVFP4 KV cache written in place, relative
RoPE over the cache, attention sinks, multi-shot masking) but give no
formula.  Where they are silent each module states the reading it takes.

Modules:
  nvfp4     E4M3 / E2M1 element codecs and the NVFP4 block encoder/decoder.
  ring      sink + sliding-window slot bookkeeping, positions and masks.
  rope      rotary position rotation in float64, and the float32 table and
            rotation that keys stored rotated go through.
  attention float64 softmax attention over the decoded cache.
  stream    a cache object that chains the above, in the library's layout
            (keys stored before rotation), and the rotate-at-write variant.

Parity status: every function here is pinned by tests under tests/ against
library routines, closed forms, invariants or brute force; none is marked
"parity unpinned".
"""
