"""Oracle for the quantized KV-cache store and compressed-domain attention.

TEST INFRASTRUCTURE ONLY.  This package is a plain, slow CPU statement of what
the hot path computes, written from the three source pages:

  [tract-RFC]     "Heads-up / RFC: int4 + Hadamard KV-cache quantization
                  (CPU + Metal)", tract discussion #2402
  [FreeToken-268] "feat(kvcache): sub-byte Q4_0 and Q6_0 KV cache
                  quantization", FreeToken PR #268
  [Open-TQ-Metal] "Open-TQ-Metal: Fused Compressed-Domain Attention for
                  Long-Context LLM Inference on Apple Silicon", arXiv 2604.16957

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import it.  It shares no code with the HIP library and never
imports it.  Floating point is float64; wherever the encoding has a rounding
point (an f32 or f16 value that the cache stores or that decides an integer
code) the value is rounded there to f32/f16 explicitly, exactly as an IEEE
single/half operation would round it.

Modules
  spec       layout constants (bytes per token, groups, code ranges)
  fwht       orthonormal Walsh-Hadamard transform: dense definition and the
             f32 butterfly encoding step
  quant      quantisers, packers, unpackers and dequantisers per layout
  attention  integer scores, decode attention, causal prefill, split-K merge
"""

from . import spec, fwht, quant, attention  # noqa: F401
