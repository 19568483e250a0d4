"""Quantized KV-cache store and compressed-domain attention for MI355X (gfx950).

A thin binding over libkvq.so, the C-ABI library declared in include/kvq.h.
PyTorch only supplies device memory and the stream; the store, the split-K
decode attention and the causal prefill all run in the library's HIP kernels.
Importing the package does not load the library; the first call does, and
fails loudly if it is not built.
"""

from ._lib import LAYOUT_IDS, KvqError, load  # noqa: F401
from .ops import (KvqCache, attend_decode, attend_decode_noalloc, attend_decode_partial, attend_decode_reduce, attend_prefill_causal,  # noqa: F401
                  attend_step, debug_qk_i32, decode_split, decode_split_lengths, debug_quantize_q, debug_stream_read, decode_workspace_bytes, prefill_full_then_store,
                  prefill_workspace_bytes, store, store_chunk)
