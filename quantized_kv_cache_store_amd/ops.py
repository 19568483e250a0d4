"""Torch-facing wrappers of the C ABI: argument checks and pointer marshalling only.

Every step of the store and attention runs in libkvq.so's HIP kernels on the
caller's current stream; nothing here computes on the data.
"""

import ctypes

import torch

from . import _lib
from ._lib import KvqCacheDesc, check, load


def _ptr(t):
    return ctypes.c_void_p(t.data_ptr()) if t is not None else ctypes.c_void_p(0)


def _stream(device):
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _need(t, name, dtype, device):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a tensor")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if t.device != device:
        raise ValueError(f"{name} must live on {device}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return t


class KvqCache:
    """Device planes of a paged quantized KV cache (caller-owned memory for the C ABI).

    k_payload/v_payload uint8 [num_pages, Hkv, page_size, payload_bytes]
    k_scale/v_scale     uint8 [num_pages, Hkv, page_size, scale_bytes]
    k_recent/v_recent   f32   [max_batch, Hkv, n_recent, D]   (None when n_recent == 0)
    """

    def __init__(self, layout, head_dim, num_kv_heads, num_pages, page_size, n_recent=0, max_batch=1,
                 device="cuda"):
        lib = load()
        self.layout = _lib.LAYOUT_IDS[layout] if isinstance(layout, str) else int(layout)
        self.head_dim = int(head_dim)
        self.num_kv_heads = int(num_kv_heads)
        self.num_pages = int(num_pages)
        self.page_size = int(page_size)
        self.n_recent = int(n_recent)
        self.max_batch = int(max_batch)
        self.device = torch.device(device)
        pb = lib.kvq_payload_bytes(self.layout, self.head_dim)
        sb = lib.kvq_scale_bytes(self.layout, self.head_dim)
        if pb == 0:
            raise ValueError(f"layout {layout} with head_dim {head_dim} is not supported")
        self.payload_bytes, self.scale_bytes = pb, sb
        shp = (self.num_pages, self.num_kv_heads, self.page_size)
        self.k_payload = torch.zeros(shp + (pb,), dtype=torch.uint8, device=self.device)
        self.v_payload = torch.zeros(shp + (pb,), dtype=torch.uint8, device=self.device)
        self.k_scale = torch.zeros(shp + (sb,), dtype=torch.uint8, device=self.device)
        self.v_scale = torch.zeros(shp + (sb,), dtype=torch.uint8, device=self.device)
        if self.n_recent > 0:
            rs = (self.max_batch, self.num_kv_heads, self.n_recent, self.head_dim)
            self.k_recent = torch.zeros(rs, dtype=torch.float32, device=self.device)
            self.v_recent = torch.zeros(rs, dtype=torch.float32, device=self.device)
        else:
            self.k_recent = self.v_recent = None
        self._desc = KvqCacheDesc(
            self.layout, self.head_dim, self.num_kv_heads, self.page_size, self.num_pages, self.n_recent,
            self.max_batch, 0, self.k_payload.data_ptr(), self.v_payload.data_ptr(), self.k_scale.data_ptr(),
            self.v_scale.data_ptr(), self.k_recent.data_ptr() if self.k_recent is not None else None,
            self.v_recent.data_ptr() if self.v_recent is not None else None)

    @property
    def desc(self):
        return ctypes.byref(self._desc)

    def nbytes(self):
        return sum(t.numel() * t.element_size() for t in
                   (self.k_payload, self.v_payload, self.k_scale, self.v_scale, self.k_recent, self.v_recent)
                   if t is not None)


def store(cache, k_new, v_new, slot, batch_idx=None, pos=None, seq_len=None):
    """kvq_store: quantize-on-append of n_tok tokens (k_new, v_new f32 [n_tok, Hkv, D])."""
    dev = cache.device
    _need(k_new, "k_new", torch.float32, dev)
    _need(v_new, "v_new", torch.float32, dev)
    _need(slot, "slot", torch.int32, dev)
    n = k_new.shape[0]
    if k_new.shape != (n, cache.num_kv_heads, cache.head_dim) or v_new.shape != k_new.shape:
        raise ValueError("k_new and v_new must be [n_tok, Hkv, D]")
    if slot.shape != (n,):
        raise ValueError("slot must be [n_tok]")
    for t, name in ((batch_idx, "batch_idx"), (pos, "pos"), (seq_len, "seq_len")):
        if t is not None:
            _need(t, name, torch.int32, dev)
    st = load().kvq_store(cache.desc, _ptr(k_new), _ptr(v_new), n, _ptr(slot), _ptr(batch_idx), _ptr(pos),
                          _ptr(seq_len), _stream(dev))
    check("kvq_store", st)


def decode_workspace_bytes(batch, num_q_heads, head_dim, max_seq_len, chunk_tokens):
    return load().kvq_decode_workspace_bytes(batch, num_q_heads, head_dim, max_seq_len, chunk_tokens)


def attend_decode(cache, q, block_table, seq_len, max_seq_len, alpha, chunk_tokens=512, out=None,
                  workspace=None, float_q=False):
    """kvq_attend_decode: q f32 [B, Hq, D] -> out f32 [B, Hq, D].

    float_q=True calls kvq_attend_decode_float_q (quantised tokens scored with the f32 query).
    """
    dev = cache.device
    _need(q, "q", torch.float32, dev)
    _need(block_table, "block_table", torch.int32, dev)
    _need(seq_len, "seq_len", torch.int32, dev)
    B, Hq, D = q.shape
    if block_table.dim() != 2 or block_table.shape[0] != B or seq_len.shape != (B,):
        raise ValueError("block_table must be [B, max_pages] and seq_len [B]")
    if out is None:
        out = torch.empty_like(q)
    _need(out, "out", torch.float32, dev)
    need = decode_workspace_bytes(B, Hq, D, max_seq_len, chunk_tokens)
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=dev)
    _need(workspace, "workspace", torch.uint8, dev)
    name = "kvq_attend_decode_float_q" if float_q else "kvq_attend_decode"
    st = getattr(load(), name)(cache.desc, _ptr(q), _ptr(out), B, Hq, float(alpha), _ptr(block_table),
                               block_table.shape[1], _ptr(seq_len), int(max_seq_len), int(chunk_tokens),
                               _ptr(workspace), workspace.numel(), _stream(dev))
    check(name, st)
    return out


def decode_split(cache, batch, num_q_heads, max_seq_len, chunk_tokens=512):
    """kvq_decode_split: (tokens per wave run, tokens per block partial) the decode executes."""
    w, p = ctypes.c_int32(0), ctypes.c_int32(0)
    st = load().kvq_decode_split(cache.desc, int(batch), int(num_q_heads), int(max_seq_len), int(chunk_tokens),
                                 ctypes.byref(w), ctypes.byref(p))
    check("kvq_decode_split", st)
    return w.value, p.value


def decode_split_lengths(cache, num_q_heads, seq_lens, max_seq_len, chunk_tokens=512):
    """kvq_decode_split_lengths: the split the decode executes for rows of these lengths (host ints)."""
    import numpy as np
    lens = np.ascontiguousarray(np.asarray(seq_lens, dtype=np.int32))
    w, p = ctypes.c_int32(0), ctypes.c_int32(0)
    st = load().kvq_decode_split_lengths(cache.desc, int(lens.size), int(num_q_heads), lens.ctypes.data,
                                         int(max_seq_len), int(chunk_tokens), ctypes.byref(w), ctypes.byref(p))
    check("kvq_decode_split_lengths", st)
    return w.value, p.value


def attend_decode_noalloc(cache, q, block_table, seq_len, max_seq_len, alpha, chunk_tokens=512, out=None):
    """kvq_attend_decode_noalloc: attend_decode with the partials in the library's device scratch
    (no workspace; calls that overlap on one device race)."""
    dev = cache.device
    _need(q, "q", torch.float32, dev)
    _need(block_table, "block_table", torch.int32, dev)
    _need(seq_len, "seq_len", torch.int32, dev)
    B, Hq, D = q.shape
    if block_table.dim() != 2 or block_table.shape[0] != B or seq_len.shape != (B,):
        raise ValueError("block_table must be [B, max_pages] and seq_len [B]")
    if out is None:
        out = torch.empty_like(q)
    _need(out, "out", torch.float32, dev)
    st = load().kvq_attend_decode_noalloc(cache.desc, _ptr(q), _ptr(out), B, Hq, float(alpha), _ptr(block_table),
                                          block_table.shape[1], _ptr(seq_len), int(max_seq_len), int(chunk_tokens),
                                          _stream(dev))
    check("kvq_attend_decode_noalloc", st)
    return out


def attend_decode_partial(cache, q, block_table, seq_len, max_seq_len, alpha, chunk_tokens, workspace):
    """kvq_attend_decode_partial: the split-K phase; partials go to ``workspace``."""
    dev = cache.device
    B, Hq, _ = q.shape
    st = load().kvq_attend_decode_partial(cache.desc, _ptr(q), B, Hq, float(alpha), _ptr(block_table),
                                          block_table.shape[1], _ptr(seq_len), int(max_seq_len), int(chunk_tokens),
                                          _ptr(workspace), workspace.numel(), _stream(dev))
    check("kvq_attend_decode_partial", st)


def attend_decode_reduce(cache, out, seq_len, max_seq_len, chunk_tokens, workspace):
    """kvq_attend_decode_reduce: merge the partials in ``workspace`` into ``out`` [B, Hq, D]."""
    dev = cache.device
    B, Hq, _ = out.shape
    st = load().kvq_attend_decode_reduce(cache.desc, _ptr(out), B, Hq, _ptr(seq_len), int(max_seq_len),
                                         int(chunk_tokens), _ptr(workspace), workspace.numel(), _stream(dev))
    check("kvq_attend_decode_reduce", st)


def prefill_workspace_bytes(batch, n_q, num_q_heads, head_dim, max_seq_len):
    return load().kvq_prefill_workspace_bytes(batch, n_q, num_q_heads, head_dim, max_seq_len)


def attend_prefill_causal(cache, q, q_start, block_table, seq_len, max_seq_len, alpha, causal=True,
                          causal_skip=True, out=None, workspace=None):
    """kvq_attend_prefill_causal: q f32 [B, Sq, Hq, D] -> out f32 [B, Sq, Hq, D].

    q_start int32 [B]: position of each row's first query (may be None when not causal).
    causal_skip=False sets KVQ_PREFILL_NO_CAUSAL_SKIP (same result, masked tiles streamed).
    """
    dev = cache.device
    _need(q, "q", torch.float32, dev)
    if q_start is not None or causal:
        _need(q_start, "q_start", torch.int32, dev)
    _need(block_table, "block_table", torch.int32, dev)
    _need(seq_len, "seq_len", torch.int32, dev)
    if q.dim() != 4:
        raise ValueError("q must be [B, Sq, Hq, D]")
    B, Sq, Hq, D = q.shape
    if block_table.dim() != 2 or block_table.shape[0] != B or seq_len.shape != (B,):
        raise ValueError("block_table must be [B, max_pages] and seq_len [B]")
    if q_start is not None and q_start.shape != (B,):
        raise ValueError("q_start must be [B]")
    if out is None:
        out = torch.empty_like(q)
    _need(out, "out", torch.float32, dev)
    need = prefill_workspace_bytes(B, Sq, Hq, D, max_seq_len)
    if workspace is None and need > 0:
        workspace = torch.empty(need, dtype=torch.uint8, device=dev)
    flags = 0 if causal_skip else _lib.PREFILL_NO_CAUSAL_SKIP
    st = load().kvq_attend_prefill_causal(cache.desc, _ptr(q), _ptr(out), B, Sq, Hq, float(alpha), int(bool(causal)),
                                          _ptr(q_start), _ptr(block_table), block_table.shape[1], _ptr(seq_len),
                                          int(max_seq_len), flags, _ptr(workspace),
                                          workspace.numel() if workspace is not None else 0, _stream(dev))
    check("kvq_attend_prefill_causal", st)
    return out


def _chunk_rows(cache, k_new, v_new, B, n_q):
    dev = cache.device
    _need(k_new, "k_new", torch.float32, dev)
    _need(v_new, "v_new", torch.float32, dev)
    if k_new.shape != (B, n_q, cache.num_kv_heads, cache.head_dim) or v_new.shape != k_new.shape:
        raise ValueError("k_new and v_new must be [B, n_q, Hkv, D]")


def store_chunk(cache, k_new, v_new, q_start, block_table, max_seq_len):
    """kvq_store_chunk: append k_new, v_new f32 [B, n_q, Hkv, D] at positions q_start[b] + i."""
    dev = cache.device
    _need(q_start, "q_start", torch.int32, dev)
    _need(block_table, "block_table", torch.int32, dev)
    B, n_q = k_new.shape[0], k_new.shape[1]
    _chunk_rows(cache, k_new, v_new, B, n_q)
    if q_start.shape != (B,) or block_table.dim() != 2 or block_table.shape[0] != B:
        raise ValueError("q_start must be [B] and block_table [B, max_pages]")
    st = load().kvq_store_chunk(cache.desc, _ptr(k_new), _ptr(v_new), B, n_q, _ptr(q_start), _ptr(block_table),
                                block_table.shape[1], int(max_seq_len), _stream(dev))
    check("kvq_store_chunk", st)


def prefill_full_then_store(cache, q, k_new, v_new, q_start, block_table, max_seq_len, alpha, causal=True,
                            out=None, workspace=None):
    """kvq_prefill_full_then_store: the chunk's queries q f32 [B, n_q, Hq, D] attend over the cached
    prefix and over the chunk's own rows k_new, v_new f32 [B, n_q, Hkv, D] in full precision; then the
    chunk is stored at positions q_start[b] + i.  Returns out f32 [B, n_q, Hq, D]."""
    dev = cache.device
    _need(q, "q", torch.float32, dev)
    _need(q_start, "q_start", torch.int32, dev)
    _need(block_table, "block_table", torch.int32, dev)
    if q.dim() != 4:
        raise ValueError("q must be [B, n_q, Hq, D]")
    B, n_q, Hq, D = q.shape
    _chunk_rows(cache, k_new, v_new, B, n_q)
    if q_start.shape != (B,) or block_table.dim() != 2 or block_table.shape[0] != B:
        raise ValueError("q_start must be [B] and block_table [B, max_pages]")
    if out is None:
        out = torch.empty_like(q)
    _need(out, "out", torch.float32, dev)
    need = prefill_workspace_bytes(B, n_q, Hq, D, max_seq_len)
    if workspace is None and need > 0:
        workspace = torch.empty(need, dtype=torch.uint8, device=dev)
    st = load().kvq_prefill_full_then_store(cache.desc, _ptr(q), _ptr(k_new), _ptr(v_new), _ptr(out), B, n_q, Hq,
                                            float(alpha), int(bool(causal)), _ptr(q_start), _ptr(block_table),
                                            block_table.shape[1], int(max_seq_len), _ptr(workspace),
                                            workspace.numel() if workspace is not None else 0, _stream(dev))
    check("kvq_prefill_full_then_store", st)
    return out


def attend_step(cache, q, k_new, v_new, q_start, seq_len, block_table, max_seq_len, alpha, cached_tokens,
                chunk_tokens=512):
    """One attention step of a model layer with the dispatch rule of [Open-TQ-Metal]'s prefill/decode
    selection: a single query with at least 32 cached tokens appends its token (kvq_store_chunk) and
    runs the fused decode over the packed cache; any other step (several queries, or fewer than 32
    cached tokens) runs the full-precision prefill and then stores the chunk.

    q f32 [B, n_q, Hq, D]; k_new, v_new f32 [B, n_q, Hkv, D]; q_start int32 [B] (cached tokens before
    the step); seq_len int32 [B] = q_start + n_q; cached_tokens: host int, the fewest cached tokens of
    any row.  Returns (out f32 [B, n_q, Hq, D], "decode" or "full").
    """
    B, n_q = q.shape[0], q.shape[1]
    if n_q == 1 and cached_tokens >= 32:
        store_chunk(cache, k_new, v_new, q_start, block_table, max_seq_len)
        out = attend_decode(cache, q[:, 0], block_table, seq_len, max_seq_len, alpha, chunk_tokens=chunk_tokens)
        return out[:, None], "decode"
    return prefill_full_then_store(cache, q, k_new, v_new, q_start, block_table, max_seq_len, alpha), "full"


def debug_quantize_q(layout, q):
    """kvq_debug_quantize_q: q f32 [n, D] -> (q8 int8 [n, D], sq f32 [n])."""
    n, D = q.shape
    lay = _lib.LAYOUT_IDS[layout] if isinstance(layout, str) else int(layout)
    q8 = torch.empty((n, D), dtype=torch.int8, device=q.device)
    sq = torch.empty((n,), dtype=torch.float32, device=q.device)
    _need(q, "q", torch.float32, q.device)
    st = load().kvq_debug_quantize_q(lay, _ptr(q), n, D, _ptr(q8), _ptr(sq), _stream(q.device))
    check("kvq_debug_quantize_q", st)
    return q8, sq


def debug_stream_read(bufs):
    """kvq_debug_stream_read: read every byte of up to four contiguous device tensors once, in one
    launch (the read probe)."""
    bufs = list(bufs)
    if not 1 <= len(bufs) <= 4 or any(not b.is_cuda or not b.is_contiguous() for b in bufs):
        raise ValueError("one to four contiguous device tensors")
    src = (ctypes.c_void_p * len(bufs))(*[b.data_ptr() for b in bufs])
    nbytes = (ctypes.c_size_t * len(bufs))(*[b.numel() * b.element_size() for b in bufs])
    st = load().kvq_debug_stream_read(len(bufs), ctypes.cast(src, ctypes.c_void_p), ctypes.cast(nbytes, ctypes.c_void_p),
                                      _stream(bufs[0].device))
    check("kvq_debug_stream_read", st)


def debug_qk_i32(cache, q, block_table, seq_len, max_seq_len):
    """kvq_debug_qk_i32: the decode kernel's per-block i32 scores [B, Hq, max_seq_len, n_groups]."""
    dev = cache.device
    _need(q, "q", torch.float32, dev)
    B, Hq, D = q.shape
    ng = 1 if cache.layout == _lib.HAD_INT4 else D // 32
    scores = torch.zeros((B, Hq, max_seq_len, ng), dtype=torch.int32, device=dev)
    ws = torch.empty(max(decode_workspace_bytes(B, Hq, D, max_seq_len, 512), 1), dtype=torch.uint8, device=dev)
    st = load().kvq_debug_qk_i32(cache.desc, _ptr(q), B, Hq, _ptr(block_table), block_table.shape[1],
                                 _ptr(seq_len), int(max_seq_len), _ptr(scores), _ptr(ws), ws.numel(), _stream(dev))
    check("kvq_debug_qk_i32", st)
    return scores
