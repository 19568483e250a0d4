"""The C ABI on the host: the library loads, exports every declared symbol, and
validates arguments before touching the GPU (no compute call runs here)."""

import ctypes
import os
import re

import pytest

import quantized_kv_cache_store_amd as kvq
from quantized_kv_cache_store_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared():
    src = open(os.path.join(ROOT, "include", "kvq.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(kvq_[a-z0-9_]+)\s*\(", src)))


def test_library_exports_every_declared_symbol():
    lib = kvq.load()
    names = _declared()
    assert "kvq_store" in names and "kvq_attend_decode" in names and "kvq_attend_prefill_causal" in names
    for n in names:
        assert hasattr(lib, n), n
    assert set(names) == set(_lib.SIGNATURES)


def test_sizes():
    lib = kvq.load()
    assert lib.kvq_payload_bytes(_lib.Q4_0, 128) == 64
    assert lib.kvq_scale_bytes(_lib.Q4_0, 128) == 8
    assert lib.kvq_payload_bytes(_lib.Q6_0, 256) == 192
    assert lib.kvq_scale_bytes(_lib.Q6_0, 256) == 16
    assert lib.kvq_payload_bytes(_lib.ASYM_INT4_G32, 128) == 64
    assert lib.kvq_scale_bytes(_lib.ASYM_INT4_G32, 128) == 16
    assert lib.kvq_scale_bytes(_lib.HAD_INT4, 128) == 4
    assert lib.kvq_payload_bytes(_lib.Q8_0, 128) == 128
    assert lib.kvq_scale_bytes(_lib.Q8_0, 256) == 16
    assert lib.kvq_payload_bytes(_lib.Q4_0, 64) == 0          # unsupported head_dim
    assert lib.kvq_payload_bytes(7, 128) == 0
    # room for the partials [B][Hq][chunks + 1][D + 4] f32
    assert lib.kvq_decode_workspace_bytes(1, 64, 128, 131072, 512) == 64 * 257 * 132 * 4
    assert lib.kvq_decode_workspace_bytes(1, 64, 128, 1000, 100) == 0  # chunk not a multiple of 128


def _desc(**kw):
    d = dict(layout=1, head_dim=128, num_kv_heads=1, page_size=16, num_pages=4, n_recent=0, max_batch=1,
             reserved=0, k_payload=16, v_payload=16, k_scale=16, v_scale=16, k_recent=None, v_recent=None)
    d.update(kw)
    return _lib.KvqCacheDesc(**d)


@pytest.mark.parametrize("kw,status", [
    (dict(layout=9), 1), (dict(head_dim=96), 2), (dict(page_size=24), 1), (dict(page_size=8), 1),
    (dict(num_kv_heads=0), 1), (dict(k_payload=None), 1), (dict(n_recent=4), 1), (dict(reserved=3), 1),
    (dict(num_pages=1 << 27, page_size=16), 1), (dict(num_pages=1 << 20, page_size=4096), 1),
])
def test_store_validates_cache(kw, status):
    lib = kvq.load()
    st = lib.kvq_store(ctypes.byref(_desc(**kw)), 16, 16, 1, 16, 16, 16, 16, None)
    assert st == status
    assert lib.kvq_last_error()


def test_attend_validates_before_launch():
    lib = kvq.load()
    d = ctypes.byref(_desc())
    d2 = ctypes.byref(_desc(num_kv_heads=2))
    assert lib.kvq_attend_decode(d2, 16, 16, 1, 3, 1.0, 16, 4, 16, 64, 512, 16, 1 << 20, None) == 1  # Hq % Hkv
    assert lib.kvq_attend_decode(d, 16, 16, 1, 4, 1.0, 16, 4, 16, 64, 100, 16, 1 << 20, None) == 1  # chunk
    assert lib.kvq_attend_decode(d, 16, 16, 1, 4, 1.0, 16, 4, 16, 64, 512, 16, 10, None) == 3       # workspace
    assert lib.kvq_attend_decode(d, 16, 16, 1, 4, 1.0, 16, 2, 16, 64, 512, 16, 1 << 20, None) == 1  # pages
    assert lib.kvq_attend_decode(d, None, 16, 1, 4, 1.0, 16, 4, 16, 64, 512, 16, 1 << 20, None) == 1
    assert lib.kvq_debug_quantize_q(1, 16, 3, 64, 16, 16, None) == 2
    assert lib.kvq_store(d, 16, 16, -1, 16, None, None, None, None) == 1
    assert lib.kvq_store(d, 16, 16, 0, 16, None, None, None, None) == 0   # empty append is a no-op
    assert kvq.load().kvq_status_string(3) == b"workspace too small"


def test_prefill_validates_before_launch():
    lib = kvq.load()
    d = ctypes.byref(_desc())
    # narrow partial records [B][n_q][Hq][slots][D / 2 + 4] floats (D f16 numerators, m, l, exponent),
    # then the prepared rows:
    # rotated f32 query, int8 query, f32 scale, int32 block sums
    rows = 512 * 16
    # partials (17 chunks of the shortest split, 512 tokens, + 8 slices of 128 f32 rows: a 512-token
    # window and the 512-token chunk) | f32 query | int8 query | scale | block sums | chunk K and V rows
    assert lib.kvq_prefill_workspace_bytes(1, 512, 16, 128, 8704) == rows * (25 * 68 * 4 + 128 * 4 + 128 + 4 + 4 * 4
                                                                             + 2 * 128 * 4)
    assert lib.kvq_prefill_workspace_bytes(1, 0, 16, 128, 8704) == 0
    big = 1 << 30
    pf = lib.kvq_attend_prefill_causal
    assert pf(d, 16, 16, 1, 0, 1, 1.0, 1, 16, 16, 4, 16, 64, 0, 16, big, None) == 1      # n_q < 1
    assert pf(d, 16, 16, 1, 4, 1, 1.0, 1, None, 16, 4, 16, 64, 0, 16, big, None) == 1    # causal without q_start
    assert pf(d, 16, 16, 1, 4, 1, 1.0, 2, 16, 16, 4, 16, 64, 0, 16, big, None) == 1      # causal not 0/1
    assert pf(d, 16, 16, 1, 4, 1, 1.0, 1, 16, 16, 4, 16, 64, 4, 16, big, None) == 1      # unknown flag
    assert pf(d, 16, None, 1, 4, 1, 1.0, 1, 16, 16, 4, 16, 64, 0, 16, big, None) == 1    # out
    assert pf(d, 16, 16, 1, 4, 1, 1.0, 1, 16, 16, 4, 16, 64, 0, 16, 100, None) == 3      # workspace
    assert b"workspace" in lib.kvq_last_error()


def test_missing_library_fails_loudly(monkeypatch, tmp_path):
    monkeypatch.setattr(_lib, "_lib", None)
    monkeypatch.setattr(_lib, "LIB_PATH", str(tmp_path / "libkvq.so"))
    with pytest.raises(RuntimeError, match="not built"):
        _lib.load()


def test_noalloc_decode_refuses_oversized_calls_on_the_host():
    """kvq_attend_decode_noalloc checks its partials against the fixed scratch before any launch."""
    lib = kvq.load()
    d = ctypes.byref(_desc(layout=_lib.Q4_0, head_dim=128, num_kv_heads=1, page_size=16, num_pages=4))
    # 64 rows x 64 query heads at 2^20 tokens: far above KVQ_DECODE_NOALLOC_SCRATCH_BYTES (32 MiB)
    st = lib.kvq_attend_decode_noalloc(d, 16, 16, 64, 64, 1.0, 16, 1 << 16, 16, 1 << 20, 512, None)
    assert st == 3
    assert b"scratch" in lib.kvq_last_error()
    assert lib.kvq_attend_decode_noalloc(d, 16, None, 1, 4, 1.0, 16, 4, 16, 64, 512, None) == 1   # out


def test_decode_split_reports_the_executed_runs():
    """kvq_decode_split: runs are whole chunks (or halves/quarters), partials four runs; bad args refused."""
    lib = kvq.load()
    d = ctypes.byref(_desc(layout=_lib.ASYM_INT4_G32, head_dim=128, num_kv_heads=8, page_size=1024, num_pages=4))
    w, p = ctypes.c_int32(0), ctypes.c_int32(0)
    assert lib.kvq_decode_split(d, 8, 64, 131072, 512, ctypes.byref(w), ctypes.byref(p)) == 0
    assert w.value in (128, 256, 512, 1024, 2048) and p.value == 4 * w.value
    assert lib.kvq_decode_split(d, 8, 63, 131072, 512, ctypes.byref(w), ctypes.byref(p)) == 1
    assert lib.kvq_decode_split(d, 8, 64, 131072, 100, ctypes.byref(w), ctypes.byref(p)) == 1
    assert lib.kvq_decode_split(d, 8, 64, 131072, 512, None, ctypes.byref(p)) == 1


def _split_lengths(lib, d, Hq, lens, max_seq_len=None, chunk=512):
    import numpy as np
    lens = np.ascontiguousarray(np.asarray(lens, dtype=np.int32))
    w, p = ctypes.c_int32(0), ctypes.c_int32(0)
    mx = int(lens.max()) if max_seq_len is None else max_seq_len
    st = lib.kvq_decode_split_lengths(d, int(lens.size), Hq, lens.ctypes.data, mx, chunk, ctypes.byref(w),
                                      ctypes.byref(p))
    return st, w.value, p.value


def test_decode_split_lengths_follows_the_rows():
    """Several rounds of blocks: the run length follows the rows' lengths (a ragged batch takes shorter
    runs that fill its last round, a uniform one its longest); one round or one row: the fixed split."""
    import workloads as W
    lib = kvq.load()
    g = W.WORKLOADS["gemma_q6_0_ragged_b16"]
    lens = [int(n) for n in W.seq_lens(g)]
    q6 = ctypes.byref(_desc(layout=_lib.Q6_0, head_dim=256, num_kv_heads=8, page_size=16, num_pages=4))
    assert _split_lengths(lib, q6, 16, lens) == (0, 768, 3072)
    assert _split_lengths(lib, q6, 16, [max(lens)] * 16) == (0, 2048, 8192)
    w, p = ctypes.c_int32(0), ctypes.c_int32(0)
    assert lib.kvq_decode_split(q6, 16, 16, max(lens), 512, ctypes.byref(w), ctypes.byref(p)) == 0
    assert (w.value, p.value) == (2048, 8192)      # rows of max_seq_len
    asym = ctypes.byref(_desc(layout=_lib.ASYM_INT4_G32, head_dim=128, num_kv_heads=8, page_size=1024, num_pages=4))
    assert _split_lengths(lib, asym, 64, [131072] * 8) == (0, 2048, 8192)    # one round
    assert _split_lengths(lib, asym, 64, [131072] * 16) == (0, 2048, 8192)   # two full rounds
    assert _split_lengths(lib, asym, 64, [131072]) == (0, 512, 2048)         # one row
    assert _split_lengths(lib, asym, 64, [131072, 200], max_seq_len=100)[0] == 1   # a row past max_seq_len
    assert lib.kvq_decode_split_lengths(asym, 1, 64, None, 10, 512, ctypes.byref(w), ctypes.byref(p)) == 1
