"""Helpers for the GPU parity tests: fill a device cache from numpy rows and read its planes back.

Inputs come from ``workloads`` (seeded) or from the tests themselves; expected
values come only from ``oracle``.  The device side is driven through the
binding, i.e. through the C ABI of libkvq.so.
"""

import numpy as np
import torch

import quantized_kv_cache_store_amd as kvq

LAYOUT_NAMES = {0: "had_int4", 1: "q4_0", 2: "q6_0", 3: "asym_int4_g32", 4: "q8_0"}
DEV = torch.device("cuda:0")


def need_gpu():
    import pytest
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    kvq.load()


def make_tables(lens, page_size, shuffle_seed=None, pages_per_row=None):
    """Block tables for rows of the given lengths; physical pages optionally shuffled."""
    need = [max(1, (int(n) + page_size - 1) // page_size) for n in lens]
    ppr = pages_per_row or max(need)
    total = int(sum(need))
    phys = np.arange(total)
    if shuffle_seed is not None:
        phys = np.random.default_rng(shuffle_seed).permutation(total)
    table = np.zeros((len(lens), ppr), dtype=np.int32)
    k = 0
    for b, n in enumerate(need):
        table[b, :n] = phys[k:k + n]
        table[b, n:] = phys[k]          # unused entries point at a page of the row
        k += n
    return table, total


def slots_for(table, b, t0, t1, page_size):
    t = np.arange(t0, t1)
    return (table[b, t // page_size].astype(np.int64) * page_size + t % page_size).astype(np.int32)


def build_cache(layout, D, Hkv, rows_k, rows_v, page_size=16, n_recent=0, shuffle_seed=7, chunk=8192):
    """Store every row's tokens through kvq_store.  rows_k[b]: f32 [S_b, Hkv, D]."""
    lens = [r.shape[0] for r in rows_k]
    B = len(lens)
    table, total = make_tables(lens, page_size, shuffle_seed)
    cache = kvq.KvqCache(layout, D, Hkv, total, page_size, n_recent=n_recent, max_batch=B, device=DEV)
    seq = torch.tensor(lens, dtype=torch.int32, device=DEV)
    for b in range(B):
        for t0 in range(0, lens[b], chunk):
            t1 = min(lens[b], t0 + chunk)
            kn = torch.from_numpy(np.ascontiguousarray(rows_k[b][t0:t1])).to(DEV)
            vn = torch.from_numpy(np.ascontiguousarray(rows_v[b][t0:t1])).to(DEV)
            sl = torch.from_numpy(slots_for(table, b, t0, t1, page_size)).to(DEV)
            bi = torch.full((t1 - t0,), b, dtype=torch.int32, device=DEV)
            ps = torch.arange(t0, t1, dtype=torch.int32, device=DEV)
            kvq.store(cache, kn, vn, sl, bi, ps, seq)
    torch.cuda.synchronize()
    return cache, torch.from_numpy(table).to(DEV), seq, table


def row_bytes(cache, which, table, b, t0, t1, h):
    """Stored payload and record bytes of tokens [t0, t1) of row b, kv head h (numpy uint8)."""
    ps = cache.page_size
    t = np.arange(t0, t1)
    page = torch.from_numpy(table[b, t // ps].astype(np.int64)).to(DEV)
    off = torch.from_numpy((t % ps).astype(np.int64)).to(DEV)
    pay = (cache.k_payload if which == "k" else cache.v_payload)[page, h, off]
    rec = (cache.k_scale if which == "k" else cache.v_scale)[page, h, off]
    return pay.cpu().numpy(), rec.cpu().numpy()


def assert_close_rel(got, ref, rel=2e-3, what="output"):
    """max |got - ref| <= rel * max |ref| over the whole case."""
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert np.all(np.isfinite(got)), f"{what}: non-finite values"
    err = np.abs(got - ref).max() if ref.size else 0.0
    scale = np.abs(ref).max() if ref.size else 0.0
    assert err <= rel * scale, f"{what}: max|diff| {err:.3e} > {rel} * max|ref| {scale:.3e} (ratio {err / max(scale, 1e-300):.2e})"
    return err / max(scale, 1e-300)
