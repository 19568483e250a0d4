"""GPU parity of the full-precision prefill followed by quantise-on-store, and of the step dispatch.

Outputs: max|diff| <= 2e-3 * max|o_ref| against ``oracle.attention.attend_prefill_full`` (the chunk's
own tokens exact, the prefix as cached).  The chunk's stored payload, records and window rows are
bit-exact against the oracle's encoding, as for ``kvq_store``.
"""

import math

import numpy as np
import pytest
import torch

import quantized_kv_cache_store_amd as kvq
from oracle import attention, quant, spec
import gpu_util as U

pytestmark = pytest.mark.gpu

ALL = [spec.HAD_INT4, spec.Q4_0, spec.Q6_0, spec.ASYM_G32, spec.Q8_0]


def _setup(layout, D, Hkv, G, prefix, n_q, n_recent, seed, page_size=16):
    """Rows of prefix + n_q tokens per batch row; the prefixes stored through kvq_store."""
    rng = np.random.default_rng(seed)
    B, Hq = len(prefix), Hkv * G
    total = [p + n_q for p in prefix]
    rows_k = [rng.standard_normal((n, Hkv, D)).astype(np.float32) for n in total]
    rows_v = [rng.standard_normal((n, Hkv, D)).astype(np.float32) for n in total]
    q = rng.standard_normal((B, n_q, Hq, D)).astype(np.float32)
    table, npages = U.make_tables(total, page_size, shuffle_seed=seed + 1)
    cache = kvq.KvqCache(layout, D, Hkv, npages, page_size, n_recent=n_recent, max_batch=B, device=U.DEV)
    seq_pre = torch.tensor(prefix, dtype=torch.int32, device=U.DEV)
    for b, p in enumerate(prefix):
        if p == 0:
            continue
        kn = torch.from_numpy(np.ascontiguousarray(rows_k[b][:p])).to(U.DEV)
        vn = torch.from_numpy(np.ascontiguousarray(rows_v[b][:p])).to(U.DEV)
        sl = torch.from_numpy(U.slots_for(table, b, 0, p, page_size)).to(U.DEV)
        bi = torch.full((p,), b, dtype=torch.int32, device=U.DEV)
        ps = torch.arange(0, p, dtype=torch.int32, device=U.DEV)
        kvq.store(cache, kn, vn, sl, bi, ps, seq_pre)
    torch.cuda.synchronize()
    kc = torch.from_numpy(np.stack([r[p:] for r, p in zip(rows_k, prefix)])).to(U.DEV)
    vc = torch.from_numpy(np.stack([r[p:] for r, p in zip(rows_v, prefix)])).to(U.DEV)
    return dict(cache=cache, table=table, bt=torch.from_numpy(table).to(U.DEV), qs=seq_pre, q=q,
                qt=torch.from_numpy(q).to(U.DEV), kc=kc, vc=vc, rows_k=rows_k, rows_v=rows_v, total=total,
                prefix=prefix, n_recent=n_recent, layout=layout, alpha=1.0 / math.sqrt(D))


def _check_stored(c):
    """Every token of every row (prefix and chunk) as the oracle encodes it; the window ring holds
    the last n_recent positions of each row after the append."""
    cache, layout, nr = c["cache"], c["layout"], c["n_recent"]
    for b, n in enumerate(c["total"]):
        for h in range(cache.num_kv_heads):
            for which, rows in (("k", c["rows_k"][b]), ("v", c["rows_v"][b])):
                e = quant.encode_rows(layout, rows[:, h, :])
                pay, rec = U.row_bytes(cache, which, c["table"], b, 0, n, h)
                np.testing.assert_array_equal(pay, e["payload"], err_msg=f"payload b{b} h{h} {which}")
                np.testing.assert_array_equal(rec, e["record"], err_msg=f"record b{b} h{h} {which}")
                if nr:
                    ring = (cache.k_recent if which == "k" else cache.v_recent)[b, h].cpu().numpy()
                    f32rows = e["rotated"] if layout == spec.HAD_INT4 else rows[:, h, :].astype(np.float64)
                    for p in range(max(0, n - nr), n):
                        np.testing.assert_array_equal(ring[p % nr], f32rows[p].astype(np.float32),
                                                      err_msg=f"ring b{b} h{h} {which} pos {p}")


@pytest.mark.parametrize("layout", ALL)
@pytest.mark.parametrize("D", [128, 256])
@pytest.mark.parametrize("prefix,n_q,n_recent", [([300, 0], 40, 0), ([1100, 77], 33, 16), ([5], 70, 64), ([0, 0], 50, 16)])
def test_prefill_full_then_store_matches_oracle(layout, D, prefix, n_q, n_recent):
    """Ragged prefixes (one empty: a fresh prompt; all empty: the launch without packed chunks),
    windows shorter and longer than the prefix, a chunk that is not a multiple of the 16-row tile;
    then the stored chunk, bit for bit."""
    U.need_gpu()
    c = _setup(layout, D, 2, 2, prefix, n_q, n_recent, seed=31 * layout + D + n_q)
    out = kvq.prefill_full_then_store(c["cache"], c["qt"], c["kc"], c["vc"], c["qs"], c["bt"], max(c["total"]),
                                      c["alpha"])
    torch.cuda.synchronize()
    ref = np.stack([attention.attend_prefill_full(layout, c["q"][b], c["rows_k"][b], c["rows_v"][b], c["alpha"],
                                                  prefix[b], n_recent=n_recent) for b in range(len(prefix))])
    U.assert_close_rel(out.cpu().numpy(), ref)
    _check_stored(c)


@pytest.mark.parametrize("layout", ALL)
@pytest.mark.parametrize("prefix,n_q,n_recent,causal", [([200, 30], 300, 64, True), ([0], 333, 0, True),
                                                        ([90, 500], 260, 128, False)])
def test_prefill_full_several_row_slices(layout, prefix, n_q, n_recent, causal):
    """More f32 rows (window + chunk) than one slice of 128: several slice groups and partial slots,
    rows of different windows in one batch, the causal reach per query in the reduce."""
    U.need_gpu()
    c = _setup(layout, 128, 2, 2, prefix, n_q, n_recent, seed=13 * layout + n_q)
    out = kvq.prefill_full_then_store(c["cache"], c["qt"], c["kc"], c["vc"], c["qs"], c["bt"], max(c["total"]),
                                      c["alpha"], causal=causal)
    torch.cuda.synchronize()
    ref = np.stack([attention.attend_prefill_full(layout, c["q"][b], c["rows_k"][b], c["rows_v"][b], c["alpha"],
                                                  prefix[b], causal=causal, n_recent=n_recent)
                    for b in range(len(prefix))])
    U.assert_close_rel(out.cpu().numpy(), ref)
    _check_stored(c)


@pytest.mark.parametrize("layout", [spec.HAD_INT4, spec.ASYM_G32])
@pytest.mark.parametrize("G", [1, 8])
def test_prefill_full_not_causal_and_gqa(layout, G):
    U.need_gpu()
    c = _setup(layout, 128, 2, G, [600, 64], 20, 8, seed=5 + G + layout)
    out = kvq.prefill_full_then_store(c["cache"], c["qt"], c["kc"], c["vc"], c["qs"], c["bt"], max(c["total"]),
                                      c["alpha"], causal=False)
    torch.cuda.synchronize()
    ref = np.stack([attention.attend_prefill_full(layout, c["q"][b], c["rows_k"][b], c["rows_v"][b], c["alpha"],
                                                  c["prefix"][b], causal=False, n_recent=8) for b in range(2)])
    U.assert_close_rel(out.cpu().numpy(), ref)


@pytest.mark.parametrize("layout", [spec.Q4_0, spec.HAD_INT4])
@pytest.mark.parametrize("cached", [20, 31, 32, 700])
def test_step_dispatch_rule(layout, cached):
    """One query: the fused decode over the packed cache from 32 cached tokens on, else the
    full-precision path (the new token exact); either way the token ends up stored."""
    U.need_gpu()
    c = _setup(layout, 128, 2, 4, [cached], 1, 0, seed=cached + layout)
    seq = c["qs"] + 1
    out, path = kvq.attend_step(c["cache"], c["qt"], c["kc"], c["vc"], c["qs"], seq, c["bt"], cached + 1, c["alpha"],
                                cached_tokens=cached)
    torch.cuda.synchronize()
    assert path == ("decode" if cached >= 32 else "full")
    if path == "decode":
        ref = attention.attend_decode(layout, c["q"][0, 0], c["rows_k"][0], c["rows_v"][0], c["alpha"])[None]
    else:
        ref = attention.attend_prefill_full(layout, c["q"][0], c["rows_k"][0], c["rows_v"][0], c["alpha"], cached)
    U.assert_close_rel(out.cpu().numpy()[0], ref)
    _check_stored(c)


def test_prefill_full_validation():
    U.need_gpu()
    c = _setup(spec.Q4_0, 128, 1, 1, [10], 4, 0, seed=1)
    with pytest.raises(kvq.KvqError, match="invalid argument"):
        kvq.prefill_full_then_store(c["cache"], c["qt"], c["kc"], c["vc"], c["qs"], c["bt"], 3, c["alpha"])
    with pytest.raises(ValueError):
        kvq.prefill_full_then_store(c["cache"], c["qt"], c["kc"][:, :2], c["vc"], c["qs"], c["bt"], 14, c["alpha"])
