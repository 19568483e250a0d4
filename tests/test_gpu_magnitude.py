"""GPU parity at input magnitudes far from unit scale, for every layout and attention path.

K and V together, and separately Q, are scaled by 1e-5, 1e-3, 1e3 and 1e5 before the store; the
outputs must stay within 2e-3 * max|o_ref| of the oracle (float64, the same stored codes) on the
decode, the float-query decode, the causal prefill and the full-precision prefill.  The Hadamard
layout keeps one f32 scale per token ([tract-RFC] Architecture > Data flow (decode)), so its V side
must hold at every one of these magnitudes.  The fp16-scale layouts form each dequantised V element
in fp16 for the P V product, so their V rows are kept inside the fp16 range: at the top magnitude
their K is scaled by 1e5 and their V by 1e4.
"""

import math

import numpy as np
import pytest
import torch

import quantized_kv_cache_store_amd as kvq
from oracle import attention, spec
import gpu_util as U

pytestmark = pytest.mark.gpu

ALL = [spec.HAD_INT4, spec.Q4_0, spec.Q6_0, spec.ASYM_G32, spec.Q8_0]
SWEEP = [("kv", 1e-5), ("kv", 1e-3), ("kv", 1e3), ("kv", 1e5), ("q", 1e-5), ("q", 1e-3), ("q", 1e3), ("q", 1e5)]


def _factors(layout, which, mag):
    """(K, V, Q) multipliers of one sweep point."""
    if which == "q":
        return 1.0, 1.0, mag
    v = mag if (layout == spec.HAD_INT4 or mag < 1e5) else 1e4
    return mag, v, 1.0


def _rows(rng, n, Hkv, D, f):
    return (rng.standard_normal((n, Hkv, D)) * f).astype(np.float32)


def _id(p):
    return f"{p[0]}{p[1]:g}"


@pytest.mark.parametrize("layout", ALL)
@pytest.mark.parametrize("point", SWEEP, ids=_id)
@pytest.mark.parametrize("float_q", [False, True], ids=["int8q", "floatq"])
def test_decode_magnitudes(layout, point, float_q):
    U.need_gpu()
    fk, fv, fq = _factors(layout, *point)
    D, Hkv, G, n_recent, lens = 128, 2, 4, 16, [700, 129, 5]
    rng = np.random.default_rng(101 + layout)
    rows_k = [_rows(rng, n, Hkv, D, fk) for n in lens]
    rows_v = [_rows(rng, n, Hkv, D, fv) for n in lens]
    q = (rng.standard_normal((len(lens), Hkv * G, D)) * fq).astype(np.float32)
    alpha = 1.0 / math.sqrt(D)
    cache, bt, seq, _ = U.build_cache(layout, D, Hkv, rows_k, rows_v, n_recent=n_recent)
    out = kvq.attend_decode(cache, torch.from_numpy(q).to(U.DEV), bt, seq, max(lens), alpha, float_q=float_q)
    torch.cuda.synchronize()
    ref = np.stack([attention.attend_decode(layout, q[b], rows_k[b], rows_v[b], alpha, n_recent=n_recent,
                                            float_q=float_q) for b in range(len(lens))])
    U.assert_close_rel(out.cpu().numpy(), ref, what=f"decode K x{fk:g} V x{fv:g} Q x{fq:g}")


@pytest.mark.parametrize("point", SWEEP, ids=_id)
def test_decode_magnitudes_had_d256_no_window(point):
    """The Hadamard layout at head_dim 256, every token packed (no window rows to lean on)."""
    U.need_gpu()
    layout = spec.HAD_INT4
    fk, fv, fq = _factors(layout, *point)
    D, Hkv, G, lens = 256, 1, 8, [1100, 40]
    rng = np.random.default_rng(7)
    rows_k = [_rows(rng, n, Hkv, D, fk) for n in lens]
    rows_v = [_rows(rng, n, Hkv, D, fv) for n in lens]
    q = (rng.standard_normal((len(lens), Hkv * G, D)) * fq).astype(np.float32)
    alpha = 1.0 / math.sqrt(D)
    cache, bt, seq, _ = U.build_cache(layout, D, Hkv, rows_k, rows_v)
    out = kvq.attend_decode(cache, torch.from_numpy(q).to(U.DEV), bt, seq, max(lens), alpha)
    torch.cuda.synchronize()
    ref = np.stack([attention.attend_decode(layout, q[b], rows_k[b], rows_v[b], alpha) for b in range(len(lens))])
    U.assert_close_rel(out.cpu().numpy(), ref, what=f"decode K x{fk:g} V x{fv:g} Q x{fq:g}")


@pytest.mark.parametrize("layout", ALL)
@pytest.mark.parametrize("point", SWEEP, ids=_id)
def test_prefill_magnitudes(layout, point):
    U.need_gpu()
    fk, fv, fq = _factors(layout, *point)
    D, Hkv, G, n_recent, lens, n_q = 128, 2, 2, 16, [300, 140], 37
    rng = np.random.default_rng(202 + layout)
    rows_k = [_rows(rng, n, Hkv, D, fk) for n in lens]
    rows_v = [_rows(rng, n, Hkv, D, fv) for n in lens]
    q = (rng.standard_normal((len(lens), n_q, Hkv * G, D)) * fq).astype(np.float32)
    q_starts = [n - n_q for n in lens]
    alpha = 1.0 / math.sqrt(D)
    cache, bt, seq, _ = U.build_cache(layout, D, Hkv, rows_k, rows_v, n_recent=n_recent)
    qs = torch.tensor(q_starts, dtype=torch.int32, device=U.DEV)
    out = kvq.attend_prefill_causal(cache, torch.from_numpy(q).to(U.DEV), qs, bt, seq, max(lens), alpha)
    torch.cuda.synchronize()
    ref = np.stack([attention.attend_prefill(layout, q[b], rows_k[b], rows_v[b], alpha, q_starts[b],
                                             n_recent=n_recent) for b in range(len(lens))])
    U.assert_close_rel(out.cpu().numpy(), ref, what=f"prefill K x{fk:g} V x{fv:g} Q x{fq:g}")


@pytest.mark.parametrize("layout", ALL)
@pytest.mark.parametrize("point", SWEEP, ids=_id)
def test_prefill_full_magnitudes(layout, point):
    U.need_gpu()
    fk, fv, fq = _factors(layout, *point)
    D, Hkv, G, n_recent, prefix, n_q = 128, 2, 2, 16, [200, 0], 33
    rng = np.random.default_rng(303 + layout)
    total = [p + n_q for p in prefix]
    rows_k = [_rows(rng, n, Hkv, D, fk) for n in total]
    rows_v = [_rows(rng, n, Hkv, D, fv) for n in total]
    q = (rng.standard_normal((len(prefix), n_q, Hkv * G, D)) * fq).astype(np.float32)
    alpha = 1.0 / math.sqrt(D)
    # the prefixes through kvq_store, the chunk through the call under test
    pre_k = [r[:p] for r, p in zip(rows_k, prefix)]
    pre_v = [r[:p] for r, p in zip(rows_v, prefix)]
    table, npages = U.make_tables(total, 16, shuffle_seed=3)
    cache = kvq.KvqCache(layout, D, Hkv, npages, 16, n_recent=n_recent, max_batch=len(prefix), device=U.DEV)
    seq_pre = torch.tensor(prefix, dtype=torch.int32, device=U.DEV)
    for b, p in enumerate(prefix):
        if p:
            kvq.store(cache, torch.from_numpy(pre_k[b]).to(U.DEV), torch.from_numpy(pre_v[b]).to(U.DEV),
                      torch.from_numpy(U.slots_for(table, b, 0, p, 16)).to(U.DEV),
                      torch.full((p,), b, dtype=torch.int32, device=U.DEV),
                      torch.arange(p, dtype=torch.int32, device=U.DEV), seq_pre)
    kc = torch.from_numpy(np.stack([r[p:] for r, p in zip(rows_k, prefix)])).to(U.DEV)
    vc = torch.from_numpy(np.stack([r[p:] for r, p in zip(rows_v, prefix)])).to(U.DEV)
    out = kvq.prefill_full_then_store(cache, torch.from_numpy(q).to(U.DEV), kc, vc, seq_pre,
                                      torch.from_numpy(table).to(U.DEV), max(total), alpha)
    torch.cuda.synchronize()
    ref = np.stack([attention.attend_prefill_full(layout, q[b], rows_k[b], rows_v[b], alpha, prefix[b],
                                                  n_recent=n_recent) for b in range(len(prefix))])
    U.assert_close_rel(out.cpu().numpy(), ref, what=f"full prefill K x{fk:g} V x{fv:g} Q x{fq:g}")
