"""GPU parity of the causal prefill against the oracle, and the causal-skip equivalence.

Outputs: max|diff| <= 2e-3 * max|o_ref| against ``oracle.attention.attend_prefill``
(compute-then-mask in float64).  Causal skip on and off must give the same bits
([tract-RFC] Causality & mixed precision), and a one-query prefill whose limit
covers the whole cache must agree with the decode output (both are the same
attention with every token visible).
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


def _case(layout, D, Hkv, G, lens, n_q, q_starts, n_recent=0, page_size=16, seed=0, alpha=None, k_ramp=False):
    rng = np.random.default_rng(seed)
    rows_k = [rng.standard_normal((n, Hkv, D)).astype(np.float32) for n in lens]
    if k_ramp:   # |K| growing along the cache: the rows' running maxima keep moving
        rows_k = [(k * np.linspace(0.2, 3.0, len(k), dtype=np.float32)[:, None, None]).astype(np.float32)
                  for k in rows_k]
    rows_v = [rng.standard_normal((n, Hkv, D)).astype(np.float32) for n in lens]
    B, Hq = len(lens), Hkv * G
    q = rng.standard_normal((B, n_q, Hq, D)).astype(np.float32)
    alpha = alpha if alpha is not None else 1.0 / math.sqrt(D)
    cache, bt, seq, _ = U.build_cache(layout, D, Hkv, rows_k, rows_v, page_size=page_size, n_recent=n_recent)
    qs = torch.tensor(q_starts, dtype=torch.int32, device=U.DEV)
    return dict(layout=layout, cache=cache, bt=bt, seq=seq, qs=qs, q=q, qt=torch.from_numpy(q).to(U.DEV),
                rows_k=rows_k, rows_v=rows_v, alpha=alpha, maxs=max(max(lens), 1), n_recent=n_recent,
                q_starts=q_starts)


def _gpu(c, causal=True, skip=True):
    out = kvq.attend_prefill_causal(c["cache"], c["qt"], c["qs"], c["bt"], c["seq"], c["maxs"], c["alpha"],
                                    causal=causal, causal_skip=skip)
    torch.cuda.synchronize()
    return out


def _ref(c, causal=True):
    return np.stack([attention.attend_prefill(c["layout"], c["q"][b], c["rows_k"][b], c["rows_v"][b], c["alpha"],
                                              c["q_starts"][b], causal=causal, n_recent=c["n_recent"])
                     for b in range(len(c["rows_k"]))])


@pytest.mark.parametrize("layout", ALL)
@pytest.mark.parametrize("D", [128, 256])
@pytest.mark.parametrize("G", [1, 2, 8])
def test_prefill_matches_oracle(layout, D, G):
    """A chunk of 37 queries appended at the tail (rows not a multiple of the 16-row tile)."""
    U.need_gpu()
    lens, n_q = [1300, 300], 37
    c = _case(layout, D, 2, G, lens, n_q, [n - n_q for n in lens], seed=7 * G + D + layout)
    got = _gpu(c).cpu().numpy()
    U.assert_close_rel(got, _ref(c))
    assert torch.equal(_gpu(c, skip=False), torch.from_numpy(got).to(U.DEV))


@pytest.mark.parametrize("layout", ALL)
@pytest.mark.parametrize("n_recent", [16, 64])
def test_prefill_window(layout, n_recent):
    """Window tokens are exact f32 and masked per query like the packed ones."""
    U.need_gpu()
    lens, n_q = [900, 70], 50
    c = _case(layout, 128, 2, 2, lens, n_q, [n - n_q for n in lens], n_recent=n_recent, seed=n_recent + layout)
    got = _gpu(c)
    U.assert_close_rel(got.cpu().numpy(), _ref(c))
    assert torch.equal(_gpu(c, skip=False), got)


def test_prefill_window_wholly_masked():
    """Queries that see none of the window tokens (their limits end before it)."""
    U.need_gpu()
    c = _case(spec.Q4_0, 128, 1, 4, [700], 10, [300], n_recent=64, seed=5)
    got = _gpu(c)
    U.assert_close_rel(got.cpu().numpy(), _ref(c))
    assert torch.equal(_gpu(c, skip=False), got)


@pytest.mark.parametrize("layout", [spec.HAD_INT4, spec.ASYM_G32])
def test_prefill_mid_cache_and_ragged_batch(layout):
    """Chunks that start inside the cache (later tokens exist but are masked), different per row."""
    U.need_gpu()
    lens = [2100, 600, 33]
    c = _case(layout, 128, 2, 4, lens, 24, [1000, 576, 0], n_recent=8, seed=21 + layout)
    got = _gpu(c)
    U.assert_close_rel(got.cpu().numpy(), _ref(c))
    assert torch.equal(_gpu(c, skip=False), got)


@pytest.mark.parametrize("layout", ALL)
@pytest.mark.parametrize("alpha", [-0.09, 0.0, 0.6], ids=["negative", "zero", "sharp"])
def test_prefill_score_scale(layout, alpha):
    """Negative, zero and large attention scales over a cache whose scores grow along it, so that the
    rows' running maxima are raised many times (and by more than the lazy threshold)."""
    U.need_gpu()
    lens, n_q = [1500, 400], 40
    c = _case(layout, 128, 2, 2, lens, n_q, [n - n_q for n in lens], n_recent=16, seed=71 + layout, alpha=alpha,
              k_ramp=True)
    got = _gpu(c)
    U.assert_close_rel(got.cpu().numpy(), _ref(c))
    assert torch.equal(_gpu(c, skip=False), got)


@pytest.mark.parametrize("layout", ALL)
def test_prefill_not_causal(layout):
    U.need_gpu()
    c = _case(layout, 128, 2, 2, [800, 129], 20, [0, 0], n_recent=16, seed=31 + layout)
    got = _gpu(c, causal=False)
    U.assert_close_rel(got.cpu().numpy(), _ref(c, causal=False))


@pytest.mark.parametrize("layout", ALL)
def test_prefill_first_queries_of_a_prompt(layout):
    """q_start = 0: query i sees tokens 0..i only (tiny prefixes, many fully masked steps)."""
    U.need_gpu()
    c = _case(layout, 128, 1, 2, [600], 600, [0], seed=41 + layout)
    got = _gpu(c)
    U.assert_close_rel(got.cpu().numpy(), _ref(c))
    assert torch.equal(_gpu(c, skip=False), got)


@pytest.mark.parametrize("layout", ALL)
@pytest.mark.parametrize("n_recent", [0, 32])
def test_last_query_equals_decode(layout, n_recent):
    """One query at the last position sees every token: the decode output (the two kernels
    differ only in float association: chunking, and where the fp16 V scale is applied)."""
    U.need_gpu()
    lens = [1700, 90]
    c = _case(layout, 128, 2, 4, lens, 1, [n - 1 for n in lens], n_recent=n_recent, seed=51 + layout)
    pre = _gpu(c)[:, 0]
    dec = kvq.attend_decode(c["cache"], c["qt"][:, 0].contiguous(), c["bt"], c["seq"], c["maxs"], c["alpha"],
                            chunk_tokens=512)
    torch.cuda.synchronize()
    U.assert_close_rel(pre.cpu().numpy(), dec.cpu().numpy(), what="prefill vs decode")
    U.assert_close_rel(pre.cpu().numpy(), _ref(c)[:, 0], what="prefill vs oracle")


def test_decode_gqa_group_above_16():
    """G = 20 spans two 16-row tiles of the same kv head."""
    U.need_gpu()
    rng = np.random.default_rng(61)
    lens, Hkv, G, D = [1000], 1, 20, 128
    rows_k = [rng.standard_normal((n, Hkv, D)).astype(np.float32) for n in lens]
    rows_v = [rng.standard_normal((n, Hkv, D)).astype(np.float32) for n in lens]
    q = rng.standard_normal((1, G, D)).astype(np.float32)
    cache, bt, seq, _ = U.build_cache(spec.Q4_0, D, Hkv, rows_k, rows_v)
    got = kvq.attend_decode(cache, torch.from_numpy(q).to(U.DEV), bt, seq, 1000, 1 / math.sqrt(D)).cpu().numpy()
    ref = attention.attend_decode(spec.Q4_0, q[0], rows_k[0], rows_v[0], 1 / math.sqrt(D))
    U.assert_close_rel(got[0], ref)


def test_prefill_validation():
    U.need_gpu()
    c = _case(spec.Q4_0, 128, 1, 1, [64], 4, [60], seed=1)
    with pytest.raises(kvq.KvqError, match="workspace"):
        kvq.attend_prefill_causal(c["cache"], c["qt"], c["qs"], c["bt"], c["seq"], c["maxs"], 1.0,
                                  workspace=torch.empty(8, dtype=torch.uint8, device=U.DEV))


def test_prefill_many_slots_sampled():
    """More split-K slots than a wave has lanes (36864 tokens: 72 chunks of the shortest split, 512
    tokens, and the window) with 4096 query rows, so that the reduce merges the narrow partial records
    on its general path; queries 200..202 of the chunk against the oracle."""
    U.need_gpu()
    L, n_q, Hkv, G, D = 36864, 256, 4, 4, 128
    c = _case(spec.HAD_INT4, D, Hkv, G, [L], n_q, [L - n_q], n_recent=64, page_size=256, seed=11)
    assert kvq.prefill_workspace_bytes(1, n_q, Hkv * G, D, L) > 0
    got = _gpu(c).cpu().numpy()
    i0 = 200
    ref = attention.attend_prefill(c["layout"], c["q"][0][i0:i0 + 3], c["rows_k"][0], c["rows_v"][0], c["alpha"],
                                   c["q_starts"][0] + i0, causal=True, n_recent=c["n_recent"])
    U.assert_close_rel(got[0, i0:i0 + 3], ref)
