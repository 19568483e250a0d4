"""The decode entry point without a workspace (kvq_attend_decode_noalloc) against kvq_attend_decode.

Both run the same kernels on the same arguments, so the outputs must be the same bits.  Two calls in
a row share the device scratch: the second, smaller, call must not see the first call's partials.
A call whose partials exceed the scratch is refused before anything is launched.
"""

import math

import numpy as np
import pytest
import torch

import quantized_kv_cache_store_amd as kvq
from oracle import attention, spec
import gpu_util as U

pytestmark = pytest.mark.gpu


def _case(layout, D, Hkv, G, lens, n_recent, seed):
    rng = np.random.default_rng(seed)
    rows_k = [rng.standard_normal((n, Hkv, D)).astype(np.float32) for n in lens]
    rows_v = [rng.standard_normal((n, Hkv, D)).astype(np.float32) for n in lens]
    q = rng.standard_normal((len(lens), Hkv * G, D)).astype(np.float32)
    cache, bt, seq, _ = U.build_cache(layout, D, Hkv, rows_k, rows_v, n_recent=n_recent)
    return cache, bt, seq, q, rows_k, rows_v


@pytest.mark.parametrize("layout", [spec.HAD_INT4, spec.ASYM_G32, spec.Q6_0])
def test_noalloc_equals_workspace_decode_two_calls(layout):
    U.need_gpu()
    D = 256 if layout == spec.Q6_0 else 128
    big = _case(layout, D, 2, 8, [5000, 1300, 77], 16, seed=1 + layout)
    small = _case(layout, D, 1, 2, [600], 0, seed=2 + layout)
    alpha = 1.0 / math.sqrt(D)
    for cache, bt, seq, q, rows_k, rows_v in (big, small):
        S = int(seq.max().item())
        qt = torch.from_numpy(q).to(U.DEV)
        got = kvq.attend_decode_noalloc(cache, qt, bt, seq, S, alpha)
        ref = kvq.attend_decode(cache, qt, bt, seq, S, alpha)
        torch.cuda.synchronize()
        assert torch.equal(got, ref)
        oracle = np.stack([attention.attend_decode(layout, q[b], rows_k[b], rows_v[b], alpha,
                                                   n_recent=cache.n_recent) for b in range(len(rows_k))])
        U.assert_close_rel(got.cpu().numpy(), oracle)


def test_noalloc_rejects_calls_beyond_the_scratch():
    U.need_gpu()
    cache, _, _, _, _, _ = _case(spec.Q4_0, 128, 1, 1, [100], 0, seed=3)
    # 64 rows x 64 query heads at 2^20 tokens need about 279 MB of partials: refused on the host
    B, S = 64, 1 << 20
    qb = torch.zeros((B, 64, 128), dtype=torch.float32, device=U.DEV)
    table = torch.zeros((B, S // 16), dtype=torch.int32, device=U.DEV)
    sl = torch.full((B,), S, dtype=torch.int32, device=U.DEV)
    with pytest.raises(kvq.KvqError, match="scratch"):
        kvq.attend_decode_noalloc(cache, qb, table, sl, S, 1.0)
