"""GPU parity of quantize-on-append: stored bytes, scales and window rows bit-exact vs the oracle."""

import numpy as np
import pytest
import torch

from oracle import quant, spec
from oracle.attention import prepare_query
from oracle.fwht import fwht_f32
import gpu_util as U

pytestmark = pytest.mark.gpu

CASES = [(spec.HAD_INT4, 128), (spec.HAD_INT4, 256), (spec.Q4_0, 128), (spec.Q4_0, 256),
         (spec.Q6_0, 128), (spec.Q6_0, 256), (spec.ASYM_G32, 128), (spec.ASYM_G32, 256),
         (spec.Q8_0, 128), (spec.Q8_0, 256)]


def _special_rows(rng, n, D):
    """Rows that stress the encoders: scales spanning decades, outliers, zeros, constants,
    huge values (fp16 saturation), exact rounding ties, negative-only and positive-only rows."""
    x = rng.standard_normal((n, D)) * (10.0 ** rng.uniform(-3, 3, size=(n, 1)))
    x[0] = 0.0
    x[1] = 1.5
    x[2, :] = rng.standard_normal(D) * 1e5        # saturates fp16 scales
    x[3, 5] = 1e6
    x[4] = np.abs(x[4])
    x[5] = -np.abs(x[5])
    # exact ties: d = 2^-3 with amax = 8d, values (k + 0.5) d
    t = (rng.integers(-7, 7, size=D) + 0.5) * 0.125
    t[::32] = -1.0
    x[6] = t
    x[7, rng.choice(D, 4, replace=False)] *= 30.0  # outlier channels
    x[8] = rng.standard_t(3, size=D)
    return x.astype(np.float32)


@pytest.mark.parametrize("layout,D", CASES)
def test_store_planes_bit_exact(layout, D):
    U.need_gpu()
    rng = np.random.default_rng(1000 + 10 * layout + D)
    Hkv, lens, n_recent = 2, [157, 40], 9
    rows_k = [np.stack([_special_rows(rng, n, D) for _ in range(Hkv)], axis=1) for n in lens]
    rows_v = [np.stack([_special_rows(rng, n, D) for _ in range(Hkv)], axis=1) for n in lens]
    cache, bt, seq, table = U.build_cache(layout, D, Hkv, rows_k, rows_v, page_size=16, n_recent=n_recent)
    for b, n in enumerate(lens):
        for h in range(Hkv):
            for which, rows in (("k", rows_k[b]), ("v", rows_v[b])):
                e = quant.encode_rows(layout, rows[:, h, :])
                pay, rec = U.row_bytes(cache, which, table, b, 0, n, h)
                np.testing.assert_array_equal(pay, e["payload"], err_msg=f"payload b{b} h{h} {which}")
                np.testing.assert_array_equal(rec, e["record"], err_msg=f"record b{b} h{h} {which}")
                # window ring: the last n_recent positions, slot = pos % n_recent
                ring = (cache.k_recent if which == "k" else cache.v_recent)[b, h].cpu().numpy()
                f32rows = e["rotated"] if layout == spec.HAD_INT4 else rows[:, h, :].astype(np.float64)
                for p in range(max(0, n - n_recent), n):
                    np.testing.assert_array_equal(ring[p % n_recent], f32rows[p].astype(np.float32),
                                                  err_msg=f"ring b{b} h{h} {which} pos {p}")


@pytest.mark.parametrize("layout,D", [(spec.HAD_INT4, 128), (spec.Q4_0, 128), (spec.HAD_INT4, 256), (spec.Q6_0, 256)])
def test_query_int8_bit_exact(layout, D):
    U.need_gpu()
    import quantized_kv_cache_store_amd as kvq
    rng = np.random.default_rng(77 + D)
    q = _special_rows(rng, 37, D)
    q8, sq = kvq.debug_quantize_q(layout, torch.from_numpy(q).to(U.DEV))
    _, q8_ref, sq_ref = prepare_query(layout, q)
    np.testing.assert_array_equal(q8.cpu().numpy(), q8_ref)
    np.testing.assert_array_equal(sq.cpu().numpy(), sq_ref.astype(np.float32))


def test_store_multi_token_append_window_slots():
    """A 40-token append with n_recent 16 writes each ring slot once: the newest 16 positions."""
    U.need_gpu()
    rng = np.random.default_rng(5)
    D, Hkv = 128, 1
    k = rng.standard_normal((100, Hkv, D)).astype(np.float32)
    v = rng.standard_normal((100, Hkv, D)).astype(np.float32)
    cache, bt, seq, table = U.build_cache(spec.Q4_0, D, Hkv, [k], [v], n_recent=16, chunk=40)
    ring = cache.k_recent[0, 0].cpu().numpy()
    for p in range(84, 100):
        np.testing.assert_array_equal(ring[p % 16], k[p, 0])
