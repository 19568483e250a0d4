"""The accuracy-envelope harness (oracle only): what it must reproduce exactly, and the orderings the
pages report.

The pages' own error figures ([FreeToken-268] Validation: q4_0 0.094, q6_0 0.024 on kurtotic K/V;
[tract-RFC]: the planted-outlier figure falls to 0 as the exact-f32 window covers the sequence)
come from undefined metrics and data, so they are not pinned as numbers; the structure is:
no quantisation gives exact attention, a full window gives exact attention, more bits give
less error, a wider window gives less error.
"""

import numpy as np
import pytest

import workloads as W
from oracle import envelope, spec
from oracle.envelope import exact_attention, quantized_attention, rel_error

pytestmark = pytest.mark.filterwarnings("ignore::RuntimeWarning")

ALL = [spec.HAD_INT4, spec.Q4_0, spec.Q6_0, spec.ASYM_G32, spec.Q8_0]


def _data(name, S=512, kv_heads=2):
    return envelope._sample(W.WORKLOADS[name], S, kv_heads) + (W.WORKLOADS[name].alpha,)


def test_exact_attention_is_plain_softmax():
    """Against a hand-written loop on a tiny case (brute force)."""
    rng = np.random.default_rng(3)
    q = rng.standard_normal((2, 8)).astype(np.float32)
    k = rng.standard_normal((5, 1, 8)).astype(np.float32)
    v = rng.standard_normal((5, 1, 8)).astype(np.float32)
    o = exact_attention(q, k, v, 0.5)
    for h in range(2):
        s = [0.5 * float(np.dot(q[h].astype(np.float64), k[t, 0].astype(np.float64))) for t in range(5)]
        m = max(s)
        e = [np.exp(x - m) for x in s]
        ref = sum(e[t] * v[t, 0].astype(np.float64) for t in range(5)) / sum(e)
        np.testing.assert_allclose(o[h], ref, rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("layout", ALL)
def test_nothing_quantised_is_exact(layout):
    """Both sides exact and an f32 query: only the f32 rounding of the rotated rows (HAD) remains."""
    q, k, v, alpha = _data("llama31_70b_asym_s128k")
    o = quantized_attention(layout, q, k, v, alpha, quant_k=False, quant_v=False, int8_q=False)
    tol = 1e-5 if layout == spec.HAD_INT4 else 1e-12
    assert rel_error(o, exact_attention(q, k, v, alpha)) < tol


@pytest.mark.parametrize("layout", ALL)
def test_full_window_is_exact(layout):
    """n_recent >= S: every token is an exact f32 row scored with the f32 query ([tract-RFC]: a window
    over the whole sequence reports zero deviation)."""
    q, k, v, alpha = _data("qwen3_1p7b_had_s8k", S=300)
    o = quantized_attention(layout, q, k, v, alpha, n_recent=300)
    tol = 1e-5 if layout == spec.HAD_INT4 else 1e-12
    assert rel_error(o, exact_attention(q, k, v, alpha)) < tol


def test_full_options_equal_the_hot_path_definition():
    from oracle import attention

    q, k, v, alpha = _data("llama3_8b_q4_0_s32k", S=200)
    for layout in ALL:
        np.testing.assert_array_equal(quantized_attention(layout, q, k, v, alpha, n_recent=32),
                                      attention.attend_decode(layout, q, k, v, alpha, n_recent=32))
        np.testing.assert_array_equal(quantized_attention(layout, q, k, v, alpha, int8_q=False, n_recent=32),
                                      attention.attend_decode(layout, q, k, v, alpha, n_recent=32, float_q=True))


@pytest.mark.parametrize("name", ["llama3_8b_q4_0_s32k", "llama31_70b_asym_s128k", "gemma_q6_0_ragged_b16"])
def test_six_bits_beat_four(name):
    """q6_0 lands closer to exact than q4_0 on the same values ([FreeToken-268] Validation ordering)."""
    q, k, v, alpha = _data(name)
    rows = {r["layout"]: r for r in envelope.envelope_rows(q, k, v, alpha, [spec.Q4_0, spec.Q6_0, spec.Q8_0])}
    assert rows[spec.Q6_0]["kv"] < rows[spec.Q4_0]["kv"]
    assert rows[spec.Q8_0]["kv"] < rows[spec.Q6_0]["kv"]
    for r in rows.values():
        assert 0.0 < r["kv"] < 1.0 and 0.0 < r["k_only"] < 1.0 and 0.0 < r["v_only"] < 1.0


def test_window_sweep_shrinks_the_error():
    q, k, v, alpha = _data("qwen3_1p7b_had_s8k", S=512)
    sweep = dict(envelope.window_sweep(spec.HAD_INT4, q, k, v, alpha, [0, 128, 384, 512]))
    assert sweep[512] < 1e-5
    assert sweep[384] < sweep[0] and sweep[128] <= sweep[0] * 1.05
