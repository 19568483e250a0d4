"""Pins of the oracle's attention: brute force, closed forms, exact-input cases and invariants."""

import math

import numpy as np
import pytest

from oracle import attention, quant, spec
from oracle.fwht import fwht_f32, hadamard_f64

ALL = [spec.HAD_INT4, spec.Q4_0, spec.Q6_0, spec.ASYM_G32, spec.Q8_0]


def _inputs(rng, S, Hq, Hkv, D, scale=1.0):
    q = rng.standard_normal((Hq, D)).astype(np.float32)
    k = (rng.standard_normal((S, Hkv, D)) * scale).astype(np.float32)
    v = rng.standard_normal((S, Hkv, D)).astype(np.float32)
    return q, k, v


def _plain_attention(q, K, V, alpha):
    """Textbook softmax attention in float64 for one query vector."""
    s = alpha * (K.astype(np.float64) @ q.astype(np.float64))
    p = np.exp(s - s.max())
    return (p / p.sum()) @ V.astype(np.float64)


# ------------------------------------------------------------------ brute force (explicit loops)
def _brute_decode(layout, q, k, v, alpha, n_recent, float_q=False):
    """Decode from the integer formulation with explicit Python loops over tokens and elements
    (float_q: each block's dot taken with the f32 query instead of the int8 codes)."""
    Hq, D = q.shape
    S, Hkv, _ = k.shape
    G = Hq // Hkv
    ng = spec.n_groups(layout, D)
    gsz = D // ng
    w0 = max(0, S - n_recent) if n_recent else S
    out = np.zeros((Hq, D))
    for h in range(Hq):
        hk = h // G
        qr, q8, sq = attention.prepare_query(layout, q[h])
        scores, rows = [], []
        for t in range(S):
            if t >= w0:
                krow = fwht_f32(k[t, hk]) if layout == spec.HAD_INT4 else k[t, hk].astype(np.float64)
                vrow = fwht_f32(v[t, hk]) if layout == spec.HAD_INT4 else v[t, hk].astype(np.float64)
                sc = 0.0
                for j in range(D):
                    sc += float(qr[j]) * float(krow[j])
                scores.append(alpha * sc)
                rows.append(np.array(vrow, dtype=np.float64))
                continue
            ek = quant.encode_rows(layout, k[t, hk])
            ev = quant.encode_rows(layout, v[t, hk])
            acc = 0.0
            for g in range(ng):
                I = 0
                qs = 0
                for j in range(g * gsz, (g + 1) * gsz):
                    if float_q:
                        I += float(qr[j]) * int(ek["codes"][j])
                        qs += float(qr[j])
                    else:
                        I += int(q8[j]) * int(ek["codes"][j])
                        qs += int(q8[j])
                acc += float(ek["scales"][g]) * I
                if layout == spec.ASYM_G32:
                    acc += float(ek["zeros"][g]) * qs
            scores.append(alpha * (1.0 if float_q else float(sq)) * acc)
            vrow = np.empty(D)
            for j in range(D):
                g = j // gsz
                vrow[j] = float(ev["codes"][j]) * float(ev["scales"][g])
                if layout == spec.ASYM_G32:
                    vrow[j] += float(ev["zeros"][g])
            rows.append(vrow)
        m = max(scores)
        w = [math.exp(s - m) for s in scores]
        o = sum(wt * r for wt, r in zip(w, rows)) / sum(w)
        out[h] = hadamard_f64(o) if layout == spec.HAD_INT4 else o
    return out


@pytest.mark.parametrize("layout", ALL)
@pytest.mark.parametrize("S", [1, 2, 3, 31, 32, 33, 513])
def test_decode_matches_brute_force(layout, S):
    rng = np.random.default_rng(100 + S)
    D = 64 if layout != spec.Q6_0 else 64
    q, k, v = _inputs(rng, S, Hq=2, Hkv=1, D=D)
    alpha = 1.0 / math.sqrt(D)
    for n_recent in ((0, 5) if S < 100 else (0,)):
        for float_q in (False, True):
            got = attention.attend_decode(layout, q, k, v, alpha, n_recent=n_recent, float_q=float_q)
            ref = _brute_decode(layout, q, k, v, alpha, n_recent, float_q)
            np.testing.assert_allclose(got, ref, rtol=0, atol=1e-12)


# ------------------------------------------------------------------ integer scores
@pytest.mark.parametrize("layout", ALL)
def test_scores_i32_brute_force_and_order_independence(layout, rng):
    D = 128
    codes = quant.encode_rows(layout, rng.standard_normal((5, D)).astype(np.float32))["codes"]
    q8 = rng.integers(-127, 128, size=D)
    I = attention.scores_i32(layout, q8, codes)
    ng = spec.n_groups(layout, D)
    for t in range(5):
        for g in range(ng):
            lo, hi = g * D // ng, (g + 1) * D // ng
            assert I[t, g] == sum(int(q8[j]) * int(codes[t, j]) for j in range(lo, hi))
    perm = np.concatenate([rng.permutation(np.arange(g * D // ng, (g + 1) * D // ng)) for g in range(ng)])
    np.testing.assert_array_equal(attention.scores_i32(layout, q8[perm], codes[:, perm]), I)


@pytest.mark.parametrize("layout", ALL)
def test_integer_reassociation_equals_dequantised_dot(layout, rng):
    """alpha*sq*sum_g(s_g I_g [+ z_g sum q8]) == alpha * (sq q8) . K_hat for every layout."""
    D = 128
    x = rng.standard_normal((40, D)).astype(np.float32) + 0.3
    e = quant.encode_rows(layout, x)
    qr, q8, sq = attention.prepare_query(layout, rng.standard_normal(D).astype(np.float32))
    I = attention.scores_i32(layout, q8, e["codes"])
    s_int = attention.scores_from_i32(layout, I, sq, e["scales"], e["zeros"], q8, 0.125)
    k_hat = quant.dequantize(layout, e["codes"], e["scales"], e["zeros"])
    s_def = 0.125 * (k_hat @ (sq * q8.astype(np.float64)))
    np.testing.assert_allclose(s_int, s_def, rtol=1e-12, atol=1e-12)


# ------------------------------------------------------------------ closed forms
@pytest.mark.parametrize("layout", ALL)
def test_single_token_returns_its_value_row(layout, rng):
    q, k, v = _inputs(rng, 1, 4, 2, 128)
    o = attention.attend_decode(layout, q, k, v, 0.1)
    for h in range(4):
        ev = quant.encode_rows(layout, v[0, h // 2])
        vh = quant.dequantize(layout, ev["codes"], ev["scales"], ev["zeros"])
        expect = hadamard_f64(vh) if layout == spec.HAD_INT4 else vh
        np.testing.assert_allclose(o[h], expect, atol=1e-12)


@pytest.mark.parametrize("layout", ALL)
def test_identical_keys_give_mean_of_values(layout, rng):
    S = 37
    q, k, v = _inputs(rng, S, 2, 1, 128)
    k[:] = k[0]
    o = attention.attend_decode(layout, q, k, v, 0.3)
    vh = attention.encode_cache(layout, k[:, 0], v[:, 0])["v_hat"]
    mean = vh.mean(axis=0)
    expect = hadamard_f64(mean) if layout == spec.HAD_INT4 else mean
    np.testing.assert_allclose(o[0], expect, atol=1e-12)
    np.testing.assert_allclose(o[1], expect, atol=1e-12)


def _exact_block_rows(rng, S, D, layout):
    """Rows that the layout encodes without error: d*n with a power-of-two scale that is hit."""
    if layout == spec.ASYM_G32:
        s = 2.0 ** rng.integers(-4, 0, size=(S, D // 32, 1))
        z = rng.integers(-20, 20, size=(S, D // 32, 1)) * 2.0 ** -3
        n = rng.integers(0, 16, size=(S, D // 32, 32))
        n[..., 0], n[..., 1] = 0, 15
        return (s * n + z).reshape(S, D).astype(np.float32)
    M = spec.max_magnitude(layout)
    lo, hi = spec.code_range(layout)
    d = 2.0 ** rng.integers(-5, 1, size=(S, D // 32, 1))
    n = rng.integers(lo, hi + 1, size=(S, D // 32, 32))
    n[..., 0] = -M
    return (d * n).reshape(S, D).astype(np.float32)


@pytest.mark.parametrize("layout", [spec.Q4_0, spec.Q6_0, spec.ASYM_G32, spec.Q8_0])
def test_exactly_encodable_inputs_give_textbook_attention(layout, rng):
    S, D = 70, 128
    k = _exact_block_rows(rng, S, D, layout)[:, None, :]
    v = _exact_block_rows(rng, S, D, layout)[:, None, :]
    e = quant.encode_rows(layout, k[:, 0])
    np.testing.assert_array_equal(quant.dequantize(layout, e["codes"], e["scales"], e["zeros"]), k[:, 0])
    # a query that int8 encodes exactly: sq = 2^-5, q8 hits 127
    q8 = rng.integers(-127, 128, size=(1, D))
    q8[0, 0] = 127
    q = (q8 * 2.0 ** -5).astype(np.float32)
    alpha = 1.0 / math.sqrt(D)
    o = attention.attend_decode(layout, q, k, v, alpha)
    np.testing.assert_allclose(o[0], _plain_attention(q[0], k[:, 0], v[:, 0], alpha), rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("layout", [spec.Q4_0, spec.Q6_0, spec.ASYM_G32, spec.Q8_0])
def test_float_q_on_exact_rows_is_textbook_attention_for_any_query(layout, rng):
    """Float-query mode: with rows the layout encodes exactly, only the query could differ from the
    f32 inputs, and in this mode it does not, whatever the query; the int8 mode does differ."""
    S, D = 70, 128
    k = _exact_block_rows(rng, S, D, layout)[:, None, :]
    v = _exact_block_rows(rng, S, D, layout)[:, None, :]
    q = rng.standard_normal((2, D)).astype(np.float32)
    alpha = 2.0 / (math.sqrt(D) * float(np.abs(k).max()))   # logits of order one (no one-hot softmax)
    o = attention.attend_decode(layout, q, k, v, alpha, float_q=True)
    o8 = attention.attend_decode(layout, q, k, v, alpha)
    for h in range(2):
        ref = _plain_attention(q[h], k[:, 0], v[:, 0], alpha)
        np.testing.assert_allclose(o[h], ref, rtol=1e-12, atol=1e-12)
        assert np.abs(o8[h] - ref).max() > 1e-6


@pytest.mark.parametrize("layout", ALL)
def test_float_q_equals_int8_mode_for_a_query_on_the_int8_grid(layout, rng):
    """A query whose (rotated) form int8 encodes exactly gives both modes the same scores.  For the
    Hadamard layout at D = 256, q = 16 * 127 * 2^-3 e_j rotates exactly to +-127 * 2^-3 (1/sqrt(D) =
    1/16), whose int8 scale is 2^-3."""
    S, D = 90, 256
    _, k, v = _inputs(rng, S, 2, 1, D)
    if layout == spec.HAD_INT4:
        q = np.zeros((2, D), dtype=np.float32)
        q[0, 5] = 16 * 127 * 2.0 ** -3
        q[1, 200] = -16 * 127 * 2.0 ** -3
    else:
        q8 = rng.integers(-127, 128, size=(2, D))
        q8[:, 0] = 127
        q = (q8 * 2.0 ** -4).astype(np.float32)
    qr, q8r, sq = attention.prepare_query(layout, q)
    np.testing.assert_array_equal(sq[:, None] * q8r, qr)   # the grid case really holds
    for n_recent in (0, 9):
        a = attention.attend_decode(layout, q, k, v, 0.2, n_recent=n_recent, float_q=True)
        b = attention.attend_decode(layout, q, k, v, 0.2, n_recent=n_recent)
        np.testing.assert_array_equal(a, b)


# ------------------------------------------------------------------ full-precision prefill
@pytest.mark.parametrize("layout", ALL)
@pytest.mark.parametrize("q_start,n_recent", [(0, 0), (0, 16), (40, 64), (40, 40)])
def test_full_prefill_without_quantised_prefix_is_textbook_causal_attention(layout, q_start, n_recent, rng):
    """A fresh prompt (no prefix), or a prefix that the window holds whole: every token is an exact
    f32 row, so each query gets textbook attention over t <= its position."""
    Sq, D = 23, 128
    _, k, v = _inputs(rng, q_start + Sq, 4, 2, D)
    q = rng.standard_normal((Sq, 4, D)).astype(np.float32)
    o = attention.attend_prefill_full(layout, q, k, v, 0.15, q_start, n_recent=n_recent)
    tol = 1e-5 if layout == spec.HAD_INT4 else 1e-12
    for i in range(Sq):
        for h in range(4):
            ref = _plain_attention(q[i, h], k[:q_start + i + 1, h // 2], v[:q_start + i + 1, h // 2], 0.15)
            np.testing.assert_allclose(o[i, h], ref, rtol=tol, atol=tol)


@pytest.mark.parametrize("layout", [spec.Q4_0, spec.Q6_0, spec.ASYM_G32, spec.Q8_0])
def test_full_prefill_equals_compressed_prefill_when_nothing_is_lost(layout, rng):
    """Rows the layout encodes exactly and queries on the int8 grid: quantising loses nothing, so the
    full-precision prefill equals the compressed-domain prefill over the cache after the append."""
    q_start, Sq, D = 70, 30, 128
    k = _exact_block_rows(rng, q_start + Sq, D, layout)[:, None, :]
    v = _exact_block_rows(rng, q_start + Sq, D, layout)[:, None, :]
    q8 = rng.integers(-127, 128, size=(Sq, 2, D))
    q8[..., 0] = 127
    q = (q8 * 2.0 ** -6).astype(np.float32)
    for causal in (True, False):
        a = attention.attend_prefill_full(layout, q, k, v, 0.05, q_start, causal=causal)
        b = attention.attend_prefill(layout, q, k, v, 0.05, q_start, causal=causal)
        np.testing.assert_allclose(a, b, rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("layout", ALL)
def test_full_prefill_last_query_not_masked(layout, rng):
    """The last query of the chunk sees every token, so causal and non-causal agree on it; with the
    chunk's tokens hidden (a one-token chunk is its own last token) the quantised prefix counts."""
    q_start, Sq = 50, 9
    _, k, v = _inputs(rng, q_start + Sq, 2, 1, 128)
    q = rng.standard_normal((Sq, 2, 128)).astype(np.float32)
    a = attention.attend_prefill_full(layout, q, k, v, 0.2, q_start, causal=True, n_recent=5)
    b = attention.attend_prefill_full(layout, q, k, v, 0.2, q_start, causal=False, n_recent=5)
    np.testing.assert_allclose(a[-1], b[-1], rtol=1e-12, atol=1e-12)
    assert np.abs(a[0] - b[0]).max() > 1e-6
    with pytest.raises(ValueError):
        attention.attend_prefill_full(layout, q, k[:-1], v[:-1], 0.2, q_start)


@pytest.mark.parametrize("layout", ALL)
def test_full_window_is_plain_attention(layout, rng):
    """n_recent >= S keeps every token in f32: the result is plain attention on the inputs."""
    S, D = 45, 128
    q, k, v = _inputs(rng, S, 2, 1, D)
    alpha = 1.0 / math.sqrt(D)
    o = attention.attend_decode(layout, q, k, v, alpha, n_recent=S + 3)
    tol = 1e-12 if layout != spec.HAD_INT4 else 2e-6   # HAD: f32 rotation of q, K, V only
    for h in range(2):
        ref = _plain_attention(q[h], k[:, 0], v[:, 0], alpha)
        np.testing.assert_allclose(o[h], ref, rtol=0, atol=tol)
    # and the quantised cache alone is not plain attention
    o0 = attention.attend_decode(layout, q, k, v, alpha, n_recent=0)
    assert np.abs(o0[0] - _plain_attention(q[0], k[:, 0], v[:, 0], alpha)).max() > 1e-4


def test_window_boundary_token(rng):
    """With n_recent = w the token at S - w is read in f32 and the one before it quantised."""
    S, D, w = 20, 128, 4
    q, k, v = _inputs(rng, S, 1, 1, D)
    alpha = 1.0 / math.sqrt(D)
    o = attention.attend_decode(spec.Q4_0, q, k, v, alpha, n_recent=w)
    np.testing.assert_allclose(o, _brute_decode(spec.Q4_0, q, k, v, alpha, w), atol=1e-12)
    # perturbing a quantisation-invisible bit of token S-w changes the output, of S-w-1 does not
    k2 = k.copy()
    k2[S - w, 0, 0] = np.nextafter(k2[S - w, 0, 0], np.float32(np.inf))
    assert np.any(attention.attend_decode(spec.Q4_0, q, k2, v, alpha, n_recent=w) != o)


# ------------------------------------------------------------------ invariants
@pytest.mark.parametrize("layout", ALL)
@pytest.mark.parametrize("chunk", [1, 7, 64, 512, 4096])
def test_split_k_merge_equals_single_pass(layout, chunk, rng):
    S = 600
    q, k, v = _inputs(rng, S, 4, 2, 128, scale=2.0)
    for float_q in (False, True):
        a = attention.attend_decode(layout, q, k, v, 0.2, n_recent=9, float_q=float_q)
        b = attention.attend_decode_split(layout, q, k, v, 0.2, chunk, n_recent=9, float_q=float_q)
        np.testing.assert_allclose(b, a, rtol=1e-12, atol=1e-13)


def test_merge_ignores_empty_chunks():
    D = 4
    o1 = np.arange(D, dtype=np.float64)
    parts = [(np.zeros(D), -np.inf, 0.0), (o1, 0.5, 2.0), (np.zeros(D), -np.inf, 0.0)]
    np.testing.assert_allclose(attention.merge_partials(parts), o1 / 2.0)
    assert attention.chunk_partial(np.array([]), np.zeros((0, D)))[1] == -np.inf
    assert attention.chunk_partial(np.full(3, -np.inf), np.ones((3, D)))[2] == 0.0


@pytest.mark.parametrize("layout", ALL)
def test_gqa_equals_mha_with_replicated_kv(layout, rng):
    S, Hkv, G, D = 50, 2, 4, 128
    q, k, v = _inputs(rng, S, Hkv * G, Hkv, D)
    o = attention.attend_decode(layout, q, k, v, 0.1)
    krep = np.repeat(k, G, axis=1)          # kv head for query head h is h // G
    vrep = np.repeat(v, G, axis=1)
    o_mha = attention.attend_decode(layout, q, krep, vrep, 0.1)
    np.testing.assert_allclose(o, o_mha, atol=1e-13)
    # the other mapping (h mod Hkv) gives a different answer
    kalt = np.tile(k, (1, G, 1))
    valt = np.tile(v, (1, G, 1))
    assert np.abs(attention.attend_decode(layout, q, kalt, valt, 0.1) - o).max() > 1e-3


@pytest.mark.parametrize("layout", ALL)
def test_causal_prefill_row_equals_decode_on_its_prefix(layout, rng):
    S, Sq, D = 90, 12, 128
    q_start = S - Sq
    qs = rng.standard_normal((Sq, 2, D)).astype(np.float32)
    _, k, v = _inputs(rng, S, 2, 1, D)
    o = attention.attend_prefill(layout, qs, k, v, 0.1, q_start, causal=True)
    for i in range(Sq):
        p = q_start + i
        ref = attention.attend_decode(layout, qs[i], k[:p + 1], v[:p + 1], 0.1)
        np.testing.assert_allclose(o[i], ref, atol=1e-12)
    # non-causal: every row sees the whole cache
    o_full = attention.attend_prefill(layout, qs, k, v, 0.1, q_start, causal=False)
    for i in (0, Sq - 1):
        np.testing.assert_allclose(o_full[i], attention.attend_decode(layout, qs[i], k, v, 0.1), atol=1e-12)
    # decode == the last prefill row (it sees every token)
    np.testing.assert_allclose(o[-1], o_full[-1], atol=1e-12)


def test_causal_prefill_with_window_brute_force(rng):
    S, Sq, D, w = 40, 6, 128, 8
    q_start = S - Sq
    qs = rng.standard_normal((Sq, 2, D)).astype(np.float32)
    _, k, v = _inputs(rng, S, 2, 2, D)
    o = attention.attend_prefill(spec.HAD_INT4, qs, k, v, 0.1, q_start, causal=True, n_recent=w)
    for i in range(Sq):
        p = q_start + i
        # visible tokens t <= p; window is the last w positions of the whole cache
        for h in range(2):
            qr, q8, sq = attention.prepare_query(spec.HAD_INT4, qs[i, h])
            sc, rows = [], []
            for t in range(p + 1):
                if t >= S - w:
                    kr, vr = fwht_f32(k[t, h]), fwht_f32(v[t, h])
                    sc.append(0.1 * float(np.dot(qr, kr)))
                else:
                    ek = quant.encode_rows(spec.HAD_INT4, k[t, h])
                    ev = quant.encode_rows(spec.HAD_INT4, v[t, h])
                    sc.append(0.1 * float(sq) * float(ek["scales"][0]) * int(np.dot(q8, ek["codes"])))
                    vr = ev["codes"] * ev["scales"][0]
                rows.append(np.asarray(vr, dtype=np.float64))
            m = max(sc)
            wts = np.exp(np.array(sc) - m)
            ref = hadamard_f64((wts[:, None] * np.array(rows)).sum(0) / wts.sum())
            np.testing.assert_allclose(o[i, h], ref, atol=1e-12)


def test_query_preparation_rotates_only_for_hadamard(rng):
    q = rng.standard_normal(128).astype(np.float32)
    qr, q8, sq = attention.prepare_query(spec.HAD_INT4, q)
    np.testing.assert_array_equal(qr, fwht_f32(q))
    qr2, _, _ = attention.prepare_query(spec.Q4_0, q)
    np.testing.assert_array_equal(qr2, q.astype(np.float64))
    assert np.abs(q8).max() == 127


def test_empty_cache_gives_zeros():
    q = np.ones((2, 128), dtype=np.float32)
    k = np.zeros((0, 1, 128), dtype=np.float32)
    assert not attention.attend_decode(spec.Q4_0, q, k, k, 0.1).any()
