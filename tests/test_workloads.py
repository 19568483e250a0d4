"""The seeded input generators: deterministic, slice-addressable, and shaped as stated."""

import numpy as np

import workloads as W


def test_deterministic_and_slice_addressable():
    w = W.WORKLOADS["llama3_8b_q4_0_s32k"]
    a = W.kv_rows(w, 0, 3, 4000, 4200, "k")
    b = W.kv_rows(w, 0, 3, 0, 8192, "k")[4000:4200]
    np.testing.assert_array_equal(a, b)
    np.testing.assert_array_equal(a, W.kv_rows(w, 0, 3, 4000, 4200, "k"))
    assert not np.array_equal(W.kv_rows(w, 0, 3, 0, 10, "k"), W.kv_rows(w, 0, 3, 0, 10, "v"))
    assert not np.array_equal(W.kv_rows(w, 0, 2, 0, 10, "k"), W.kv_rows(w, 0, 3, 0, 10, "k"))
    toks = W.kv_tokens(w, 0, 10, 20, "v")
    assert toks.shape == (10, w.Hkv, w.D) and toks.dtype == np.float32
    np.testing.assert_array_equal(toks[:, 5], W.kv_rows(w, 0, 5, 10, 20, "v"))


def test_outlier_channels_are_scaled():
    w = W.WORKLOADS["qwen3_1p7b_had_s8k"]
    ch = W.outlier_channels(w, 1)
    assert ch.size == 4
    x = W.kv_rows(w, 0, 1, 0, 4096, "k")
    rms = np.sqrt((x.astype(np.float64) ** 2).mean(axis=0))
    assert np.all(rms[ch] > 7.0)
    assert np.all(np.delete(rms, ch) < 1.3)


def test_student_t_unit_variance_and_rms_norm():
    w = W.WORKLOADS["llama31_70b_asym_s128k"]
    x = W.kv_rows(w, 1, 0, 0, 8192, "v").astype(np.float64)
    assert 0.8 < x.var() < 1.25            # t3 / sqrt(3) has unit variance (heavy tail)
    assert np.abs(x).max() > 8.0           # kurtotic: far tails present
    g = W.WORKLOADS["gemma_q6_0_ragged_b16"]
    k = W.kv_rows(g, 0, 0, 0, 64, "k").astype(np.float64)
    np.testing.assert_allclose((k ** 2).mean(axis=-1), 1.0, rtol=1e-4)
    q = W.queries(g, 0).astype(np.float64)
    np.testing.assert_allclose((q ** 2).mean(axis=-1), 1.0, rtol=1e-4)


def test_ragged_lengths_and_shuffled_pages():
    g = W.WORKLOADS["gemma_q6_0_ragged_b16"]
    lens = W.seq_lens(g)
    assert lens.shape == (16,) and lens.min() >= 4096 and lens.max() <= 65536
    np.testing.assert_array_equal(lens, W.seq_lens(g))
    table, total = W.block_tables(g, lens)
    used = table[table >= 0]
    assert used.size == total and np.array_equal(np.sort(used), np.arange(total))
    assert not np.array_equal(used, np.arange(total))     # shuffled
    w = W.WORKLOADS["tiny_q4_0_s1024"]
    t1, n1 = W.block_tables(w, W.seq_lens(w))
    assert n1 == 4 and list(t1[0]) == [0, 1, 2, 3]
