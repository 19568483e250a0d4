"""GPU parity on the five workloads at their full sizes, in the launch configuration the bench times.

Small workloads are compared in full.  The 128K and ragged batches are too large
for the float64 oracle in a test, so the cache is filled with device-drawn
values except for a few sampled (batch row, kv head) pairs, whose K/V come from
the seeded CPU generator; those pairs' outputs (all G query heads) are checked
against the oracle.  The other rows still run through the same launch.

Bar: stored bytes bit-exact; outputs max|diff| <= 2e-3 * max|o_ref| per case.
"""

import numpy as np
import pytest
import torch

import quantized_kv_cache_store_amd as kvq
import workloads as W
from oracle import attention, quant, spec
import gpu_util as U

pytestmark = pytest.mark.gpu

LAYOUT = {"had_int4": spec.HAD_INT4, "q4_0": spec.Q4_0, "q6_0": spec.Q6_0, "asym_int4_g32": spec.ASYM_G32, "q8_0": spec.Q8_0}
BLOCK = 16384


def _fill(w, cache, table, lens, cpu_pairs=(), gen_seed=0, upto=None):
    """Store tokens [0, upto_b) of every row; rows/heads in cpu_pairs take the seeded CPU values."""
    g = torch.Generator(device=U.DEV)
    g.manual_seed(1000 + gen_seed)
    seq = torch.tensor(lens, dtype=torch.int32, device=U.DEV)
    for b, n in enumerate(lens):
        end = n if upto is None else upto[b]
        heads = [hk for (bb, hk) in cpu_pairs if bb == b]
        for t0 in range(0, end, BLOCK):
            t1 = min(end, t0 + BLOCK)
            k = W.kv_tokens_device(w, t1 - t0, "k", g, U.DEV)
            v = W.kv_tokens_device(w, t1 - t0, "v", g, U.DEV)
            for hk in heads:
                k[:, hk] = torch.from_numpy(W.kv_rows(w, b, hk, t0, t1, "k")).to(U.DEV)
                v[:, hk] = torch.from_numpy(W.kv_rows(w, b, hk, t0, t1, "v")).to(U.DEV)
            sl = torch.from_numpy(U.slots_for(table, b, t0, t1, w.page_size)).to(U.DEV)
            kvq.store(cache, k, v, sl, torch.full((t1 - t0,), b, dtype=torch.int32, device=U.DEV),
                      torch.arange(t0, t1, dtype=torch.int32, device=U.DEV), seq)
    torch.cuda.synchronize()
    return seq


def _cache_for(w, lens, B):
    if w.shuffle_pages:
        table, total = W.block_tables(w, lens)
        table = np.where(table < 0, table[:, :1], table).astype(np.int32)   # unused entries: a page of the row
    else:
        table, total = U.make_tables(lens, w.page_size)
    cache = kvq.KvqCache(LAYOUT[w.layout], w.D, w.Hkv, total, w.page_size, n_recent=w.n_recent, max_batch=B,
                         device=U.DEV)
    return cache, table


def _decode(w, cache, table, seq, q, maxs):
    out = kvq.attend_decode(cache, torch.from_numpy(q).to(U.DEV), torch.from_numpy(table).to(U.DEV), seq, maxs,
                            w.alpha, chunk_tokens=w.chunk_tokens)
    torch.cuda.synchronize()
    return out.cpu().numpy()


def _check_pair(w, got, q, b, hk, S):
    k = W.kv_rows(w, b, hk, 0, S, "k")[:, None, :]
    v = W.kv_rows(w, b, hk, 0, S, "v")[:, None, :]
    hs = slice(hk * w.G, (hk + 1) * w.G)
    ref = attention.attend_decode(LAYOUT[w.layout], q[b, hs], k, v, w.alpha, n_recent=w.n_recent)
    U.assert_close_rel(got[b, hs], ref, what=f"{w.name} b{b} hk{hk}")


def test_tiny_q4_0_full():
    U.need_gpu()
    w = W.WORKLOADS["tiny_q4_0_s1024"]
    lens = [w.S]
    cache, table = _cache_for(w, lens, 1)
    seq = _fill(w, cache, table, lens, cpu_pairs=[(0, 0)])
    q = W.queries(w, 0)
    got = _decode(w, cache, table, seq, q, w.S)
    _check_pair(w, got, q, 0, 0, w.S)


def test_llama3_8b_store_one_then_attend_full():
    """32767 cached tokens, store the new token, attend: every head against the oracle."""
    U.need_gpu()
    w = W.WORKLOADS["llama3_8b_q4_0_s32k"]
    S = w.S
    cache, table = _cache_for(w, [S], 1)
    seq = _fill(w, cache, table, [S], cpu_pairs=[(0, hk) for hk in range(w.Hkv)], upto=[S - 1])
    k_new = W.kv_tokens(w, 0, S - 1, S, "k")
    v_new = W.kv_tokens(w, 0, S - 1, S, "v")
    kvq.store(cache, torch.from_numpy(k_new).to(U.DEV), torch.from_numpy(v_new).to(U.DEV),
              torch.from_numpy(U.slots_for(table, 0, S - 1, S, w.page_size)).to(U.DEV),
              torch.zeros(1, dtype=torch.int32, device=U.DEV),
              torch.full((1,), S - 1, dtype=torch.int32, device=U.DEV), seq)
    torch.cuda.synchronize()
    for hk in range(w.Hkv):      # the appended token's bytes
        for which, x in (("k", k_new), ("v", v_new)):
            pay, rec = U.row_bytes(cache, which, table, 0, S - 1, S, hk)
            enc = quant.encode_rows(spec.Q4_0, x[:, hk, :])
            np.testing.assert_array_equal(pay, enc["payload"])
            np.testing.assert_array_equal(rec.reshape(-1), enc["record"].reshape(-1))
    q = W.queries(w, 0)
    got = _decode(w, cache, table, seq, q, S)
    for hk in range(w.Hkv):
        _check_pair(w, got, q, 0, hk, S)


def test_qwen3_hadamard_decode_then_prefill_full():
    """Decode at 8192 with the 64-token window, then a 512-query causal prefill appended at the tail."""
    U.need_gpu()
    w = W.WORKLOADS["qwen3_1p7b_had_s8k"]
    S0, Sq = w.S, w.prefill_q
    S1 = S0 + Sq
    cache, table = _cache_for(w, [S1], 1)
    pairs = [(0, hk) for hk in range(w.Hkv)]
    seq = _fill(w, cache, table, [S0], cpu_pairs=pairs)
    q = W.queries(w, 0)
    got = _decode(w, cache, table, seq, q, S1)
    for hk in range(w.Hkv):
        _check_pair(w, got, q, 0, hk, S0)
    # append the chunk, then attend it causally
    seq = _fill(w, cache, table, [S1], cpu_pairs=pairs)           # rewrites 0..S0 identically, appends the chunk
    qp = W.queries(w, 0, n=Sq, tag=1)[None]                        # [1, Sq, Hq, D]
    qs = torch.tensor([S0], dtype=torch.int32, device=U.DEV)
    bt = torch.from_numpy(table).to(U.DEV)
    qpt = torch.from_numpy(qp).to(U.DEV)
    out = kvq.attend_prefill_causal(cache, qpt, qs, bt, seq, S1, w.alpha)
    out_ns = kvq.attend_prefill_causal(cache, qpt, qs, bt, seq, S1, w.alpha, causal_skip=False)
    torch.cuda.synchronize()
    assert torch.equal(out, out_ns)
    k = W.kv_tokens(w, 0, 0, S1, "k")
    v = W.kv_tokens(w, 0, 0, S1, "v")
    ref = attention.attend_prefill(spec.HAD_INT4, qp[0], k, v, w.alpha, S0, causal=True, n_recent=w.n_recent)
    U.assert_close_rel(out[0].cpu().numpy(), ref, what="prefill")


@pytest.mark.parametrize("B,pairs", [(1, [(0, 0), (0, 5)]), (8, [(3, 2), (7, 7)])])
def test_llama31_70b_asym_128k(B, pairs):
    U.need_gpu()
    w = W.WORKLOADS["llama31_70b_asym_s128k"]
    lens = [w.S] * B
    cache, table = _cache_for(w, lens, B)
    seq = _fill(w, cache, table, lens, cpu_pairs=pairs, gen_seed=B)
    q = np.stack([W.queries(w, b)[0] for b in range(B)])
    got = _decode(w, cache, table, seq, q, w.S)
    assert np.isfinite(got).all()
    for b, hk in pairs:
        _check_pair(w, got, q, b, hk, w.S)


def test_gemma_q6_0_ragged_b16():
    U.need_gpu()
    w = W.WORKLOADS["gemma_q6_0_ragged_b16"]
    lens = [int(n) for n in W.seq_lens(w)]
    pairs = [(int(np.argmax(lens)), 1), (int(np.argmin(lens)), 6), (10, 3)]
    cache, table = _cache_for(w, lens, w.B)
    seq = _fill(w, cache, table, lens, cpu_pairs=pairs, gen_seed=5)
    q = np.stack([W.queries(w, b)[0] for b in range(w.B)])
    got = _decode(w, cache, table, seq, q, max(lens))
    assert np.isfinite(got).all()
    for b, hk in pairs:
        _check_pair(w, got, q, b, hk, lens[b])


def test_qwen3_hadamard_full_precision_prefill_then_store():
    """The same 512-query chunk at 8192 through the full-precision prefill: the chunk's own rows exact,
    the prefix as cached (packed, plus the 64-token window), then the chunk stored bit for bit."""
    U.need_gpu()
    w = W.WORKLOADS["qwen3_1p7b_had_s8k"]
    S0, Sq = w.S, w.prefill_q
    S1 = S0 + Sq
    cache, table = _cache_for(w, [S1], 1)
    pairs = [(0, hk) for hk in range(w.Hkv)]
    _fill(w, cache, table, [S0], cpu_pairs=pairs)
    k = W.kv_tokens(w, 0, 0, S1, "k")
    v = W.kv_tokens(w, 0, 0, S1, "v")
    qp = W.queries(w, 0, n=Sq, tag=1)[None]
    out = kvq.prefill_full_then_store(cache, torch.from_numpy(qp).to(U.DEV), torch.from_numpy(k[None, S0:]).to(U.DEV),
                                      torch.from_numpy(v[None, S0:]).to(U.DEV),
                                      torch.tensor([S0], dtype=torch.int32, device=U.DEV),
                                      torch.from_numpy(table).to(U.DEV), S1, w.alpha)
    torch.cuda.synchronize()
    ref = attention.attend_prefill_full(spec.HAD_INT4, qp[0], k, v, w.alpha, S0, n_recent=w.n_recent)
    U.assert_close_rel(out[0].cpu().numpy(), ref, what="full-precision prefill")
    for hk in (0, 5):
        for which, x in (("k", k), ("v", v)):
            pay, rec = U.row_bytes(cache, which, table, 0, S0, S1, hk)
            enc = quant.encode_rows(spec.HAD_INT4, x[S0:, hk, :])
            np.testing.assert_array_equal(pay, enc["payload"])
            np.testing.assert_array_equal(rec.reshape(-1), enc["record"].reshape(-1))


@pytest.mark.parametrize("mode", ["q8_0", "float_q"])
def test_llama31_70b_128k_next_modes(mode):
    """The 128K Llama-3.1-70B shape in the q8_0 layout, and in the float-query mode on its own layout;
    sampled (batch row, kv head) pairs against the oracle."""
    import dataclasses
    U.need_gpu()
    w = W.WORKLOADS["llama31_70b_asym_s128k"]
    if mode == "q8_0":
        w = dataclasses.replace(w, layout="q8_0")
    B, pairs = 2, [(0, 3), (1, 6)]
    lens = [w.S] * B
    cache, table = _cache_for(w, lens, B)
    seq = _fill(w, cache, table, lens, cpu_pairs=pairs, gen_seed=11)
    q = np.stack([W.queries(w, b)[0] for b in range(B)])
    fq = mode == "float_q"
    out = kvq.attend_decode(cache, torch.from_numpy(q).to(U.DEV), torch.from_numpy(table).to(U.DEV), seq, w.S,
                            w.alpha, chunk_tokens=w.chunk_tokens, float_q=fq)
    torch.cuda.synchronize()
    got = out.cpu().numpy()
    assert np.isfinite(got).all()
    for b, hk in pairs:
        kk = W.kv_rows(w, b, hk, 0, w.S, "k")[:, None, :]
        vv = W.kv_rows(w, b, hk, 0, w.S, "v")[:, None, :]
        hs = slice(hk * w.G, (hk + 1) * w.G)
        ref = attention.attend_decode(LAYOUT[w.layout], q[b, hs], kk, vv, w.alpha, float_q=fq)
        U.assert_close_rel(got[b, hs], ref, what=f"{mode} b{b} hk{hk}")
