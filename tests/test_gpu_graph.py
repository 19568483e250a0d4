"""The decode step (store one token, partial, reduce) and the causal prefill captured into HIP graphs.

The library launches on the caller's stream, allocates nothing and issues no memset, so its calls can
be captured.  Each graph is replayed several times with eager work and synchronisations in between,
and every replay must give the bits of the eager call (the kernels are deterministic); the eager
output itself is checked against the oracle.
"""

import math

import numpy as np
import pytest
import torch

import quantized_kv_cache_store_amd as kvq
from oracle import attention, spec
import gpu_util as U

pytestmark = pytest.mark.gpu


def _capture(fn):
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            fn()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    return g


@pytest.mark.parametrize("layout", [spec.ASYM_G32, spec.HAD_INT4])
def test_decode_step_graph_replays(layout):
    U.need_gpu()
    rng = np.random.default_rng(77 + layout)
    D, Hkv, G, n_recent = 128, 2, 8, 16
    lens = [900, 333]
    rows_k = [rng.standard_normal((n, Hkv, D)).astype(np.float32) for n in lens]
    rows_v = [rng.standard_normal((n, Hkv, D)).astype(np.float32) for n in lens]
    # the cache holds all but the last token of each row; the step stores that token, then attends
    head_k = [r[:-1] for r in rows_k]
    head_v = [r[:-1] for r in rows_v]
    cache, bt, _, table = U.build_cache(layout, D, Hkv, head_k, head_v, n_recent=n_recent)
    B, Hq, S = len(lens), Hkv * G, max(lens)
    seq = torch.tensor(lens, dtype=torch.int32, device=U.DEV)
    k_new = torch.from_numpy(np.stack([r[-1] for r in rows_k])).to(U.DEV)
    v_new = torch.from_numpy(np.stack([r[-1] for r in rows_v])).to(U.DEV)
    slot = torch.from_numpy(np.concatenate([U.slots_for(table, b, n - 1, n, 16) for b, n in enumerate(lens)])).to(U.DEV)
    bidx = torch.arange(B, dtype=torch.int32, device=U.DEV)
    pos = (seq - 1).to(torch.int32)
    q = rng.standard_normal((B, Hq, D)).astype(np.float32)
    qt = torch.from_numpy(q).to(U.DEV)
    alpha = 1.0 / math.sqrt(D)
    chunk = 256
    ws = torch.empty(kvq.decode_workspace_bytes(B, Hq, D, S, chunk), dtype=torch.uint8, device=U.DEV)
    out = torch.empty((B, Hq, D), dtype=torch.float32, device=U.DEV)

    def step():
        kvq.store(cache, k_new, v_new, slot, bidx, pos, seq)
        kvq.attend_decode_partial(cache, qt, bt, seq, S, alpha, chunk, ws)
        kvq.attend_decode_reduce(cache, out, seq, S, chunk, ws)

    step()
    torch.cuda.synchronize()
    eager = out.clone()
    ref = np.stack([attention.attend_decode(layout, q[b], rows_k[b], rows_v[b], alpha, n_recent=n_recent)
                    for b in range(B)])
    U.assert_close_rel(eager.cpu().numpy(), ref)

    g = _capture(step)
    for i in range(3):
        out.fill_(float("nan"))
        ws.fill_(0xA5)          # stale workspace contents must not matter
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, eager), f"replay {i} differs from the eager step"
        _ = (qt * 2.0).sum().item()   # eager work between replays


def test_prefill_graph_replays():
    U.need_gpu()
    rng = np.random.default_rng(91)
    layout, D, Hkv, G, n_q = spec.Q4_0, 128, 2, 2, 40
    lens = [700, 200]
    rows_k = [rng.standard_normal((n, Hkv, D)).astype(np.float32) for n in lens]
    rows_v = [rng.standard_normal((n, Hkv, D)).astype(np.float32) for n in lens]
    cache, bt, seq, _ = U.build_cache(layout, D, Hkv, rows_k, rows_v, n_recent=8)
    qs = torch.tensor([n - n_q for n in lens], dtype=torch.int32, device=U.DEV)
    q = rng.standard_normal((len(lens), n_q, Hkv * G, D)).astype(np.float32)
    qt = torch.from_numpy(q).to(U.DEV)
    alpha = 1.0 / math.sqrt(D)
    S = max(lens)
    ws = torch.empty(kvq.prefill_workspace_bytes(len(lens), n_q, Hkv * G, D, S), dtype=torch.uint8, device=U.DEV)
    out = torch.empty_like(qt)

    def call():
        kvq.attend_prefill_causal(cache, qt, qs, bt, seq, S, alpha, out=out, workspace=ws)

    call()
    torch.cuda.synchronize()
    eager = out.clone()
    ref = np.stack([attention.attend_prefill(layout, q[b], rows_k[b], rows_v[b], alpha, lens[b] - n_q,
                                             causal=True, n_recent=8) for b in range(len(lens))])
    U.assert_close_rel(eager.cpu().numpy(), ref)

    g = _capture(call)
    for i in range(3):
        out.fill_(float("nan"))
        ws.fill_(0x5A)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, eager), f"replay {i} differs from the eager call"
        _ = (qt + 1.0).abs().max().item()
