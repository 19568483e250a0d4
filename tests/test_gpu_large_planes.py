"""Payload planes larger than 4 GiB: the kernels' byte offsets are 64-bit.

A q8_0 cache (128 payload bytes per token and kv head at D = 128) of 1.2 M pages of 16 tokens and two kv
heads holds 4.9 GB in each payload plane.  The rows live in the last pages of the planes, so every access
of the store (token-slot and chunk forms), the decode and the causal prefill lies past the 4 GiB mark.
Stored bytes are compared bit-exact with the oracle's encoding, outputs with the oracle's attention
(max|diff| <= 2e-3 * max|o_ref|).  Device memory: about 10.5 GB.
"""

import math

import numpy as np
import pytest
import torch

import quantized_kv_cache_store_amd as kvq
from oracle import attention, quant, spec
import gpu_util as U

pytestmark = pytest.mark.gpu

NUM_PAGES, PAGE, HKV, D, G, N_RECENT = 1_200_000, 16, 2, 128, 4, 16


def test_store_decode_prefill_past_4_gib():
    U.need_gpu()
    layout = spec.Q8_0
    rng = np.random.default_rng(4242)
    lens = [700, 333]
    rows_k = [rng.standard_normal((n, HKV, D)).astype(np.float32) for n in lens]
    rows_v = [rng.standard_normal((n, HKV, D)).astype(np.float32) for n in lens]
    cache = kvq.KvqCache(layout, D, HKV, NUM_PAGES, PAGE, n_recent=N_RECENT, max_batch=2, device=U.DEV)
    assert cache.k_payload.numel() > (1 << 32)

    # the rows' pages: the last ones of the planes, shuffled
    need = [(n + PAGE - 1) // PAGE for n in lens]
    phys = NUM_PAGES - sum(need) + rng.permutation(sum(need))
    table = np.zeros((2, max(need)), dtype=np.int32)
    table[0, :need[0]] = phys[:need[0]]
    table[1, :need[1]] = phys[need[0]:]
    table[1, need[1]:] = phys[need[0]]
    assert int(table.min()) * HKV * PAGE * 128 > (1 << 32)
    bt = torch.from_numpy(table).to(U.DEV)

    # tokens [0, n - 33) of each row through the token-slot form, the last 33 through the chunk form
    tail = 33
    seq_head = torch.tensor([n - tail for n in lens], dtype=torch.int32, device=U.DEV)
    for b, n in enumerate(lens):
        t1 = n - tail
        sl = torch.from_numpy(U.slots_for(table, b, 0, t1, PAGE)).to(U.DEV)
        kvq.store(cache, torch.from_numpy(np.ascontiguousarray(rows_k[b][:t1])).to(U.DEV),
                  torch.from_numpy(np.ascontiguousarray(rows_v[b][:t1])).to(U.DEV), sl,
                  torch.full((t1,), b, dtype=torch.int32, device=U.DEV),
                  torch.arange(t1, dtype=torch.int32, device=U.DEV), seq_head)
    kc = torch.from_numpy(np.stack([r[-tail:] for r in rows_k])).to(U.DEV)
    vc = torch.from_numpy(np.stack([r[-tail:] for r in rows_v])).to(U.DEV)
    qs = torch.tensor([n - tail for n in lens], dtype=torch.int32, device=U.DEV)
    kvq.store_chunk(cache, kc, vc, qs, bt, max(lens))
    torch.cuda.synchronize()

    for b, n in enumerate(lens):
        for h in range(HKV):
            for which, rows in (("k", rows_k[b]), ("v", rows_v[b])):
                e = quant.encode_rows(layout, rows[:, h, :])
                pay, rec = U.row_bytes(cache, which, table, b, 0, n, h)
                np.testing.assert_array_equal(pay, e["payload"], err_msg=f"payload b{b} h{h} {which}")
                np.testing.assert_array_equal(rec, e["record"], err_msg=f"record b{b} h{h} {which}")

    seq = torch.tensor(lens, dtype=torch.int32, device=U.DEV)
    alpha = 1.0 / math.sqrt(D)
    for g in (G, 12):   # 8-row tiles (direct-to-LDS ring) and 16-row tiles (register ring)
        q = rng.standard_normal((2, HKV * g, D)).astype(np.float32)
        got = kvq.attend_decode(cache, torch.from_numpy(q).to(U.DEV), bt, seq, max(lens), alpha, chunk_tokens=256)
        torch.cuda.synchronize()
        ref = np.stack([attention.attend_decode(layout, q[b], rows_k[b], rows_v[b], alpha, n_recent=N_RECENT)
                        for b in range(2)])
        U.assert_close_rel(got.cpu().numpy(), ref, what=f"decode G={g}")

    qp = rng.standard_normal((2, tail, HKV * G, D)).astype(np.float32)
    got = kvq.attend_prefill_causal(cache, torch.from_numpy(qp).to(U.DEV), qs, bt, seq, max(lens), alpha)
    torch.cuda.synchronize()
    ref = np.stack([attention.attend_prefill(layout, qp[b], rows_k[b], rows_v[b], alpha, lens[b] - tail,
                                             causal=True, n_recent=N_RECENT) for b in range(2)])
    U.assert_close_rel(got.cpu().numpy(), ref, what="prefill")
    del cache
    torch.cuda.empty_cache()
