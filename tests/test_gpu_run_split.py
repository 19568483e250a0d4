"""The decode's run length chosen per call from the rows' lengths (batches whose blocks take several
rounds of the chip): outputs against the oracle on sampled rows, and the partial slots the kernels
wrote against the run length kvq_decode_split_lengths reports for the same lengths."""

import math

import numpy as np
import pytest
import torch

import quantized_kv_cache_store_amd as kvq
from oracle import attention, spec
import gpu_util as U

pytestmark = pytest.mark.gpu

# layout, head_dim, kv heads, query heads per kv head, rows, length range, seed
CASES = [
    (spec.Q4_0, 128, 8, 2, 80, (64, 9000), 0),
    (spec.Q6_0, 256, 2, 2, 96, (64, 20000), 0),
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: f"L{c[0]}-D{c[1]}-B{c[4]}")
def test_run_length_from_the_rows(case):
    U.need_gpu()
    layout, D, Hkv, G, B, (lo, hi), seed = case
    rng = np.random.default_rng(seed)
    lens = [int(n) for n in rng.integers(lo, hi, size=B)]
    rows_k = [rng.standard_normal((n, Hkv, D)).astype(np.float32) for n in lens]
    rows_v = [rng.standard_normal((n, Hkv, D)).astype(np.float32) for n in lens]
    Hq, S, chunk = Hkv * G, max(lens), 512
    q = rng.standard_normal((B, Hq, D)).astype(np.float32)
    qt = torch.from_numpy(q).to(U.DEV)
    alpha = 1.0 / math.sqrt(D)
    cache, bt, seq, _ = U.build_cache(layout, D, Hkv, rows_k, rows_v)
    span, part = kvq.decode_split_lengths(cache, Hq, lens, S, chunk)
    assert span < 4 * chunk, "the case should take runs shorter than four chunks"

    out = kvq.attend_decode(cache, qt, bt, seq, S, alpha, chunk_tokens=chunk).cpu().numpy()
    for b in sorted({0, 1, int(np.argmax(lens)), int(np.argmin(lens)), B - 1}):
        ref = attention.attend_decode(layout, q[b], rows_k[b], rows_v[b], alpha)
        U.assert_close_rel(out[b], ref, what=f"row {b} ({lens[b]} tokens)")

    # the partial phase alone, on a workspace of NaN: a row of n tokens fills ceil(n / part) slots
    ws = torch.full((kvq.decode_workspace_bytes(B, Hq, D, S, chunk),), 0xFF, dtype=torch.uint8, device=U.DEV)
    kvq.attend_decode_partial(cache, qt, bt, seq, S, alpha, chunk, ws)
    torch.cuda.synchronize()
    nc1 = -(-S // (6 * chunk)) + 1          # slots of the shortest runs (1.5 chunks), which size the grid
    f = ws.view(torch.float32)[:B * Hq * nc1 * (D + 4)].view(B, Hq, nc1, D + 4).cpu().numpy()
    written = (~np.isnan(f[:, :, :, D])).sum(axis=2)
    expect = np.array([-(-n // part) for n in lens])[:, None].repeat(Hq, axis=1)
    np.testing.assert_array_equal(written, expect)
