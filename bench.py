"""Decode-attention bench on one MI355X: packed-KV GB/s and us/layer at 128K context.

Workload: Llama-3.1-70B-shaped attention layer (64 query heads, 8 kv heads,
head_dim 128), per-group asymmetric int4 cache (g = 32, fp16 scale + zero),
131072 cached tokens per row, batch 8, split-K chunks of 512 tokens, K/V drawn
as Student-t(3) / sqrt(3) on the device.

One step = the whole hot path for one layer: quantize-on-append of the new
token of every row (kvq_store), then the split-K decode partial and the reduce
(kvq_attend_decode_partial + kvq_attend_decode_reduce).  Steps walk L distinct
layer caches (L * packed bytes >= 2.5 GB) so the 256 MB Infinity Cache cannot
serve the reads.  Timed with HIP events on the launch stream after warm-up.

Prints one JSON line.  ``--gpus`` above 1 is refused: the benchmark runs on one GPU.
"""

import argparse
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "decode-attention packed-KV GB/s (% HBM peak) and µs/layer at 128K ctx"
HBM_PEAK_GBS = 8000.0


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=40)
    p.add_argument("--warmup", type=int, default=5)
    p.add_argument("--batch", type=int, default=8)
    p.add_argument("--chunk", type=int, default=512)
    p.add_argument("--layers", type=int, default=0, help="layer caches walked (0: enough for >= 2.5 GB)")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--cpu-kv-heads", type=int, default=8, help="kv heads of one row timed on the oracle")
    p.add_argument("--batch1", action="store_true", help="also time batch 1 (reported under extra)")
    p.add_argument("--no-prefill", action="store_true", help="skip the causal prefill timing")
    p.add_argument("--configs", action="store_true",
                   help="also time one decode step of each workload at its own shape (reported under extra)")
    p.add_argument("--copy-calibration", action="store_true",
                   help="only run a 1 GiB device-to-device copy 10 times (HBM counter calibration) and exit")
    return p.parse_args()


TRAFFIC_PROFILE = os.path.join(ROOT, "profiles", "attend_partial_asym_int4_g32_llama31_70b_s128k_b8_hbm_traffic.md")
KERNEL_SOURCES = [os.path.join(ROOT, "quantized_kv_cache_store_amd", "csrc", f)
                  for f in ("kvq_attend.hip", "kvq_attend_common.h", "kvq_internal.h")]


def measured_traffic():
    """HBM bytes per partial launch from the committed FETCH_SIZE/WRITE_SIZE summary (copy-calibrated),
    or None when the kernel sources changed since the counters were taken."""
    import hashlib
    import re
    try:
        text = open(TRAFFIC_PROFILE).read()
    except OSError:
        return None
    h = hashlib.sha256()
    for f in KERNEL_SOURCES:
        h.update(open(f, "rb").read())
    m_sha = re.search(r"^source_sha256: (\w+)", text, re.M)
    m_val = re.search(r"^traffic_bytes_per_launch: (\S+)", text, re.M)
    if not m_sha or not m_val or m_sha.group(1) != h.hexdigest():
        return None
    return float(m_val.group(1))


def copy_calibration():
    """A plain copy of known size: 1 GiB read + 1 GiB written per launch, 10 launches."""
    import torch
    n = 1 << 30
    src = torch.empty(n, dtype=torch.uint8, device="cuda:0")
    src.fill_(1)
    dst = torch.empty_like(src)
    for _ in range(10):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_calibration_bytes": n, "launches": 10}), flush=True)


def time_prefill(steps, warmup, dev, seed=2):
    """Causal prefill of the Hadamard workload: 512 queries appended at 8192 (cache of 8704 tokens)."""
    import torch
    import quantized_kv_cache_store_amd as kvq
    import workloads as W

    w = W.WORKLOADS["qwen3_1p7b_had_s8k"]
    gen = torch.Generator(device=dev)
    gen.manual_seed(seed)
    S0, Sq = w.S, w.prefill_q
    S1 = S0 + Sq
    ps = w.page_size
    npages = (S1 + ps - 1) // ps
    cache = kvq.KvqCache(w.layout, w.D, w.Hkv, npages, ps, n_recent=w.n_recent, max_batch=1, device=dev)
    table = torch.arange(npages, dtype=torch.int32, device=dev).reshape(1, npages)
    seq = torch.full((1,), S1, dtype=torch.int32, device=dev)
    k = W.kv_tokens_device(w, S1, "k", gen, dev)
    v = W.kv_tokens_device(w, S1, "v", gen, dev)
    pos = torch.arange(S1, dtype=torch.int32, device=dev)
    kvq.store(cache, k, v, pos.clone(), torch.zeros(S1, dtype=torch.int32, device=dev), pos, seq)
    q = torch.randn((1, Sq, w.Hq, w.D), generator=gen, device=dev, dtype=torch.float32)
    qs = torch.full((1,), S0, dtype=torch.int32, device=dev)
    out = torch.empty_like(q)
    ws = torch.empty(kvq.prefill_workspace_bytes(1, Sq, w.Hq, w.D, S1), dtype=torch.uint8, device=dev)
    for _ in range(warmup):
        kvq.attend_prefill_causal(cache, q, qs, table, seq, S1, w.alpha, out=out, workspace=ws)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(steps):
        kvq.attend_prefill_causal(cache, q, qs, table, seq, S1, w.alpha, out=out, workspace=ws)
    e1.record()
    torch.cuda.synchronize()
    us = e0.elapsed_time(e1) * 1e3 / steps
    assert torch.isfinite(out).all(), "non-finite prefill output"
    # visible (query, token) pairs per query head: query i sees S0 + i + 1 tokens
    pairs = sum(S0 + i + 1 for i in range(Sq)) * w.Hq
    ops = 2.0 * pairs * w.D * 2                   # Q K^T (int8 MACs) + P V (f16 MACs), 2 ops per MAC
    t_min = 2.0 * pairs * w.D / 5.0e15 + 2.0 * pairs * w.D / 2.5e15   # int8 at 5.0 POP/s, f16 at 2.5 PFLOP/s
    return dict(workload=w.name, n_q=Sq, q_start=S0, seq_len=S1, us=round(us, 2), visible_pairs=pairs,
                achieved_tops=round(ops / (us * 1e-6) / 1e12, 1), roofline_us=round(t_min * 1e6, 2),
                frac=round(t_min * 1e6 / us, 4),
                bound="mfma (int8 Q K^T at 5.0 POP/s + f16 P V at 2.5 PFLOP/s)")


def time_prefill_full(steps, warmup, dev, q_start, n_q, seed=3):
    """Full-precision prefill then store, Hadamard workload shape: n_q queries at q_start (the prefix
    stored first), the chunk's own tokens exact, then the chunk quantised into the cache."""
    import torch
    import quantized_kv_cache_store_amd as kvq
    import workloads as W

    w = W.WORKLOADS["qwen3_1p7b_had_s8k"]
    gen = torch.Generator(device=dev)
    gen.manual_seed(seed)
    S1 = q_start + n_q
    ps = w.page_size
    npages = (S1 + ps - 1) // ps
    cache = kvq.KvqCache(w.layout, w.D, w.Hkv, npages, ps, n_recent=w.n_recent, max_batch=1, device=dev)
    table = torch.arange(npages, dtype=torch.int32, device=dev).reshape(1, npages)
    qs = torch.full((1,), q_start, dtype=torch.int32, device=dev)
    if q_start > 0:
        k = W.kv_tokens_device(w, q_start, "k", gen, dev)
        v = W.kv_tokens_device(w, q_start, "v", gen, dev)
        pos = torch.arange(q_start, dtype=torch.int32, device=dev)
        kvq.store(cache, k, v, pos.clone(), torch.zeros(q_start, dtype=torch.int32, device=dev), pos, qs)
    kc = W.kv_tokens_device(w, n_q, "k", gen, dev).reshape(1, n_q, w.Hkv, w.D)
    vc = W.kv_tokens_device(w, n_q, "v", gen, dev).reshape(1, n_q, w.Hkv, w.D)
    q = torch.randn((1, n_q, w.Hq, w.D), generator=gen, device=dev, dtype=torch.float32)
    out = torch.empty_like(q)
    ws = torch.empty(kvq.prefill_workspace_bytes(1, n_q, w.Hq, w.D, S1), dtype=torch.uint8, device=dev)
    # the same chunk is stored at the same positions on every call
    for _ in range(warmup):
        kvq.prefill_full_then_store(cache, q, kc, vc, qs, table, S1, w.alpha, out=out, workspace=ws)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(steps):
        kvq.prefill_full_then_store(cache, q, kc, vc, qs, table, S1, w.alpha, out=out, workspace=ws)
    e1.record()
    torch.cuda.synchronize()
    us = e0.elapsed_time(e1) * 1e3 / steps
    assert torch.isfinite(out).all(), "non-finite prefill output"
    prefix_pairs = q_start * n_q * w.Hq              # every query sees the whole prefix
    chunk_pairs = n_q * (n_q + 1) // 2 * w.Hq        # causal within the chunk
    t_min = (2.0 * prefix_pairs * w.D / 5.0e15 + 2.0 * prefix_pairs * w.D / 2.5e15   # int8 Q K^T + f16 P V
             + 2.0 * 2.0 * chunk_pairs * w.D / 157.3e12)                              # f32 Q K^T + P V (window MFMA)
    return dict(workload=w.name, n_q=n_q, q_start=q_start, us=round(us, 2), prefix_pairs=prefix_pairs,
                chunk_pairs=chunk_pairs, roofline_us=round(t_min * 1e6, 2), frac=round(t_min * 1e6 / us, 4),
                bound="mfma (prefix: int8 + f16; chunk rows: f32 at 157.3 TFLOP/s)")


def time_store(steps, warmup, dev, seed=1):
    """kvq_store of one new token per kv head into the Llama-3-8B-shaped q4_0 cache (32768 slots)."""
    import torch
    import quantized_kv_cache_store_amd as kvq
    import workloads as W

    w = W.WORKLOADS["llama3_8b_q4_0_s32k"]
    gen = torch.Generator(device=dev)
    gen.manual_seed(seed)
    npages = w.S // w.page_size
    cache = kvq.KvqCache(w.layout, w.D, w.Hkv, npages, w.page_size, device=dev)
    k = W.kv_tokens_device(w, 1, "k", gen, dev)
    v = W.kv_tokens_device(w, 1, "v", gen, dev)
    slot = torch.full((1,), w.S - 1, dtype=torch.int32, device=dev)
    for _ in range(warmup):
        kvq.store(cache, k, v, slot)
    torch.cuda.synchronize()
    # A one-token store takes a few microseconds on the GPU, less than one host launch through the
    # binding, so launches are captured into a graph (no memset nodes: the store issues none) and the
    # graph replays are timed.
    per_graph = 64
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            for _ in range(per_graph):
                kvq.store(cache, k, v, slot)
    torch.cuda.current_stream().wait_stream(s)
    g.replay()
    torch.cuda.synchronize()
    reps = max(1, steps // 4)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        g.replay()
    e1.record()
    torch.cuda.synchronize()
    return dict(workload=w.name, tokens=1, us=round(e0.elapsed_time(e1) * 1e3 / (reps * per_graph), 2),
                timing="graph of 64 launches", bytes_in=2 * w.Hkv * w.D * 4, bytes_out=2 * w.Hkv * (64 + 8))


def build_layers(w, B, L, dev, gen):
    import torch
    import quantized_kv_cache_store_amd as kvq
    import workloads as W

    S = w.S
    ps = w.page_size
    ppr = S // ps
    table = torch.arange(B * ppr, dtype=torch.int32, device=dev).reshape(B, ppr)
    seq_full = torch.full((B,), S, dtype=torch.int32, device=dev)
    fill = 16384
    caches = []
    for _ in range(L):
        c = kvq.KvqCache(w.layout, w.D, w.Hkv, B * ppr, ps, device=dev)
        for b in range(B):
            for t0 in range(0, S - 1, fill):
                t1 = min(S - 1, t0 + fill)
                k = W.kv_tokens_device(w, t1 - t0, "k", gen, dev)
                v = W.kv_tokens_device(w, t1 - t0, "v", gen, dev)
                # row b owns physical pages b*ppr .. b*ppr+ppr-1, so slot = b*S + t
                slot = (b * S + torch.arange(t0, t1, device=dev, dtype=torch.int32)).to(torch.int32)
                kvq.store(c, k, v, slot)
        caches.append(c)
    torch.cuda.synchronize()
    return caches, table, seq_full


def time_decode(w, B, chunk, steps, warmup, layers, dev, seed):
    import torch
    import quantized_kv_cache_store_amd as kvq
    import workloads as W

    gen = torch.Generator(device=dev)
    gen.manual_seed(seed)
    S = w.S
    lay = kvq.LAYOUT_IDS[w.layout]
    bytes_layer = B * w.Hkv * S * 2 * (kvq.load().kvq_payload_bytes(lay, w.D) + kvq.load().kvq_scale_bytes(lay, w.D))
    L = layers or max(2, math.ceil(2.5e9 / bytes_layer))
    caches, table, seq = build_layers(w, B, L, dev, gen)
    q = torch.randn((B, w.Hq, w.D), generator=gen, device=dev, dtype=torch.float32)
    k_new = W.kv_tokens_device(w, B, "k", gen, dev)
    v_new = W.kv_tokens_device(w, B, "v", gen, dev)
    slot_new = (torch.arange(B, device=dev, dtype=torch.int32) * S + (S - 1)).to(torch.int32)
    out = torch.empty((B, w.Hq, w.D), dtype=torch.float32, device=dev)
    ws = torch.empty(kvq.decode_workspace_bytes(B, w.Hq, w.D, S, chunk), dtype=torch.uint8, device=dev)

    def step(i, ev=None):
        c = caches[i % L]
        kvq.store(c, k_new, v_new, slot_new)
        if ev is not None:
            ev[0].record()
        kvq.attend_decode_partial(c, q, table, seq, S, w.alpha, chunk, ws)
        if ev is not None:
            ev[1].record()
        kvq.attend_decode_reduce(c, out, seq, S, chunk, ws)

    for i in range(warmup):
        step(i)
    torch.cuda.synchronize()
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    wall0 = time.perf_counter()
    t0.record()
    for i in range(steps):
        step(warmup + i, evs[i])
    t1.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    total_ms = t0.elapsed_time(t1)
    part_ms = [a.elapsed_time(b) for a, b in evs]
    assert torch.isfinite(out).all(), "non-finite attention output"
    # read probe: the same layers' planes (the algorithmic bytes of one launch) read once each
    planes = lambda c: (c.k_payload, c.v_payload, c.k_scale, c.v_scale)
    for i in range(warmup):
        kvq.debug_stream_read(planes(caches[i % L]))
    torch.cuda.synchronize()
    p0, p1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    p0.record()
    for i in range(steps):
        kvq.debug_stream_read(planes(caches[i % L]))
    p1.record()
    torch.cuda.synchronize()
    probe_us = p0.elapsed_time(p1) * 1e3 / steps
    del caches
    torch.cuda.empty_cache()
    srt = sorted(part_ms)
    return dict(bytes_layer=bytes_layer, layers=L, ms_per_step=total_ms / steps, wall_s=wall,
                partial_ms_mean=sum(part_ms) / len(part_ms), partial_ms_min=min(part_ms),
                partial_ms_median=srt[len(srt) // 2], partial_ms_p10=srt[len(srt) // 10],
                partial_ms_p90=srt[min(len(srt) - 1, (9 * len(srt)) // 10)], probe_us=probe_us)


# Layer caches walked per configuration so that the walk spans about 1 GiB or more (the tiny case stays
# cache-resident: it is launch-bound and reported in microseconds only).
CONFIG_LAYERS = {"tiny_q4_0_s1024": 1, "llama3_8b_q4_0_s32k": 32, "qwen3_1p7b_had_s8k": 128,
                 "llama31_70b_asym_s128k": 2, "gemma_q6_0_ragged_b16": 2}


def time_config(w, steps, warmup, dev, seed=5):
    """One decode step of a workload at its own shape: store one token per row at its last position,
    then the split-K partial and the reduce, walking CONFIG_LAYERS[w.name] layer caches."""
    import numpy as np
    import torch
    import quantized_kv_cache_store_amd as kvq
    import workloads as W

    gen = torch.Generator(device=dev)
    gen.manual_seed(seed)
    lens = [int(n) for n in W.seq_lens(w)]
    B, S = len(lens), max(lens)
    table_np, total = W.block_tables(w, lens)
    for b in range(B):   # unused entries: a page of the row (never read below its length)
        table_np[b][table_np[b] < 0] = table_np[b, 0]
    ps = w.page_size
    table = torch.from_numpy(table_np).to(dev)
    seq = torch.tensor(lens, dtype=torch.int32, device=dev)
    lay = kvq.LAYOUT_IDS[w.layout]
    per_tok = 2 * (kvq.load().kvq_payload_bytes(lay, w.D) + kvq.load().kvq_scale_bytes(lay, w.D))
    window = sum(min(n, w.n_recent) for n in lens) * w.Hkv * 2 * w.D * 4
    packed = sum(max(0, n - w.n_recent) if w.n_recent else n for n in lens) * w.Hkv * per_tok
    L = CONFIG_LAYERS.get(w.name, 2)

    def slots(b, t0, t1):
        t = torch.arange(t0, t1, device=dev, dtype=torch.int64)
        return (table[b, t // ps].to(torch.int64) * ps + t % ps).to(torch.int32)

    caches = []
    fill = 16384
    for _ in range(L):
        c = kvq.KvqCache(w.layout, w.D, w.Hkv, total, ps, n_recent=w.n_recent, max_batch=B, device=dev)
        for b, n in enumerate(lens):
            for t0 in range(0, n - 1, fill):
                t1 = min(n - 1, t0 + fill)
                k = W.kv_tokens_device(w, t1 - t0, "k", gen, dev)
                v = W.kv_tokens_device(w, t1 - t0, "v", gen, dev)
                kvq.store(c, k, v, slots(b, t0, t1), torch.full((t1 - t0,), b, dtype=torch.int32, device=dev),
                          torch.arange(t0, t1, dtype=torch.int32, device=dev), seq)
        caches.append(c)
    q = torch.randn((B, w.Hq, w.D), generator=gen, device=dev, dtype=torch.float32)
    k_new = W.kv_tokens_device(w, B, "k", gen, dev)
    v_new = W.kv_tokens_device(w, B, "v", gen, dev)
    slot_new = torch.cat([slots(b, n - 1, n) for b, n in enumerate(lens)])
    bidx = torch.arange(B, dtype=torch.int32, device=dev)
    pos_new = (seq - 1).to(torch.int32)
    out = torch.empty((B, w.Hq, w.D), dtype=torch.float32, device=dev)
    ws = torch.empty(kvq.decode_workspace_bytes(B, w.Hq, w.D, S, w.chunk_tokens), dtype=torch.uint8, device=dev)

    def step(i, partial_only=False):
        c = caches[i % L]
        if not partial_only:
            kvq.store(c, k_new, v_new, slot_new, bidx, pos_new, seq)
        kvq.attend_decode_partial(c, q, table, seq, S, w.alpha, w.chunk_tokens, ws)
        if not partial_only:
            kvq.attend_decode_reduce(c, out, seq, S, w.chunk_tokens, ws)

    for i in range(warmup):
        step(i)
    torch.cuda.synchronize()
    # The small shapes take less GPU time per step than the binding's host launches, so the steps
    # are captured into graphs (the decode issues no memset nodes) and the replays are timed: one graph
    # of whole steps and one of the partial kernel alone, each walking the layer caches.
    per_graph = max(L, 16)

    def capture(partial_only):
        g = torch.cuda.CUDAGraph()
        st = torch.cuda.Stream()
        st.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(st):
            with torch.cuda.graph(g, stream=st):
                for i in range(per_graph):
                    step(i, partial_only)
        torch.cuda.current_stream().wait_stream(st)
        g.replay()
        torch.cuda.synchronize()
        return g

    def timed(g):
        reps = max(2, steps // 4)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(reps):
            g.replay()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) * 1e3 / (reps * per_graph)

    us = timed(capture(False))
    assert torch.isfinite(out).all(), "non-finite attention output"
    part_us = timed(capture(True))
    del caches
    torch.cuda.empty_cache()
    return dict(workload=w.name, layout=w.layout, batch=B, seq_len_max=S, q_heads=w.Hq, kv_heads=w.Hkv,
                head_dim=w.D, n_recent=w.n_recent, layers_walked=L, bytes_per_layer=packed + window,
                us_per_layer=round(us, 2), partial_us=round(part_us, 2), timing=f"graphs of {per_graph} steps",
                gbs=round((packed + window) / (us * 1e-6) / 1e9, 1),
                ideal_us_at_8tbs=round((packed + window) / 8e12 * 1e6, 2))


def cpu_baseline(w, kv_heads):
    """The oracle (as it stands) on one row, ``kv_heads`` kv heads, the full 131072 tokens."""
    import numpy as np
    import workloads as W
    from oracle import attention, spec

    try:
        from threadpoolctl import threadpool_info
        blas = max([i.get("num_threads", 1) for i in threadpool_info()] + [1])
    except Exception:  # pragma: no cover
        blas = 1
    S = w.S
    k = np.stack([W.kv_rows(w, 0, hk, 0, S, "k") for hk in range(kv_heads)], axis=1)
    v = np.stack([W.kv_rows(w, 0, hk, 0, S, "v") for hk in range(kv_heads)], axis=1)
    q = W.queries(w, 0)[0][: kv_heads * w.G]
    t = time.perf_counter()
    attention.attend_decode(spec.ASYM_G32, q, k, v, w.alpha)
    dt = time.perf_counter() - t
    packed = kv_heads * S * 2 * 80
    return dict(value=packed / dt / 1e9, unit="GB/s", cores=blas, kind="oracle",
                sample=f"one row, {kv_heads} of 8 kv heads ({kv_heads * w.G} query heads), {S} tokens: "
                       f"float64 numpy encode + attend of {packed} packed bytes in {dt:.2f} s "
                       f"(elementwise numpy on 1 thread, BLAS on {blas})")


def main():
    a = parse()
    if a.copy_calibration:
        copy_calibration()
        return
    if a.gpus != 1:
        print(json.dumps({"error": "the benchmark runs on one GPU; --gpus above 1 is not supported",
                          "n_gpus": a.gpus}))
        sys.exit(2)
    import torch
    import workloads as W

    w = W.WORKLOADS["llama31_70b_asym_s128k"]
    dev = torch.device("cuda:0")
    r = time_decode(w, a.batch, a.chunk, a.steps, a.warmup, a.layers, dev, seed=3)
    extra = {}
    if a.batch1:
        r1 = time_decode(w, 1, a.chunk, a.steps, a.warmup, 0, dev, seed=4)
        extra["batch1"] = dict(us_per_layer=r1["ms_per_step"] * 1e3,
                               packed_gbs=r1["bytes_layer"] / (r1["ms_per_step"] * 1e-3) / 1e9,
                               partial_us=r1["partial_ms_mean"] * 1e3, layers_walked=r1["layers"])
    if not a.no_prefill:
        extra["prefill"] = time_prefill(max(a.steps, 20), a.warmup, dev)
        extra["prefill_full_precision"] = [time_prefill_full(max(a.steps, 20), a.warmup, dev, qs, nq)
                                           for qs, nq in ((8192, 512), (0, 512), (0, 4096))]
        extra["store"] = time_store(max(a.steps, 20), a.warmup, dev)
    if a.configs:
        extra["configs"] = [time_config(W.WORKLOADS[n], max(a.steps, 20), a.warmup, dev) for n in W.WORKLOADS]
    gbs = r["bytes_layer"] / (r["ms_per_step"] * 1e-3) / 1e9
    ach = r["bytes_layer"] / (r["partial_ms_mean"] * 1e-3) / 1e9
    line = {
        "metric": METRIC,
        "value": round(gbs, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": a.steps,
        "warmup": a.warmup,
        "ms_per_step": round(r["ms_per_step"], 4),
        "us_per_layer": round(r["ms_per_step"] * 1e3, 2),
        "pct_hbm_peak": round(100.0 * gbs / HBM_PEAK_GBS, 1),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "int8(Q) x int4(K) -> i32; f16 x f16 -> f32 (P.V); f32 softmax",
        "data": "synthetic: K/V ~ Student-t(3)/sqrt(3) drawn on the device, Q ~ N(0,1); no model weights",
        "config": {"workload": w.name, "batch": a.batch, "seq_len": w.S, "q_heads": w.Hq, "kv_heads": w.Hkv,
                   "head_dim": w.D, "layout": w.layout, "chunk_tokens": a.chunk, "layers_walked": r["layers"],
                   "packed_bytes_per_layer": r["bytes_layer"]},
        "roofline": {"bound": "hbm", "kernel": "decode_partial", "achieved": round(ach, 1),
                     "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": round(ach / HBM_PEAK_GBS, 4),
                     "traffic": measured_traffic() if (a.batch, a.chunk) == (8, 512) else None, "traffic_unit": "HBM bytes per launch (rocprofv3 FETCH_SIZE + "
                     "WRITE_SIZE, copy-calibrated; null if the kernel changed since)",
                     "avg_launch_us": round(r["partial_ms_mean"] * 1e3, 2),
                     "min_launch_us": round(r["partial_ms_min"] * 1e3, 2),
                     "median_launch_us": round(r["partial_ms_median"] * 1e3, 2),
                     "p10_launch_us": round(r["partial_ms_p10"] * 1e3, 2),
                     "p90_launch_us": round(r["partial_ms_p90"] * 1e3, 2)},
    }
    probe_gbs = r["bytes_layer"] / (r["probe_us"] * 1e-6) / 1e9
    extra["read_probe"] = dict(gbs=round(probe_gbs, 1), us_per_layer=round(r["probe_us"], 2),
                               bytes_per_layer=r["bytes_layer"], decode_partial_frac_of_probe=round(ach / probe_gbs, 4),
                               kernel="kvq_debug_stream_read: the layer's four planes read once, in one launch, "
                                      "with the decode's direct-to-LDS 16-byte nontemporal loads")
    if extra:
        line["extra"] = extra
    if not a.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(w, a.cpu_kv_heads)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
