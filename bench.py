"""Decode-attention bench on one MI355X: packed-KV GB/s and us/layer at 128K context.

Headline workload: Llama-3.1-70B-shaped attention layer (64 query heads, 8 kv
heads, head_dim 128), per-group asymmetric int4 cache (g = 32, fp16 scale +
zero), 131072 cached tokens per row, batch 8, split-K chunks of 512 tokens, K/V
drawn as Student-t(3) / sqrt(3) on the device.

One step = the whole hot path for one layer: quantize-on-append of the new
token of every row (kvq_store), then the split-K decode partial and the reduce
(kvq_attend_decode_partial + kvq_attend_decode_reduce).  Steps walk L distinct
layer caches (L * packed bytes >= 2.5 GB) so the 256 MB Infinity Cache cannot
serve the reads.  Timed with HIP events on the launch stream.

Settling.  From idle, a run of decode steps first sees the shader clock fall
(about 2.4 GHz idle, about 1.96 GHz under sustained decode load) through a
transient in which steps run up to 25 % slower than at steady state before they
recover (about 100 steps).  Before the warm-up steps the bench therefore runs
untimed decode steps until the per-step time has settled (``--settle-ms`` of GPU
time at least, then until two consecutive 20-step windows agree within 2 %, at
most four times that); their count is reported.  The timed steps measure steady
state, the rate a serving loop sees.

Besides the headline line, ``extra`` carries batch 1 at 128K, one decode step of
every workload at its own shape (µs/layer, GB/s, fractions of 8 TB/s and of the
read probe, and the split the decode executed), the causal and full-precision
prefills, the one-token store and the read probe.  ``cpu_baseline`` is the
float64 oracle timed on this host.  Progress goes to stderr; stdout holds one
JSON line.  ``--gpus`` above 1 is refused: the benchmark runs on one GPU.
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
    p.add_argument("--settle-ms", type=float, default=60.0,
                   help="untimed decode steps before the warm-up: at least this much GPU time, then until "
                        "the step time settles (0: none)")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--no-extra", action="store_true",
                   help="only the headline decode and its read probe (no batch 1, configs, prefill or store)")
    p.add_argument("--copy-calibration", action="store_true",
                   help="only run a 1 GiB device-to-device copy 10 times (HBM counter calibration) and exit")
    return p.parse_args()


def progress(msg):
    print(f"[bench {time.strftime('%H:%M:%S')}] {msg}", file=sys.stderr, flush=True)


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


def _events(n):
    import torch
    return [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(n)]


def _median(xs):
    s = sorted(xs)
    return s[len(s) // 2] if s else 0.0


def settle(step, settle_ms):
    """Untimed steps until the GPU's clock has settled under this load: at least settle_ms of GPU time,
    then until two consecutive 20-step windows have medians within 2 % (at most 4 * settle_ms).
    Returns (steps run, median µs of the last window)."""
    import torch
    if settle_ms <= 0:
        return 0, None
    done, spent, last = 0, 0.0, None
    while True:
        evs = _events(20)
        for i in range(20):
            evs[i][0].record()
            step(done + i)
            evs[i][1].record()
        torch.cuda.synchronize()
        us = [a.elapsed_time(b) * 1e3 for a, b in evs]
        done += 20
        spent += sum(us) / 1e3
        med = _median(us)
        if spent >= settle_ms and last is not None and abs(med - last) <= 0.02 * last:
            return done, med
        if spent >= 4 * settle_ms:
            return done, med
        last = med


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


def read_probe(planes_of, layers, steps, warmup):
    """kvq_debug_stream_read over one layer's four planes per launch, walking the layer caches: µs per
    layer (the attainable read rate for the decode's bytes)."""
    import torch
    import quantized_kv_cache_store_amd as kvq
    for i in range(warmup):
        kvq.debug_stream_read(planes_of(i % layers))
    torch.cuda.synchronize()
    p0, p1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    p0.record()
    for i in range(steps):
        kvq.debug_stream_read(planes_of(i % layers))
    p1.record()
    torch.cuda.synchronize()
    return p0.elapsed_time(p1) * 1e3 / steps


def time_decode(w, B, chunk, steps, warmup, layers, dev, seed, settle_ms):
    """The headline step (store one token per row, partial, reduce) with events around each partial."""
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
    wave_tokens, partial_tokens = kvq.decode_split(caches[0], B, w.Hq, S, chunk)

    def step(i, ev=None):
        c = caches[i % L]
        kvq.store(c, k_new, v_new, slot_new)
        if ev is not None:
            ev[0].record()
        kvq.attend_decode_partial(c, q, table, seq, S, w.alpha, chunk, ws)
        if ev is not None:
            ev[1].record()
        kvq.attend_decode_reduce(c, out, seq, S, chunk, ws)

    n_settle, settle_us = settle(step, settle_ms)
    for i in range(warmup):
        step(n_settle + i)
    torch.cuda.synchronize()
    evs = _events(steps)
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    wall0 = time.perf_counter()
    t0.record()
    for i in range(steps):
        step(n_settle + warmup + i, evs[i])
    t1.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    total_ms = t0.elapsed_time(t1)
    part_ms = [a.elapsed_time(b) for a, b in evs]
    assert torch.isfinite(out).all(), "non-finite attention output"
    planes = lambda i: (caches[i].k_payload, caches[i].v_payload, caches[i].k_scale, caches[i].v_scale)
    probe_us = read_probe(planes, L, steps, warmup)
    del caches
    torch.cuda.empty_cache()
    srt = sorted(part_ms)
    return dict(bytes_layer=bytes_layer, layers=L, ms_per_step=total_ms / steps, wall_s=wall,
                partial_ms_mean=sum(part_ms) / len(part_ms), partial_ms_min=min(part_ms),
                partial_ms_median=srt[len(srt) // 2], partial_ms_p10=srt[len(srt) // 10],
                partial_ms_p90=srt[min(len(srt) - 1, (9 * len(srt)) // 10)], probe_us=probe_us,
                settle_steps=n_settle, settle_last_window_us=None if settle_us is None else round(settle_us, 1),
                wave_tokens=wave_tokens, partial_tokens=partial_tokens)


# Layer caches walked per configuration so that the walk spans about 1 GiB or more (the tiny case stays
# cache-resident: it is launch-bound and reported in microseconds only).
CONFIG_LAYERS = {"tiny_q4_0_s1024": 1, "llama3_8b_q4_0_s32k": 32, "qwen3_1p7b_had_s8k": 128,
                 "llama31_70b_asym_s128k": 2, "gemma_q6_0_ragged_b16": 2}


def time_config(w, steps, warmup, dev, batch=None, seed=5):
    """One decode step of a workload at its own shape (batch rows: the workload's, or ``batch``): store
    one token per row at its last position, then the split-K partial and the reduce, walking
    CONFIG_LAYERS[w.name] layer caches (about 1 GiB), replayed from HIP graphs; the read probe over the
    same layers' planes; the split the decode executed."""
    import torch
    import quantized_kv_cache_store_amd as kvq
    import workloads as W

    gen = torch.Generator(device=dev)
    gen.manual_seed(seed)
    lens = [int(n) for n in W.seq_lens(w)]
    if batch is not None:
        lens = lens[:batch]
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
    if batch is not None and batch < w.B:
        L = max(L, math.ceil(1.0e9 / max(packed, 1)))

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
    wave_tokens, partial_tokens = kvq.decode_split_lengths(caches[0], w.Hq, lens, S, w.chunk_tokens)

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
    planes = lambda i: (caches[i].k_payload, caches[i].v_payload, caches[i].k_scale, caches[i].v_scale)
    probe_us = read_probe(planes, L, max(steps, 8), 2)
    plane_bytes = sum(t.numel() for t in planes(0))
    del caches
    torch.cuda.empty_cache()
    alg = packed + window
    probe_gbs = plane_bytes / (probe_us * 1e-6) / 1e9
    gbs = alg / (us * 1e-6) / 1e9
    return dict(workload=w.name, layout=w.layout, batch=B, seq_len_max=S, seq_len_mean=round(sum(lens) / B, 1),
                q_heads=w.Hq, kv_heads=w.Hkv, head_dim=w.D, n_recent=w.n_recent, chunk_tokens=w.chunk_tokens,
                wave_tokens=wave_tokens, partial_tokens=partial_tokens, layers_walked=L,
                bytes_per_layer=alg, us_per_layer=round(us, 2), partial_us=round(part_us, 2),
                gbs=round(gbs, 1), frac_of_8tbs=round(gbs / HBM_PEAK_GBS, 4),
                partial_gbs=round(alg / (part_us * 1e-6) / 1e9, 1),
                probe_gbs=round(probe_gbs, 1), frac_of_probe=round(gbs / probe_gbs, 4),
                probe_bytes=plane_bytes, ideal_us_at_8tbs=round(alg / 8e12 * 1e6, 2),
                timing=f"graphs of {per_graph} steps (store, partial, reduce); partial alone likewise",
                cache_resident=(L * alg < 5e8))


# ------------------------------------------------------------------------------------------- CPU oracle
# Samples of each workload timed on the oracle (float64 numpy): (batch rows, kv heads per row, prefill
# queries).  Rates are per packed byte (GB/s) and extrapolate to the whole layer by the sampled share.
CPU_SAMPLES = {"tiny_q4_0_s1024": ([0], 1, 0), "llama3_8b_q4_0_s32k": ([0], 2, 0),
               "qwen3_1p7b_had_s8k": ([0], 2, 64), "llama31_70b_asym_s128k": ([0], 2, 0),
               "gemma_q6_0_ragged_b16": ([0, 1], 1, 0)}


def cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    import platform
    return platform.processor() or "unknown"


def cpu_oracle_config(w, threads=None):
    """The oracle's store (encode of the sampled K and V rows) and decode attend (which encodes again and
    attends), and for the Hadamard workload its causal prefill, timed on a sample of the workload."""
    from threadpoolctl import threadpool_limits
    import numpy as np
    import quantized_kv_cache_store_amd as kvq
    import workloads as W
    from oracle import attention, quant, spec

    rows, nkv, n_pre = CPU_SAMPLES[w.name]
    layout = {"had_int4": spec.HAD_INT4, "q4_0": spec.Q4_0, "q6_0": spec.Q6_0,
              "asym_int4_g32": spec.ASYM_G32, "q8_0": spec.Q8_0}[w.layout]
    lay = kvq.LAYOUT_IDS[w.layout]
    per_tok = 2 * (kvq.load().kvq_payload_bytes(lay, w.D) + kvq.load().kvq_scale_bytes(lay, w.D))
    lens = [int(n) for n in W.seq_lens(w)]
    t_store = t_attend = t_pre = 0.0
    sampled = 0
    with threadpool_limits(limits=threads):
        for b in rows:
            S = lens[b]
            k = np.stack([W.kv_rows(w, b, hk, 0, S, "k") for hk in range(nkv)], axis=1)
            v = np.stack([W.kv_rows(w, b, hk, 0, S, "v") for hk in range(nkv)], axis=1)
            q = W.queries(w, b)[0][: nkv * w.G]
            t = time.perf_counter()
            for hk in range(nkv):
                quant.encode_rows(layout, k[:, hk, :])
                quant.encode_rows(layout, v[:, hk, :])
            t_store += time.perf_counter() - t
            t = time.perf_counter()
            attention.attend_decode(layout, q, k, v, w.alpha, n_recent=w.n_recent)
            t_attend += time.perf_counter() - t
            sampled += (max(0, S - w.n_recent) if w.n_recent else S) * nkv
            if n_pre:
                qp = W.queries(w, b, n=n_pre, tag=1)[:, : nkv * w.G]
                q_start = S - n_pre
                t = time.perf_counter()
                attention.attend_prefill(layout, qp, k, v, w.alpha, q_start, n_recent=w.n_recent)
                t_pre += time.perf_counter() - t
    total = sum((max(0, n - w.n_recent) if w.n_recent else n) for n in lens) * w.Hkv
    share = sampled / total
    sbytes = sampled * per_tok
    res = dict(workload=w.name, sample=f"rows {rows}, {nkv} of {w.Hkv} kv heads, all tokens"
                                       + (f"; prefill {n_pre} of {w.prefill_q} queries" if n_pre else ""),
               store_s=round(t_store, 3), decode_s=round(t_attend, 3),
               decode_gbs=round(sbytes / t_attend / 1e9, 4),
               decode_us_per_layer=round(t_attend / share * 1e6, 1))
    if n_pre:
        res["prefill_s"] = round(t_pre, 3)
        res["prefill_us_per_chunk"] = round(t_pre * (w.prefill_q / n_pre) * (w.Hkv / nkv) * 1e6, 1)
    return res


def cpu_baseline_all(w_head):
    """cpu_baseline: the oracle's decode rate on the headline workload's sample, with every workload's
    sample on all cores of this process and the three smallest on one thread."""
    import os as _os
    import workloads as W
    cores = len(_os.sched_getaffinity(0))
    cpu_oracle_config(W.WORKLOADS["tiny_q4_0_s1024"])   # first-call costs (imports, allocations) untimed
    per = []
    for name, w in W.WORKLOADS.items():
        progress(f"cpu oracle: {name}")
        per.append(dict(cpu_oracle_config(w), threads=cores))
    for name in ("tiny_q4_0_s1024", "llama3_8b_q4_0_s32k", "qwen3_1p7b_had_s8k"):
        progress(f"cpu oracle, one thread: {name}")
        per.append(dict(cpu_oracle_config(W.WORKLOADS[name], threads=1), threads=1))
    head = next(p for p in per if p["workload"] == w_head.name and p["threads"] == cores)
    return dict(value=head["decode_gbs"], unit="GB/s", cores=cores, kind="oracle",
                sample=f"{w_head.name}: {head['sample']}: float64 numpy encode + decode attend of the sampled "
                       f"packed bytes in {head['decode_s']:.2f} s (numpy elementwise work on one thread, "
                       f"BLAS on up to {cores})",
                cpu_model=cpu_model(), per_config=per)


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
    progress(f"headline decode: {w.name}, batch {a.batch}")
    r = time_decode(w, a.batch, a.chunk, a.steps, a.warmup, a.layers, dev, seed=3, settle_ms=a.settle_ms)
    progress(f"headline decode done: partial {r['partial_ms_mean'] * 1e3:.1f} us, step {r['ms_per_step'] * 1e3:.1f} us,"
             f" {r['settle_steps']} settle steps")
    extra = {}
    probe_gbs = r["bytes_layer"] / (r["probe_us"] * 1e-6) / 1e9
    if not a.no_extra:
        progress("batch 1 at 128K")
        r1 = time_decode(w, 1, a.chunk, a.steps, a.warmup, 0, dev, seed=4, settle_ms=a.settle_ms / 3)
        gbs1 = r1["bytes_layer"] / (r1["ms_per_step"] * 1e-3) / 1e9
        pg1 = r1["bytes_layer"] / (r1["probe_us"] * 1e-6) / 1e9
        extra["batch1"] = dict(us_per_layer=round(r1["ms_per_step"] * 1e3, 2), packed_gbs=round(gbs1, 1),
                               frac_of_8tbs=round(gbs1 / HBM_PEAK_GBS, 4), frac_of_probe=round(gbs1 / pg1, 4),
                               partial_us=round(r1["partial_ms_mean"] * 1e3, 2),
                               partial_median_us=round(r1["partial_ms_median"] * 1e3, 2),
                               partial_frac_of_8tbs=round(r1["bytes_layer"] / (r1["partial_ms_mean"] * 1e-3) / 1e9
                                                          / HBM_PEAK_GBS, 4),
                               probe_gbs=round(pg1, 1), layers_walked=r1["layers"], settle_steps=r1["settle_steps"],
                               wave_tokens=r1["wave_tokens"], partial_tokens=r1["partial_tokens"])
        progress("configs")
        confs = []
        for n, wc in W.WORKLOADS.items():
            progress(f"config {n}")
            confs.append(time_config(wc, max(a.steps, 20), a.warmup, dev))
        progress(f"config {w.name} at batch 1")
        confs.append(time_config(w, max(a.steps, 20), a.warmup, dev, batch=1))
        extra["configs"] = confs
        progress("prefill")
        extra["prefill"] = time_prefill(max(a.steps, 20), a.warmup, dev)
        extra["prefill_full_precision"] = [time_prefill_full(max(a.steps, 20), a.warmup, dev, qs, nq)
                                           for qs, nq in ((8192, 512), (0, 512), (0, 4096))]
        extra["store"] = time_store(max(a.steps, 20), a.warmup, dev)
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
                   "head_dim": w.D, "layout": w.layout, "chunk_tokens": a.chunk,
                   "executed_split": {"wave_tokens": r["wave_tokens"], "partial_tokens": r["partial_tokens"]},
                   "layers_walked": r["layers"], "packed_bytes_per_layer": r["bytes_layer"],
                   "settle_steps": r["settle_steps"], "settle_last_window_us": r["settle_last_window_us"]},
        "roofline": {"bound": "hbm", "kernel": "decode_partial", "achieved": round(ach, 1),
                     "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": round(ach / HBM_PEAK_GBS, 4),
                     "traffic": measured_traffic() if (a.batch, a.chunk) == (8, 512) else None,
                     "traffic_unit": "HBM bytes per launch (rocprofv3 FETCH_SIZE + WRITE_SIZE, copy-calibrated; "
                                     "null if the kernel changed since)",
                     "avg_launch_us": round(r["partial_ms_mean"] * 1e3, 2),
                     "min_launch_us": round(r["partial_ms_min"] * 1e3, 2),
                     "median_launch_us": round(r["partial_ms_median"] * 1e3, 2),
                     "p10_launch_us": round(r["partial_ms_p10"] * 1e3, 2),
                     "p90_launch_us": round(r["partial_ms_p90"] * 1e3, 2)},
    }
    extra["read_probe"] = dict(gbs=round(probe_gbs, 1), us_per_layer=round(r["probe_us"], 2),
                               bytes_per_layer=r["bytes_layer"], decode_partial_frac_of_probe=round(ach / probe_gbs, 4),
                               decode_step_frac_of_probe=round(gbs / probe_gbs, 4),
                               kernel="kvq_debug_stream_read: the layer's four planes read once, in one launch, "
                                      "with the decode's direct-to-LDS 16-byte nontemporal loads")
    line["extra"] = extra
    if not a.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline_all(w)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
