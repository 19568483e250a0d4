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

Prints one JSON line.  ``--gpus`` above 1 is refused: this build runs on one GPU.
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
    p.add_argument("--cpu-kv-heads", type=int, default=4, help="kv heads of one row timed on the oracle")
    p.add_argument("--batch1", action="store_true", help="also time batch 1 (reported under extra)")
    return p.parse_args()


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
    bytes_layer = B * w.Hkv * S * 2 * (kvq.load().kvq_payload_bytes(3, w.D) + kvq.load().kvq_scale_bytes(3, w.D))
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
    del caches
    torch.cuda.empty_cache()
    return dict(bytes_layer=bytes_layer, layers=L, ms_per_step=total_ms / steps, wall_s=wall,
                partial_ms_mean=sum(part_ms) / len(part_ms), partial_ms_min=min(part_ms),
                partial_ms_median=sorted(part_ms)[len(part_ms) // 2])


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
    if a.gpus != 1:
        print(json.dumps({"error": "this build runs on one GPU; --gpus above 1 is not supported",
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
                     "traffic": None, "avg_launch_us": round(r["partial_ms_mean"] * 1e3, 2),
                     "min_launch_us": round(r["partial_ms_min"] * 1e3, 2)},
    }
    if extra:
        line["extra"] = extra
    if not a.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(w, a.cpu_kv_heads)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
