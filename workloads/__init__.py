"""Seeded synthetic inputs for the quantized-KV workloads.

This module only draws random numbers and shapes them (distributions,
outlier channels, RMS normalisation of the inputs, ragged lengths, page
permutations).  It holds none of the quantisation or attention arithmetic and
imports neither the oracle nor the HIP binding, so both sides can take their
inputs from it.

Addressability.  K/V values are drawn in 4096-token chunks per
(batch row, kv head, tensor) from ``numpy.random.SeedSequence`` keys, so any
slice of a cache can be regenerated on its own: a test can feed a full-size
cache to the GPU and recompute any single output on the CPU.

The workloads take the shapes of the models the pages run (Llama-3-8B,
Qwen3-1.7B, Llama-3.1-70B, Gemma-style wide heads) and the value shapes the pages
describe: N(0,1) with planted outlier channels ([tract-RFC] Appendix 7,
planted-outlier data) and heavy-tailed "kurtotic" K/V ([FreeToken-268]
Validation table), here Student-t with 3 degrees of freedom scaled to unit
variance.  No model weights or datasets are involved.
"""

import math
from dataclasses import dataclass, field

import numpy as np

CHUNK = 4096
_K, _V, _Q, _OUTL, _LEN, _PAGES = 0, 1, 2, 3, 4, 5


@dataclass(frozen=True)
class Workload:
    name: str
    seed: int
    layout: str               # "had_int4" | "q4_0" | "q6_0" | "asym_int4_g32"
    Hq: int
    Hkv: int
    D: int
    S: int                    # cached tokens per row (upper bound when ragged)
    B: int
    alpha: float
    dist: str                 # "normal" | "t3"
    outliers: int = 0         # outlier channels per kv head (x10)
    n_recent: int = 0
    chunk_tokens: int = 512   # split-K chunk
    page_size: int = 256
    ragged: tuple = ()        # (lo, hi) inclusive bounds of per-row lengths
    rms_norm_qk: bool = False
    shuffle_pages: bool = False
    prefill_q: int = 0        # queries of the causal prefill chunk (appended at the tail)
    extra: dict = field(default_factory=dict)

    @property
    def G(self):
        return self.Hq // self.Hkv


WORKLOADS = {
    # 1 head, S=1024, q4_0 -- the small case the oracle finishes in well under a second
    "tiny_q4_0_s1024": Workload(
        name="tiny_q4_0_s1024", seed=0, layout="q4_0", Hq=1, Hkv=1, D=128, S=1024, B=1,
        alpha=1.0 / math.sqrt(128), dist="normal", chunk_tokens=512, page_size=256),
    # Llama-3-8B-shaped decode layer, GQA 4, store one token then attend
    "llama3_8b_q4_0_s32k": Workload(
        name="llama3_8b_q4_0_s32k", seed=1, layout="q4_0", Hq=32, Hkv=8, D=128, S=32768, B=1,
        alpha=1.0 / math.sqrt(128), dist="normal", outliers=4, chunk_tokens=512, page_size=256),
    # Qwen3-1.7B-shaped Hadamard layout with a 64-token f32 window, decode plus a 512-query prefill
    "qwen3_1p7b_had_s8k": Workload(
        name="qwen3_1p7b_had_s8k", seed=2, layout="had_int4", Hq=16, Hkv=8, D=128, S=8192, B=1,
        alpha=1.0 / math.sqrt(128), dist="normal", outliers=4, n_recent=64, chunk_tokens=512,
        page_size=256, prefill_q=512),
    # Llama-3.1-70B-shaped long context, per-group asymmetric int4, split-K chunks of 512
    "llama31_70b_asym_s128k": Workload(
        name="llama31_70b_asym_s128k", seed=3, layout="asym_int4_g32", Hq=64, Hkv=8, D=128,
        S=131072, B=8, alpha=1.0 / math.sqrt(128), dist="t3", chunk_tokens=512, page_size=1024),
    # Gemma-style d=256 heads, q6_0, ragged batch of 16 in shuffled 16-token pages
    "gemma_q6_0_ragged_b16": Workload(
        name="gemma_q6_0_ragged_b16", seed=4, layout="q6_0", Hq=16, Hkv=8, D=256, S=65536, B=16,
        alpha=1.0, dist="t3", chunk_tokens=512, page_size=16, ragged=(4096, 65536),
        rms_norm_qk=True, shuffle_pages=True),
}


def _rng(*key):
    return np.random.default_rng(np.random.SeedSequence([int(k) for k in key]))


def seq_lens(w: Workload):
    """Per-row cached lengths: S for every row, or uniform integers in the ragged bounds."""
    if not w.ragged:
        return np.full(w.B, w.S, dtype=np.int64)
    lo, hi = w.ragged
    return _rng(w.seed, _LEN).integers(lo, hi, size=w.B, endpoint=True).astype(np.int64)


def outlier_channels(w: Workload, hk):
    """The planted outlier channels of kv head ``hk`` (shared by K and V)."""
    if w.outliers == 0:
        return np.zeros(0, dtype=np.int64)
    return np.sort(_rng(w.seed, _OUTL, hk).choice(w.D, size=w.outliers, replace=False))


def _draw(w: Workload, rng, shape):
    if w.dist == "normal":
        return rng.standard_normal(shape, dtype=np.float64)
    if w.dist == "t3":
        return rng.standard_t(3, size=shape) / math.sqrt(3.0)
    raise ValueError(w.dist)


def _rms_normalise(x, eps=1e-6):
    """x / sqrt(mean(x^2) + eps) per row (unit weight): the Q/K norms of wide-head models."""
    return x / np.sqrt(np.mean(x * x, axis=-1, keepdims=True) + eps)


def kv_rows(w: Workload, b, hk, t0, t1, which):
    """K (``which='k'``) or V rows of tokens [t0, t1) of row b, kv head hk: float32 [t1-t0, D]."""
    out = np.empty((max(0, t1 - t0), w.D), dtype=np.float32)
    tensor = _K if which == "k" else _V
    t = t0
    while t < t1:
        c = t // CHUNK
        c0, c1 = c * CHUNK, (c + 1) * CHUNK
        x = _draw(w, _rng(w.seed, tensor, b, hk, c), (CHUNK, w.D))
        ch = outlier_channels(w, hk)
        if ch.size:
            x[:, ch] *= 10.0
        if w.rms_norm_qk and which == "k":
            x = _rms_normalise(x)
        e = min(t1, c1)
        out[t - t0:e - t0] = x[t - c0:e - c0].astype(np.float32)
        t = e
    return out


def kv_tokens(w: Workload, b, t0, t1, which):
    """Rows of all kv heads for tokens [t0, t1): float32 [t1-t0, Hkv, D]."""
    return np.stack([kv_rows(w, b, hk, t0, t1, which) for hk in range(w.Hkv)], axis=1)


def queries(w: Workload, b, n=1, tag=0):
    """Query vectors of row b: float32 [n, Hq, D] (``tag`` separates independent draws)."""
    x = _rng(w.seed, _Q, b, tag).standard_normal((n, w.Hq, w.D), dtype=np.float64)
    if w.rms_norm_qk:
        x = _rms_normalise(x)
    return x.astype(np.float32)


def block_tables(w: Workload, lens, page_size=None, pages_per_row=None):
    """Logical-to-physical page map per row, int32 [B, pages_per_row].

    Rows get consecutive physical pages unless the workload shuffles them, in
    which case the physical page ids are a seeded permutation.  Unused entries
    are -1.  Returns (table, num_pages).
    """
    ps = page_size or w.page_size
    need = [(int(n) + ps - 1) // ps for n in lens]
    ppr = pages_per_row or max(need)
    total = int(sum(need))
    phys = np.arange(total, dtype=np.int64)
    if w.shuffle_pages:
        phys = _rng(w.seed, _PAGES).permutation(total)
    table = np.full((len(lens), ppr), -1, dtype=np.int32)
    k = 0
    for b, n in enumerate(need):
        table[b, :n] = phys[k:k + n]
        k += n
    return table, total


def kv_tokens_device(w: Workload, n, which, generator, device):
    """Rows of all kv heads for ``n`` tokens drawn on the device: float32 [n, Hkv, D].

    Same distribution, outlier channels and K normalisation as ``kv_tokens``, but
    a different stream (torch's device generator): for filling multi-GB caches
    whose values no CPU-side check reads.
    """
    import torch

    shape = (n, w.Hkv, w.D)
    x = torch.randn(shape, generator=generator, device=device, dtype=torch.float32)
    if w.dist == "t3":
        chi = torch.randn((3,) + shape, generator=generator, device=device, dtype=torch.float32)
        x = x / torch.sqrt((chi * chi).sum(0) / 3.0) / math.sqrt(3.0)
    if w.outliers:
        for hk in range(w.Hkv):
            ch = torch.as_tensor(outlier_channels(w, hk), device=device)
            x[:, hk, ch] *= 10.0
    if w.rms_norm_qk and which == "k":
        x = x / torch.sqrt((x * x).mean(-1, keepdim=True) + 1e-6)
    return x
