"""Accuracy envelope of the cache layouts against exact attention (float64).

Test infrastructure only (see the package docstring).  The pages report how far
quantised-cache attention lands from full-precision attention without defining
the measure or the data ([FreeToken-268] Validation table; [tract-RFC] accuracy
figures for the planted-outlier data and the n_recent window sweep;
[Open-TQ-Metal] evaluation).  The reading taken here is the relative L2 error
over all query heads of a batch row,

    rel = ||o - o_exact||_2 / ||o_exact||_2,

with o_exact = softmax(alpha q k^T) v computed in float64 on the f32 inputs,
and o the hot path's result as the oracle defines it (``attention``).  Two
ablations separate the sources: each cache side (K or V) can be left exact, and
the query can be kept in f32 instead of int8 on the quantised tokens.

``python -m oracle.envelope`` prints the table for the workloads' value shapes.
"""

import numpy as np

from . import spec
from .attention import encode_cache, _softmax_rows, prepare_query
from .fwht import hadamard_f64
from .quant import f32


def exact_attention(q, k, v, alpha):
    """softmax(alpha q . k^T) . v per query head, float64 on the f32 inputs.

    q [Hq, D]; k, v [S, Hkv, D]; query head h reads kv head h // G.
    """
    q = f32(q)
    k = f32(k)
    v = f32(v)
    Hq, D = q.shape
    S, Hkv, _ = k.shape
    G = Hq // Hkv
    out = np.zeros((Hq, D), dtype=np.float64)
    for h in range(Hq):
        hk = h // G
        p = _softmax_rows(alpha * (k[:, hk, :] @ q[h]))
        out[h] = p @ v[:, hk, :]
    return out


def quantized_attention(layout, q, k, v, alpha, quant_k=True, quant_v=True, int8_q=True, n_recent=0):
    """Decode attention of one batch row with the layout applied as selected.

    quant_k / quant_v: read that side from the dequantised cache (else its exact
    f32 rows, rotated for the Hadamard layout, whose output is rotated back, so
    the rotation itself is exact).  int8_q: score the quantised tokens with the
    dequantised int8 query, as the hot path does (else the f32 query).  The
    newest n_recent tokens are exact f32 rows scored with the f32 query.
    With every option on this is ``attention.attend_decode``.
    """
    q = np.asarray(q)
    Hq, D = q.shape
    S, Hkv, _ = k.shape
    G = Hq // Hkv
    w0 = max(0, S - n_recent) if n_recent > 0 else S
    out = np.zeros((Hq, D), dtype=np.float64)
    for hk in range(Hkv):
        c = encode_cache(layout, k[:, hk, :], v[:, hk, :])
        K = (c["k_hat"] if quant_k else c["k_win"]).copy()
        V = (c["v_hat"] if quant_v else c["v_win"]).copy()
        K[w0:] = c["k_win"][w0:]
        V[w0:] = c["v_win"][w0:]
        for h in range(hk * G, (hk + 1) * G):
            qr, q8, sq = prepare_query(layout, q[h])
            q_quant = sq * q8.astype(np.float64) if int8_q else qr
            s = np.empty(S, dtype=np.float64)
            s[:w0] = K[:w0] @ q_quant
            s[w0:] = K[w0:] @ qr
            o = _softmax_rows(alpha * s) @ V
            out[h] = hadamard_f64(o) if layout == spec.HAD_INT4 else o
    return out


def rel_error(o, o_ref):
    """||o - o_ref||_2 / ||o_ref||_2 over every element."""
    o = np.asarray(o, dtype=np.float64)
    o_ref = np.asarray(o_ref, dtype=np.float64)
    return float(np.linalg.norm(o - o_ref) / np.linalg.norm(o_ref))


def envelope_rows(q, k, v, alpha, layouts, n_recent=0):
    """Relative errors of every layout: both sides, K only, V only, and both with an f32 query."""
    exact = exact_attention(q, k, v, alpha)
    rows = []
    for layout in layouts:
        rows.append(dict(
            layout=layout,
            kv=rel_error(quantized_attention(layout, q, k, v, alpha, n_recent=n_recent), exact),
            k_only=rel_error(quantized_attention(layout, q, k, v, alpha, quant_v=False, n_recent=n_recent), exact),
            v_only=rel_error(quantized_attention(layout, q, k, v, alpha, quant_k=False, n_recent=n_recent), exact),
            kv_f32q=rel_error(quantized_attention(layout, q, k, v, alpha, int8_q=False, n_recent=n_recent), exact),
        ))
    return rows


def window_sweep(layout, q, k, v, alpha, windows):
    """Relative error of the full layout for each window size n_recent."""
    exact = exact_attention(q, k, v, alpha)
    return [(n, rel_error(quantized_attention(layout, q, k, v, alpha, n_recent=n), exact)) for n in windows]


def _sample(w, S, kv_heads):
    """A batch row of a workload's value shapes at S tokens and the first kv_heads kv heads."""
    import workloads as W

    k = np.stack([W.kv_rows(w, 0, hk, 0, S, "k") for hk in range(kv_heads)], axis=1)
    v = np.stack([W.kv_rows(w, 0, hk, 0, S, "v") for hk in range(kv_heads)], axis=1)
    q = W.queries(w, 0)[0][: kv_heads * w.G]
    return q, k, v


def main(S=2048, kv_heads=2):
    import workloads as W

    names = {spec.HAD_INT4: "HAD int4", spec.Q4_0: "q4_0", spec.Q6_0: "q6_0", spec.ASYM_G32: "asym int4 g32",
             spec.Q8_0: "q8_0"}
    layouts = [spec.HAD_INT4, spec.Q4_0, spec.Q6_0, spec.ASYM_G32, spec.Q8_0]
    print(f"relative L2 error vs exact attention, one batch row, {kv_heads} kv heads, S = {S}, no window\n")
    print("| values (workload) | layout | K and V | K only | V only | K and V, f32 query |")
    print("|---|---|---|---|---|---|")
    for wname in ("llama3_8b_q4_0_s32k", "llama31_70b_asym_s128k", "gemma_q6_0_ragged_b16"):
        w = W.WORKLOADS[wname]
        q, k, v = _sample(w, S, kv_heads)
        for r in envelope_rows(q, k, v, w.alpha, layouts):
            print(f"| {wname} | {names[r['layout']]} | {r['kv']:.4f} | {r['k_only']:.4f} | {r['v_only']:.4f} | "
                  f"{r['kv_f32q']:.4f} |")
    w = W.WORKLOADS["qwen3_1p7b_had_s8k"]
    q, k, v = _sample(w, S, kv_heads)
    sweep = window_sweep(spec.HAD_INT4, q, k, v, w.alpha, [0, 16, 64, 256, 1024, S])
    print(f"\nHAD int4 on {w.name} values, window sweep (n_recent: rel error): "
          + ", ".join(f"{n}: {e:.4f}" for n, e in sweep))


if __name__ == "__main__":
    main()
