"""Integer scores, decode attention, causal prefill and the split-K merge (float64).

Test infrastructure only (see the package docstring).

What the hot path computes, written as its plain definition.  For query head h
of a batch row, with kv head h // G ([Open-TQ-Metal] SIMD and threadgroup
organization: kv_head = head_idx / gqa_factor):

    o = softmax(alpha * q_tilde . K_hat^T + mask) . V_hat

* K_hat, V_hat: the dequantised cache rows ([tract-RFC] Architecture > Data
  flow (decode); [FreeToken-268] Storage layouts; [Open-TQ-Metal] Background).
  For the Hadamard layout they are in the rotated basis.
* q_tilde: for quantised tokens the dequantised int8 query sq * q8 (rotated for
  the Hadamard layout) -- [tract-RFC] scores int8(Q_rot) . int4(K_rot) -> i32,
  scales outside.  For the newest ``n_recent`` tokens the cache keeps exact f32
  rows ([tract-RFC] Causality & mixed precision, n_recent) and the score uses
  the f32 query (reading: the pages report that a full window is exact, which
  only holds with an unquantised query).
* mask: causal prefill hides t > q_start + i from query i ([tract-RFC]
  Causality & mixed precision; Architecture: the chunk is stored first and
  each query is then bounded by its own position).  Decode is single-query and
  sees every cached token.
* Hadamard layout: the output is rotated back, o <- H o ([tract-RFC] data
  flow, un-rotate step).

Float-query mode (``float_q``): the quantised tokens are scored with the f32
query (rotated for the Hadamard layout) instead of its int8 form, q_tilde = q
everywhere.  This is how the other two pages read the cache: [FreeToken-268]
Changes (the attention kernel's K/V load gains unpack paths, i.e. the codes
become floats inside a standard attention) and [Open-TQ-Metal]'s fused kernel
(its nibble-extraction step multiplies the packed codes by a pre-divided
floating-point query).

The integer path that the kernels take is an exact re-association of the same
scores; ``scores_i32`` gives its i32 intermediates for the bit-exact gates, and
``scores_from_i32`` rebuilds the float score from them so that the two forms
can be checked against each other.
"""

import numpy as np

from . import spec
from .fwht import fwht_f32, hadamard_f64
from .quant import encode_rows, dequantize, quantize_q_int8, f32


# --------------------------------------------------------------------- query preparation
def prepare_query(layout, q):
    """Rotate (Hadamard layout) and int8-quantise query vectors [..., D].

    Returns (q_f32 float64 [..., D], q8 int64 [..., D], sq float64 [...]) where
    q_f32 is the (rotated) f32 query used for window tokens.
    """
    q = f32(q)
    qr = fwht_f32(q) if layout == spec.HAD_INT4 else q
    q8, sq = quantize_q_int8(qr)
    return qr, q8, sq


# --------------------------------------------------------------------- integer scores
def scores_i32(layout, q8, codes):
    """I[t, g] = sum over group g of q8[j] * code[t, j], exact integers.

    ``q8`` [D] and ``codes`` [T, D].  Groups are the 32-element blocks, or the
    whole row for the per-token Hadamard layout.  Bound: |I| <= 127 * 32 * 256.
    """
    q8 = np.asarray(q8, dtype=np.int64)
    codes = np.asarray(codes, dtype=np.int64)
    D = q8.shape[-1]
    ng = spec.n_groups(layout, D)
    g = D // ng
    prod = codes * q8[None, :]
    return prod.reshape(codes.shape[0], ng, g).sum(axis=-1)


def scores_from_i32(layout, I, sq, scales, zeros, q8, alpha):
    """alpha * sq * sum_g (s_g * I_g [+ z_g * sum(q8 over g)]) in float64."""
    I = np.asarray(I, dtype=np.float64)
    acc = (np.asarray(scales, dtype=np.float64) * I).sum(axis=-1)
    if layout == spec.ASYM_G32:
        q8 = np.asarray(q8, dtype=np.int64)
        qsum = q8.reshape(-1, spec.BLOCK).sum(axis=-1).astype(np.float64)
        acc = acc + (np.asarray(zeros, dtype=np.float64) * qsum[None, :]).sum(axis=-1)
    return alpha * sq * acc


# --------------------------------------------------------------------- cache view
def encode_cache(layout, k, v):
    """Quantise K and V rows [S, D] of one kv head; returns the dequantised rows and the
    f32 rows the window keeps (rotated for the Hadamard layout)."""
    ek = encode_rows(layout, k)
    ev = encode_rows(layout, v)
    k_hat = dequantize(layout, ek["codes"], ek["scales"], ek["zeros"])
    v_hat = dequantize(layout, ev["codes"], ev["scales"], ev["zeros"])
    if layout == spec.HAD_INT4:
        k_win, v_win = ek["rotated"], ev["rotated"]
    else:
        k_win, v_win = f32(k), f32(v)
    return dict(k_hat=k_hat, v_hat=v_hat, k_win=k_win, v_win=v_win, ek=ek, ev=ev)


def _effective_rows(cache, S, n_recent):
    """K, V rows as attention sees them: f32 for t >= S - n_recent, dequantised before."""
    w0 = max(0, S - n_recent) if n_recent > 0 else S
    K = cache["k_hat"][:S].copy()
    V = cache["v_hat"][:S].copy()
    K[w0:] = cache["k_win"][w0:S]
    V[w0:] = cache["v_win"][w0:S]
    return K, V, w0


def _softmax_rows(s):
    """Row-wise softmax in float64; rows whose entries are all -inf give zeros."""
    m = np.max(s, axis=-1, keepdims=True)
    m = np.where(np.isfinite(m), m, 0.0)
    e = np.exp(s - m)
    den = e.sum(axis=-1, keepdims=True)
    return e / np.where(den == 0.0, 1.0, den)


def _query_rows(layout, q):
    """Query forms: the dequantised int8 query (quantised tokens) and the f32 query (window)."""
    qr, q8, sq = prepare_query(layout, q)
    q_quant = sq[..., None] * q8.astype(np.float64)
    return q_quant, qr


# --------------------------------------------------------------------- decode
def attend_decode(layout, q, k, v, alpha, n_recent=0, float_q=False):
    """Single-query decode attention of one batch row.

    q [Hq, D] f32; k, v [S, Hkv, D] f32 (every cached token, in position order);
    returns o [Hq, D] float64.  float_q: the float-query mode (module docstring).
    """
    q = np.asarray(q)
    Hq, D = q.shape
    S, Hkv, _ = k.shape
    if Hq % Hkv:
        raise ValueError("query heads must be a multiple of kv heads")
    G = Hq // Hkv
    out = np.zeros((Hq, D), dtype=np.float64)
    if S == 0:
        return out
    for hk in range(Hkv):
        cache = encode_cache(layout, k[:, hk, :], v[:, hk, :])
        K, V, w0 = _effective_rows(cache, S, n_recent)
        for h in range(hk * G, (hk + 1) * G):
            q_quant, q_f = _query_rows(layout, q[h])
            if float_q:
                q_quant = q_f
            s = np.empty(S, dtype=np.float64)
            s[:w0] = K[:w0] @ q_quant
            s[w0:] = K[w0:] @ q_f
            p = _softmax_rows(alpha * s)
            o = p @ V
            out[h] = hadamard_f64(o) if layout == spec.HAD_INT4 else o
    return out


# --------------------------------------------------------------------- causal prefill
def attend_prefill(layout, q, k, v, alpha, q_start, causal=True, n_recent=0):
    """Multi-query attention of a prefill chunk of one batch row.

    q [Sq, Hq, D]; query i sits at absolute position q_start + i and, when
    ``causal``, sees tokens t <= q_start + i.  k, v [S, Hkv, D] hold every
    cached token after the chunk was appended (S >= q_start + Sq).  Window
    tokens are the last ``n_recent`` positions of the cache, the same for every
    query of the chunk.  Computed as compute-then-mask.  Returns [Sq, Hq, D].
    """
    q = np.asarray(q)
    Sq, Hq, D = q.shape
    S, Hkv, _ = k.shape
    G = Hq // Hkv
    out = np.zeros((Sq, Hq, D), dtype=np.float64)
    pos = q_start + np.arange(Sq)
    t = np.arange(S)
    for hk in range(Hkv):
        cache = encode_cache(layout, k[:, hk, :], v[:, hk, :])
        K, V, w0 = _effective_rows(cache, S, n_recent)
        for h in range(hk * G, (hk + 1) * G):
            q_quant, q_f = _query_rows(layout, q[:, h, :])   # [Sq, D]
            s = np.empty((Sq, S), dtype=np.float64)
            s[:, :w0] = q_quant @ K[:w0].T
            s[:, w0:] = q_f @ K[w0:].T
            s = alpha * s
            if causal:
                s = np.where(t[None, :] <= pos[:, None], s, -np.inf)
            p = _softmax_rows(s)
            o = p @ V
            out[:, h, :] = hadamard_f64(o) if layout == spec.HAD_INT4 else o
    return out


# --------------------------------------------------------------------- full-precision prefill
def attend_prefill_full(layout, q, k, v, alpha, q_start, causal=True, n_recent=0):
    """Prefill of a chunk in full precision, before the chunk is quantised into the cache.

    [Open-TQ-Metal] prefill/decode selection paragraph: a multi-query step runs
    attention on the full-precision K, V and only then quantises and stores
    them; decode reads the packed cache.  Reading taken for a chunk that follows
    a cached prefix: the chunk's own tokens are read as the exact f32 rows
    (rotated for the Hadamard layout) scored with the f32 query, and the prefix
    as the cache held it before the chunk was stored -- quantised, except the
    newest min(q_start, n_recent) positions, which the window keeps in f32.

    q [Sq, Hq, D], query i at position q_start + i; k, v [q_start + Sq, Hkv, D]:
    the cached prefix followed by the chunk's rows.  causal: query i sees
    t <= q_start + i.  Returns [Sq, Hq, D] float64.
    """
    q = np.asarray(q)
    Sq, Hq, D = q.shape
    S, Hkv, _ = k.shape
    if S != q_start + Sq:
        raise ValueError("k, v must hold the prefix and the chunk")
    G = Hq // Hkv
    out = np.zeros((Sq, Hq, D), dtype=np.float64)
    pos = q_start + np.arange(Sq)
    t = np.arange(S)
    for hk in range(Hkv):
        if q_start > 0:
            cache = encode_cache(layout, k[:q_start, hk, :], v[:q_start, hk, :])
            Kp, Vp, w0 = _effective_rows(cache, q_start, n_recent)
        else:
            Kp, Vp, w0 = np.zeros((0, D)), np.zeros((0, D)), 0
        if layout == spec.HAD_INT4:
            kc, vc = fwht_f32(k[q_start:, hk, :]), fwht_f32(v[q_start:, hk, :])
        else:
            kc, vc = f32(k[q_start:, hk, :]), f32(v[q_start:, hk, :])
        K = np.concatenate([Kp, kc])
        V = np.concatenate([Vp, vc])
        for h in range(hk * G, (hk + 1) * G):
            q_quant, q_f = _query_rows(layout, q[:, h, :])
            s = np.empty((Sq, S), dtype=np.float64)
            s[:, :w0] = q_quant @ K[:w0].T
            s[:, w0:] = q_f @ K[w0:].T
            s = alpha * s
            if causal:
                s = np.where(t[None, :] <= pos[:, None], s, -np.inf)
            o = _softmax_rows(s) @ V
            out[:, h, :] = hadamard_f64(o) if layout == spec.HAD_INT4 else o
    return out


# --------------------------------------------------------------------- split-K
def chunk_partial(scores, V):
    """One split-K chunk: (o_c unnormalised, m_c, l_c) of scores [T] and rows V [T, D].

    [Open-TQ-Metal] split-K paragraphs: each chunk emits its partial output,
    running max and sum of exponentials.  An empty or fully masked chunk gives
    (0, -inf, 0).
    """
    scores = np.asarray(scores, dtype=np.float64)
    D = V.shape[-1]
    if scores.size == 0 or not np.isfinite(scores).any():
        return np.zeros(D), -np.inf, 0.0
    m = np.max(scores)
    p = np.exp(scores - m)
    return p @ V, m, p.sum()


def merge_partials(parts):
    """Online-softmax merge of chunk partials (the split-K reduce).

    m = max_c m_c, w_c = exp(m_c - m) (0 for an empty chunk),
    o = sum_c w_c o_c / sum_c w_c l_c.  The page's own formula is missing; this
    is the log-sum-exp combination that reproduces the single pass.
    """
    ms = np.array([p[1] for p in parts], dtype=np.float64)
    D = parts[0][0].shape[-1]
    if not np.isfinite(ms).any():
        return np.zeros(D)
    m = np.max(ms)
    w = np.where(np.isfinite(ms), np.exp(np.where(np.isfinite(ms), ms - m, 0.0)), 0.0)
    num = sum(wc * p[0] for wc, p in zip(w, parts))
    den = sum(wc * p[2] for wc, p in zip(w, parts))
    return num / den


def attend_decode_split(layout, q, k, v, alpha, chunk, n_recent=0, float_q=False):
    """Decode attention computed as split-K chunks of ``chunk`` tokens plus the merge.

    Same inputs and result as ``attend_decode`` up to float re-association.
    """
    q = np.asarray(q)
    Hq, D = q.shape
    S, Hkv, _ = k.shape
    G = Hq // Hkv
    out = np.zeros((Hq, D), dtype=np.float64)
    if S == 0:
        return out
    for hk in range(Hkv):
        cache = encode_cache(layout, k[:, hk, :], v[:, hk, :])
        K, V, w0 = _effective_rows(cache, S, n_recent)
        for h in range(hk * G, (hk + 1) * G):
            q_quant, q_f = _query_rows(layout, q[h])
            if float_q:
                q_quant = q_f
            s = np.empty(S, dtype=np.float64)
            s[:w0] = K[:w0] @ q_quant
            s[w0:] = K[w0:] @ q_f
            s = alpha * s
            parts = [chunk_partial(s[c:c + chunk], V[c:c + chunk]) for c in range(0, S, chunk)]
            o = merge_partials(parts)
            out[h] = hadamard_f64(o) if layout == spec.HAD_INT4 else o
    return out
