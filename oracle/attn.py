"""Block-sparse attention as masked dense softmax attention — oracle, fp64, CPU.

Definition followed ("Block-Sparse Attention", "Math Or Compute Schema": the
block mask is applied before the softmax so that only selected query-block ×
key-block regions carry weight; "How It Works": skipped blocks are never
scored; the per-head formula softmax(Q_i K_i^T / sqrt(d_k)) V_i):

    M[t, s] = (block(s) in R(block(t))) and (s <= t) and (s < n) and (t < n)
    S       = Q K^T * scale                      (scale = 1/sqrt(d) by default)
    S[~M]   = -inf
    P       = exp(S - rowmax S) / rowsum         (excluded pairs get exactly 0)
    O       = P V

Readings of the pages used here:

* the mask is additive -inf (weight exactly zero), not a 0/1 product with the
  scores — the product form printed in the formula would leave weight e^0 on
  excluded pairs, which contradicts "skipped blocks are never scored";
* causality inside a block: a query block reads itself causally ("BF1 ...",
  Method; "bsbr", Solution, the within-chunk causal mask M_in), i.e. s <= t;
* grouped-query attention (not on the pages): query head h reads key/value
  head floor(h / G), G = heads_q / heads_kv;
* inputs of any float dtype are converted exactly to float64 first, so the
  oracle sees the same rounded values the GPU path reads.

Rows are processed one query row-panel at a time (softmax is row-wise, so
this is the definition, not a reformulation) to bound memory.
"""

from __future__ import annotations

import numpy as np


def _to_f64(x) -> np.ndarray:
    """Exact conversion of a torch tensor (any float dtype) or array to float64."""
    if hasattr(x, "detach"):
        return x.detach().to("cpu").double().numpy()
    return np.asarray(x, dtype=np.float64)


def token_mask(n: int, B: int, row_ptr, col_idx, rows) -> np.ndarray:
    """Boolean mask M[len(rows), n] for the given query token indices."""
    rows = np.asarray(rows, dtype=np.int64)
    rp = np.asarray(row_ptr, dtype=np.int64)
    ci = np.asarray(col_idx, dtype=np.int64)
    nqb = len(rp) - 1
    blk_allowed = np.zeros((nqb, nqb), dtype=bool)
    for i in range(nqb):
        blk_allowed[i, ci[rp[i]:rp[i + 1]]] = True
    s = np.arange(n, dtype=np.int64)
    m = blk_allowed[(rows // B)[:, None], (s // B)[None, :]]
    m &= s[None, :] <= rows[:, None]
    return m


def attention(q, k, v, B: int, row_ptr, col_idx, scale: float | None = None,
              rows=None, return_lse: bool = False):
    """Masked-dense fp64 attention.

    q: [batch, Hq, n, d]; k, v: [batch, Hkv, n, d] (torch tensors or arrays).
    rows: optional 1-D array of query token indices to evaluate (default all).
    Returns O [batch, Hq, len(rows), d] in float64 (and LSE [batch, Hq, len(rows)]
    = scale*max + log(sum) in natural log when ``return_lse``).
    """
    Q, K, V = _to_f64(q), _to_f64(k), _to_f64(v)
    b, hq, n, d = Q.shape
    hkv = K.shape[1]
    if hq % hkv:
        raise ValueError("heads_q must be a multiple of heads_kv")
    G = hq // hkv
    if scale is None or scale <= 0:
        scale = 1.0 / np.sqrt(d)
    rows = np.arange(n) if rows is None else np.asarray(rows, dtype=np.int64)
    out = np.empty((b, hq, len(rows), d), dtype=np.float64)
    lse = np.empty((b, hq, len(rows)), dtype=np.float64)
    # one panel per query block touched by `rows`
    blocks = rows // B
    for blk in np.unique(blocks):
        sel = np.nonzero(blocks == blk)[0]
        r = rows[sel]
        M = token_mask(n, B, row_ptr, col_idx, r)
        for bi in range(b):
            for h in range(hq):
                kv = h // G
                S = (Q[bi, h, r, :] @ K[bi, kv].T) * scale
                S = np.where(M, S, -np.inf)
                mx = S.max(axis=1, keepdims=True)
                E = np.exp(S - mx)
                den = E.sum(axis=1, keepdims=True)
                P = E / den
                out[bi, h, sel, :] = P @ V[bi, kv]
                lse[bi, h, sel] = mx[:, 0] + np.log(den[:, 0])
    return (out, lse) if return_lse else out


def attention_probs(q, k, B: int, row_ptr, col_idx, scale: float | None = None):
    """The attention weights P [batch, Hq, n, n] (small n only; used by the pins)."""
    Q, K = _to_f64(q), _to_f64(k)
    b, hq, n, d = Q.shape
    G = hq // K.shape[1]
    if scale is None or scale <= 0:
        scale = 1.0 / np.sqrt(d)
    M = token_mask(n, B, row_ptr, col_idx, np.arange(n))
    P = np.empty((b, hq, n, n))
    for bi in range(b):
        for h in range(hq):
            S = np.where(M, (Q[bi, h] @ K[bi, h // G].T) * scale, -np.inf)
            E = np.exp(S - S.max(axis=1, keepdims=True))
            P[bi, h] = E / E.sum(axis=1, keepdims=True)
    return P


def decode_attention(q, k_cache, v_cache, seq_lens, B: int, row_ptr, col_idx, scale: float | None = None,
                     return_lse: bool = False):
    """Selected-page decode, fp64: the newest token of each sequence against its route row.

    Follows "BF1 ...", section 5 ("Selected-page decode characterization"): sequence b holds
    ``seq_lens[b]`` cached tokens; its newest token t = seq_lens[b] - 1 (query block
    i = t // B) attends to the cached keys s <= t whose block is in R(i), the row of the same
    route the prefill uses — so the result is the prefill's row t ("decode-reference
    agreement", section 4).  Lengths are clamped to [1, n_max].

    q: [batch, Hq, d]; k_cache, v_cache: [batch, Hkv, n_max, d].
    Returns o [batch, Hq, d] float64 (and LSE [batch, Hq], natural log, when ``return_lse``).
    """
    Q, K, V = _to_f64(q), _to_f64(k_cache), _to_f64(v_cache)
    b, hq, d = Q.shape
    hkv, n_max = K.shape[1], K.shape[2]
    G = hq // hkv
    if scale is None or scale <= 0:
        scale = 1.0 / np.sqrt(d)
    lens = np.clip(np.asarray(seq_lens, dtype=np.int64), 1, n_max)
    out = np.empty((b, hq, d))
    lse = np.empty((b, hq))
    for bi in range(b):
        t = int(lens[bi]) - 1
        M = token_mask(n_max, B, row_ptr, col_idx, [t])[0]
        for h in range(hq):
            S = np.where(M, (K[bi, h // G] @ Q[bi, h]) * scale, -np.inf)
            mx = S.max()
            E = np.exp(S - mx)
            den = E.sum()
            out[bi, h] = (E / den) @ V[bi, h // G]
            lse[bi, h] = mx + np.log(den)
    return (out, lse) if return_lse else out


def attention_backward(q, k, v, d_o, B: int, row_ptr, col_idx, scale: float | None = None,
                       q_rows=None, k_rows=None):
    """Gradients of block-sparse attention, fp64 (the "gradients" correctness gate of "BF1 ...",
    section 4).

    With O = P V, P = softmax(S) row-wise over the selected keys, S = scale Q K^T, and
    f = sum(O * dO) for the given upstream gradient dO, the chain rule gives, per (b, head):

        dV = P^T dO                       (summed over the query heads sharing a key/value head)
        dP = dO V^T
        dS = P * (dP - D),  D[t] = sum_d dO[t, d] O[t, d]   (= sum_s P[t, s] dP[t, s])
        dQ = scale * dS K
        dK = scale * dS^T Q               (summed over the query heads sharing a key/value head)

    Excluded pairs have P = 0 and therefore dS = 0: no gradient flows through them.  O is
    recomputed here from the inputs.  ``q_rows`` / ``k_rows`` restrict the returned dq rows and
    dk/dv rows (default: all); only the query blocks those rows need are evaluated (dq[t] needs
    its own block; dk[s], dv[s] need every query block whose route row holds block(s)).
    Returns (dq [b, Hq, len(q_rows), d], dk [b, Hkv, len(k_rows), d], dv [same]) in float64.
    """
    Q, K, V, dO = _to_f64(q), _to_f64(k), _to_f64(v), _to_f64(d_o)
    b, hq, n, d = Q.shape
    hkv = K.shape[1]
    G = hq // hkv
    if scale is None or scale <= 0:
        scale = 1.0 / np.sqrt(d)
    q_rows = np.arange(n) if q_rows is None else np.asarray(q_rows, dtype=np.int64)
    k_rows = np.arange(n) if k_rows is None else np.asarray(k_rows, dtype=np.int64)
    rp = np.asarray(row_ptr, dtype=np.int64)
    ci = np.asarray(col_idx, dtype=np.int64)
    nqb = len(rp) - 1
    kblocks = set(int(x) for x in np.unique(k_rows // B))
    need = set(int(x) for x in np.unique(q_rows // B))
    for i in range(nqb):
        if kblocks & set(int(j) for j in ci[rp[i]:rp[i + 1]]):
            need.add(i)
    dq = np.zeros((b, hq, len(q_rows), d))
    dk = np.zeros((b, hkv, n, d))
    dv = np.zeros((b, hkv, n, d))
    qpos = {int(t): x for x, t in enumerate(q_rows)}
    for i in sorted(need):
        r = np.arange(i * B, min((i + 1) * B, n))
        M = token_mask(n, B, row_ptr, col_idx, r)
        for bi in range(b):
            for h in range(hq):
                kv = h // G
                S = np.where(M, (Q[bi, h, r] @ K[bi, kv].T) * scale, -np.inf)
                E = np.exp(S - S.max(axis=1, keepdims=True))
                P = E / E.sum(axis=1, keepdims=True)
                O = P @ V[bi, kv]
                dP = dO[bi, h, r] @ V[bi, kv].T
                Dt = (dO[bi, h, r] * O).sum(axis=1, keepdims=True)
                dS = P * (dP - Dt)
                dQ = scale * (dS @ K[bi, kv])
                for x, t in enumerate(r):
                    if int(t) in qpos:
                        dq[bi, h, qpos[int(t)]] = dQ[x]
                dk[bi, kv] += scale * (dS.T @ Q[bi, h, r])
                dv[bi, kv] += P.T @ dO[bi, h, r]
    return dq, dk[:, :, k_rows], dv[:, :, k_rows]
