"""BSBR between-chunk retrieval term — oracle, fp64, CPU (test infrastructure).

Only tests/, the smoke check and bench.py's CPU baseline may use this module; the HIP path
shares no code with it.

Definition followed ("bsbr", Solution: the combined formula with a retrieval term over chunk
states and a within-chunk attention term).  With chunks of B tokens, c(t) = floor(t / B) and
nch = ceil(n / B):

    F_c      = K_c^T V_c                      chunk state: the d x d sum over the chunk's tokens
                                              s < n of k_s v_s^T (the page flattens it; a vector
                                              of d*d numbers and the matrix are the same data)
    W[c, :]  = softmax over c' < c of scale * (R_c . H_c')     meta attention over chunks
    A_c      = sum over c' < c of W[c, c'] F_c'                 the retrieved chunk-level state
    out[t]   = Q[t]^T A_c(t)                                     broadcast over the chunk's tokens
    O        = out + within-chunk attention                      (block-diagonal route)

Readings of the page, each chosen as the plainest one the rest supports:

* R (meta queries) and H (meta keys) are inputs of the operator, one d-vector per chunk and
  query head (R) or key/value head (H); the page names them but not how a model forms them;
* M_out, "the causal mask over chunks", admits strictly earlier chunks only: chunk c's own state
  holds keys later than most of its queries, and its tokens already see each other exactly in
  the within-chunk term.  Chunk 0 therefore retrieves nothing (its row of W is empty: out = 0);
* the mask is applied before the softmax as -inf (weight exactly zero), as for the token masks;
* "Q (elementwise) ... F.repeat(B)": the retrieved state A_c is a d x d matrix per chunk and each
  token t applies its own query to it, out[t] = Q[t]^T A_c(t) — the read-out of a K^T V state, as
  in linear attention; an elementwise product of a d-vector with a d*d-vector is undefined;
* the meta scores use the same scale as the token scores (1/sqrt(d) unless given); the page's
  formula omits the scale in both softmaxes and the rest of the pages use 1/sqrt(d_k);
* no compression of the chunk states (the package's compression factor 1) and no chunk overlap.

Parity for this term is relative: the states are unnormalised sums of B outer products, so the
output is far from unit scale and an absolute bar would be a statement about the inputs' size.
The GPU path accumulates in fp32 and rounds the output to bf16 once or twice (relative error
<= 2^-8 per element), so rel-L2 <= 5e-3 and max-abs <= 1e-2 * max|reference| hold with margin.
"""

from __future__ import annotations

import math

import numpy as np

from .attn import _to_f64


def chunk_states(k, v, B: int) -> np.ndarray:
    """F[b, h_kv, c] = K_c^T V_c (fp64, [batch, heads_kv, nch, d, d]); a partial last chunk sums
    only its tokens s < n."""
    kk, vv = _to_f64(k), _to_f64(v)
    b, hkv, n, d = kk.shape
    nch = (n + B - 1) // B
    F = np.zeros((b, hkv, nch, d, d))
    for c in range(nch):
        s0, s1 = c * B, min(n, (c + 1) * B)
        F[:, :, c] = np.einsum("bhsi,bhsj->bhij", kk[:, :, s0:s1], vv[:, :, s0:s1])
    return F


def meta_weights(r, h, heads_q: int, scale: float) -> np.ndarray:
    """W[b, h_q, c, c'] = softmax over c' < c of scale * R_c . H_c' (zero elsewhere; row 0 is
    all zero)."""
    rr, hh = _to_f64(r), _to_f64(h)
    b, hq, nch, d = rr.shape
    G = hq // hh.shape[1]
    W = np.zeros((b, hq, nch, nch))
    for hd in range(hq):
        sc = scale * np.einsum("bci,bei->bce", rr[:, hd], hh[:, hd // G])
        for c in range(1, nch):
            row = sc[:, c, :c]
            e = np.exp(row - row.max(axis=1, keepdims=True))
            W[:, hd, c, :c] = e / e.sum(axis=1, keepdims=True)
    return W


def retrieval(q, k, v, r, h, B: int, scale: float | None = None, rows=None) -> np.ndarray:
    """The between-chunk term out[b, h_q, t] = Q[t]^T A_c(t) (fp64, [b, h_q, len(rows), d];
    rows defaults to every token)."""
    qq = _to_f64(q)
    b, hq, n, d = qq.shape
    hkv = _to_f64(k).shape[1]
    G = hq // hkv
    sc = 1.0 / math.sqrt(d) if scale is None or scale <= 0 else float(scale)
    rows = np.arange(n) if rows is None else np.asarray(rows, dtype=np.int64)
    F = chunk_states(k, v, B)
    W = meta_weights(r, h, hq, sc)
    out = np.zeros((b, hq, len(rows), d))
    for hd in range(hq):
        for c in np.unique(rows // B):
            A = np.einsum("be,beij->bij", W[:, hd, c], F[:, hd // G])  # retrieved state of chunk c
            sel = np.nonzero(rows // B == c)[0]
            out[:, hd, sel] = np.einsum("bti,bij->btj", qq[:, hd, rows[sel]], A)
    return out


def bsbr_forward(q, k, v, r, h, B: int, scale: float | None = None, rows=None) -> np.ndarray:
    """O = retrieval term + within-chunk causal attention (the block-diagonal route)."""
    from . import attn, routes
    n = _to_f64(q).shape[2]
    rp, ci = routes.route_csr(routes.BLOCK_DIAGONAL, n, B)
    within = attn.attention(q, k, v, B, rp, ci, scale=scale, rows=rows)
    return within + retrieval(q, k, v, r, h, B, scale=scale, rows=rows)
