"""Pins of the BSBR retrieval oracle (oracle/bsbr.py) against facts fixed by the page ("bsbr",
Solution) and by the algebra, not by retyping the oracle's formula:

* chunk states equal a token-by-token sum of outer products (pure Python, partial last chunk);
* chunk 0 retrieves exactly nothing; chunk 1 retrieves chunk 0 with weight 1, which equals the
  token-level sum over chunk 0 of (q . k_s) v_s — the same quantity associated the other way;
* with all meta keys equal the weights are uniform, and the term is prefix linear attention with
  uniform weight per earlier chunk (token-level brute force);
* with scores growing along the chunks the weights concentrate on the previous chunk;
* weights are a distribution over strictly earlier chunks and ignore a shift of every meta key
  by one vector; token order inside a chunk does not matter; GQA equals repeated heads.
"""

import itertools
import math

import numpy as np
import pytest

from oracle import bsbr as OB
from oracle import attn as A
from oracle import routes as R


def rng_inputs(seed, b=1, hq=2, hkv=1, n=11, d=3, B=4):
    g = np.random.default_rng(seed)
    nch = -(-n // B)
    q = g.standard_normal((b, hq, n, d))
    k = g.standard_normal((b, hkv, n, d))
    v = g.standard_normal((b, hkv, n, d))
    r = g.standard_normal((b, hq, nch, d))
    h = g.standard_normal((b, hkv, nch, d))
    return q, k, v, r, h


def test_chunk_states_are_sums_of_outer_products():
    q, k, v, r, h = rng_inputs(1, n=11, B=4)  # chunks of 4, 4, 3 tokens
    F = OB.chunk_states(k, v, 4)
    assert F.shape == (1, 1, 3, 3, 3)
    for c in range(3):
        want = [[0.0] * 3 for _ in range(3)]
        for s in range(4 * c, min(11, 4 * c + 4)):
            for i in range(3):
                for j in range(3):
                    want[i][j] += k[0, 0, s, i] * v[0, 0, s, j]
        assert np.allclose(F[0, 0, c], np.array(want), rtol=1e-13, atol=1e-13)


def token_level(q, k, v, t, chunk_weights, B):
    """sum over earlier chunks c' of w_c' * sum_{s in c'} (q_t . k_s) v_s, in plain loops"""
    d = len(q)
    out = [0.0] * d
    for c, w in chunk_weights.items():
        for s in range(c * B, (c + 1) * B):
            dot = sum(q[i] * k[s][i] for i in range(d))
            for j in range(d):
                out[j] += w * dot * v[s][j]
    return np.array(out)


def test_first_chunk_retrieves_nothing_and_second_retrieves_the_first():
    q, k, v, r, h = rng_inputs(2, n=12, B=4)
    out = OB.retrieval(q, k, v, r, h, 4)
    assert np.array_equal(out[:, :, :4], np.zeros_like(out[:, :, :4]))
    for hd in range(2):
        for t in range(4, 8):
            want = token_level(q[0, hd, t], k[0, 0], v[0, 0], t, {0: 1.0}, 4)
            assert np.allclose(out[0, hd, t], want, rtol=1e-12, atol=1e-12)


def test_equal_meta_keys_give_uniform_prefix_linear_attention():
    q, k, v, r, h = rng_inputs(3, n=16, B=4)
    h[:] = h[:, :, :1]  # every chunk has the same meta key
    out = OB.retrieval(q, k, v, r, h, 4)
    for hd, t in itertools.product(range(2), range(16)):
        c = t // 4
        want = token_level(q[0, hd, t], k[0, 0], v[0, 0], t, {cp: 1.0 / c for cp in range(c)}, 4) if c else np.zeros(3)
        assert np.allclose(out[0, hd, t], want, rtol=1e-12, atol=1e-12)


def test_scores_rising_along_the_chunks_select_the_previous_chunk():
    q, k, v, r, h = rng_inputs(4, hq=1, n=20, B=4)
    r[:] = 0.0
    r[..., 0] = 40.0
    h[:] = 0.0
    h[0, 0, :, 0] = np.arange(h.shape[2])  # score 40 * c' * scale: the latest earlier chunk wins
    W = OB.meta_weights(r, h, 1, 1.0 / math.sqrt(3))
    for c in range(1, 5):
        assert W[0, 0, c, c - 1] > 1 - 1e-9
    out = OB.retrieval(q, k, v, r, h, 4)
    F = OB.chunk_states(k, v, 4)
    for t in range(4, 20):
        assert np.allclose(out[0, 0, t], q[0, 0, t] @ F[0, 0, t // 4 - 1], rtol=1e-8, atol=1e-8)


def test_weights_are_a_distribution_over_earlier_chunks_and_shift_invariant():
    q, k, v, r, h = rng_inputs(5, n=29, B=4)
    W = OB.meta_weights(r, h, 2, 0.7)
    nch = W.shape[2]
    assert np.array_equal(W[:, :, 0], np.zeros_like(W[:, :, 0]))
    for c in range(1, nch):
        assert np.allclose(W[:, :, c, :c].sum(axis=-1), 1.0, rtol=0, atol=1e-14)
        assert (W[:, :, c, :c] > 0).all() and (W[:, :, c, c:] == 0).all()
    shifted = h + np.random.default_rng(6).standard_normal((1, 1, 1, 3))  # same vector for all chunks
    assert np.allclose(OB.meta_weights(r, shifted, 2, 0.7), W, rtol=1e-12, atol=1e-14)


def test_token_order_inside_a_chunk_does_not_matter():
    q, k, v, r, h = rng_inputs(7, n=12, B=4)
    perm = np.arange(12)
    perm[0:4] = [2, 0, 3, 1]
    perm[4:8] = [7, 5, 4, 6]
    out = OB.retrieval(q, k, v, r, h, 4)
    out_p = OB.retrieval(q, k[:, :, perm], v[:, :, perm], r, h, 4)
    assert np.allclose(out[:, :, 8:], out_p[:, :, 8:], rtol=1e-12, atol=1e-12)


def test_gqa_equals_repeated_heads():
    q, k, v, r, h = rng_inputs(8, hq=4, hkv=2, n=13, B=4)
    out = OB.retrieval(q, k, v, r, h, 4)
    rep = lambda x: np.repeat(x, 2, axis=1)  # noqa: E731
    out_rep = OB.retrieval(q, rep(k), rep(v), r, rep(h), 4)
    assert np.allclose(out, out_rep, rtol=1e-13, atol=1e-13)


def test_full_operator_adds_the_within_chunk_term():
    q, k, v, r, h = rng_inputs(9, n=10, B=4)
    O = OB.bsbr_forward(q, k, v, r, h, 4)
    rp, ci = R.route_csr(R.BLOCK_DIAGONAL, 10, 4)
    within = A.attention(q, k, v, 4, rp, ci)
    assert np.allclose(O - within, OB.retrieval(q, k, v, r, h, 4), rtol=1e-13, atol=1e-13)
    # chunk 0 is exactly within-chunk attention
    assert np.array_equal(O[:, :, :4], within[:, :, :4])


@pytest.mark.parametrize("n,B", [(1, 64), (64, 64), (65, 64), (300, 128)])
def test_shapes_and_partial_chunks(n, B):
    q, k, v, r, h = rng_inputs(10, n=n, d=4, B=B)
    out = OB.retrieval(q, k, v, r, h, B)
    assert out.shape == q.shape and np.isfinite(out).all()
    assert np.array_equal(out[:, :, :min(n, B)], np.zeros_like(out[:, :, :min(n, B)]))


def test_two_earlier_chunks_weigh_by_the_logistic_of_the_scaled_score_gap():
    # chunk 2 sees chunks 0 and 1: w1 = 1 / (1 + exp(-scale * (R_2.H_1 - R_2.H_0)))
    q, k, v, r, h = rng_inputs(11, hq=1, n=12, d=3, B=4)
    for scale in (0.25, 1.0 / math.sqrt(3), 2.0):
        W = OB.meta_weights(r, h, 1, scale)
        gap = sum(r[0, 0, 2, i] * (h[0, 0, 1, i] - h[0, 0, 0, i]) for i in range(3))
        w1 = 1.0 / (1.0 + math.exp(-scale * gap))
        assert abs(W[0, 0, 2, 1] - w1) < 1e-14 and abs(W[0, 0, 2, 0] - (1 - w1)) < 1e-14
    # the default scale is 1/sqrt(d): the full term uses it
    out = OB.retrieval(q, k, v, r, h, 4)
    W = OB.meta_weights(r, h, 1, 1.0 / math.sqrt(3))
    F = OB.chunk_states(k, v, 4)
    want = q[0, 0, 9] @ (W[0, 0, 2, 0] * F[0, 0, 0] + W[0, 0, 2, 1] * F[0, 0, 1])
    assert np.allclose(out[0, 0, 9], want, rtol=1e-13, atol=1e-13)


def test_row_subsets_equal_the_full_result():
    q, k, v, r, h = rng_inputs(12, hq=2, hkv=1, n=23, d=3, B=4)
    full = OB.bsbr_forward(q, k, v, r, h, 4)
    rows = np.array([0, 3, 4, 9, 22])
    assert np.allclose(OB.bsbr_forward(q, k, v, r, h, 4, rows=rows), full[:, :, rows], rtol=1e-13, atol=1e-13)
