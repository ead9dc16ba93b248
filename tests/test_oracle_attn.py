"""Pins for the oracle's masked-dense attention (CPU only).

Ties oracle/attn.py to a library routine (torch's scaled_dot_product_attention
in float64 for the dense-causal and per-chunk reductions), to invariants of the
softmax (rows sum to one, exact zeros outside the route), to closed forms
(uniform weights when K = 0, single-key rows) and to a pure-Python scalar
brute force on tiny inputs whose route membership is restated independently.
"""

import math

import numpy as np
import pytest
import torch
import torch.nn.functional as F

from oracle import attn as A
from oracle import routes as R

KINDS = [R.BF1, R.BLOCK_DIAGONAL, R.DENSE_CAUSAL, R.STATIC_RANDOM, R.SLIDING_WINDOW]


def _qkv(b, hq, hkv, n, d, seed=0, dtype=torch.float64):
    g = torch.Generator("cpu").manual_seed(seed)
    q = torch.randn(b, hq, n, d, generator=g, dtype=torch.float64).to(dtype)
    k = torch.randn(b, hkv, n, d, generator=g, dtype=torch.float64).to(dtype)
    v = torch.randn(b, hkv, n, d, generator=g, dtype=torch.float64).to(dtype)
    return q, k, v


def _pow2(x):
    return x > 0 and (x & (x - 1)) == 0


def _member(kind, i, j, nl=2):
    """Block membership restated without oracle.routes (static-random excepted)."""
    if kind == R.BF1:
        off = i - j
        return 0 <= j <= i and (off <= nl or _pow2(off) or j == 0)
    if kind == R.BLOCK_DIAGONAL:
        return i == j
    if kind == R.DENSE_CAUSAL:
        return 0 <= j <= i
    if kind == R.SLIDING_WINDOW:
        return 0 <= i - j <= nl
    return j in R.static_random_set(i, 14, 17, True)


@pytest.mark.parametrize("n,B", [(256, 32), (100, 16)])
def test_dense_route_is_causal_sdpa(n, B):
    q, k, v = _qkv(2, 3, 3, n, 16, seed=1)
    rp, ci = R.route_csr(R.DENSE_CAUSAL, n, B)
    got = A.attention(q, k, v, B, rp, ci)
    ref = F.scaled_dot_product_attention(q, k, v, is_causal=True).numpy()
    assert np.abs(got - ref).max() < 1e-12


def test_explicit_scale_matches_sdpa():
    q, k, v = _qkv(1, 2, 2, 64, 8, seed=2)
    rp, ci = R.route_csr(R.DENSE_CAUSAL, 64, 16)
    got = A.attention(q, k, v, 16, rp, ci, scale=0.3)
    ref = F.scaled_dot_product_attention(q, k, v, is_causal=True, scale=0.3).numpy()
    assert np.abs(got - ref).max() < 1e-12


@pytest.mark.parametrize("n,B,nl", [(256, 32, 2), (100, 16, 3), (64, 8, 0)])
def test_sliding_window_is_banded_sdpa(n, B, nl):
    # the library routine with an explicit boolean mask: key block within nl blocks before the
    # query block, and causal
    q, k, v = _qkv(2, 2, 1, n, 16, seed=11)
    rp, ci = R.route_csr(R.SLIDING_WINDOW, n, B, n_local=nl)
    got = A.attention(q, k, v, B, rp, ci)
    t = torch.arange(n)
    band = ((t[:, None] // B) - (t[None, :] // B) <= nl) & (t[None, :] <= t[:, None])
    kk, vv = k.repeat_interleave(2, 1), v.repeat_interleave(2, 1)
    ref = F.scaled_dot_product_attention(q, kk, vv, attn_mask=band).numpy()
    assert np.abs(got - ref).max() < 1e-12


@pytest.mark.parametrize("n,B", [(256, 32), (96, 16)])
def test_block_diagonal_is_per_chunk_attention(n, B):
    q, k, v = _qkv(2, 2, 2, n, 16, seed=3)
    rp, ci = R.route_csr(R.BLOCK_DIAGONAL, n, B)
    got = A.attention(q, k, v, B, rp, ci)
    for c in range(n // B):
        sl = slice(c * B, (c + 1) * B)
        ref = F.scaled_dot_product_attention(q[:, :, sl], k[:, :, sl], v[:, :, sl], is_causal=True).numpy()
        assert np.abs(got[:, :, sl] - ref).max() < 1e-12
    # permuting chunks permutes the outputs identically
    perm = np.random.default_rng(0).permutation(n // B)
    idx = np.concatenate([np.arange(p * B, (p + 1) * B) for p in perm])
    got_p = A.attention(q[:, :, idx], k[:, :, idx], v[:, :, idx], B, rp, ci)
    assert np.abs(got_p - got[:, :, idx]).max() < 1e-12


@pytest.mark.parametrize("kind", KINDS)
def test_probs_rows_sum_to_one_and_exact_zeros(kind):
    n, B = 72, 8
    q, k, v = _qkv(1, 2, 1, n, 8, seed=4)
    rp, ci = R.route_csr(kind, n, B)
    P = A.attention_probs(q, k, B, rp, ci)
    assert np.abs(P.sum(-1) - 1).max() < 1e-12
    for t in range(n):
        for s in range(n):
            inside = s <= t and _member(kind, t // B, s // B)
            if inside:
                assert (P[:, :, t, s] > 0).all()
            else:
                assert (P[:, :, t, s] == 0.0).all()


def _brute(q, k, v, B, kind, scale, G):
    """Pure-Python scalar triple loop with math.exp."""
    b, hq, n, d = q.shape
    out = np.zeros((b, hq, n, d))
    for bi in range(b):
        for h in range(hq):
            kv = h // G
            for t in range(n):
                sel = [s for s in range(t + 1) if _member(kind, t // B, s // B)]
                sc = [scale * sum(float(q[bi, h, t, e]) * float(k[bi, kv, s, e]) for e in range(d)) for s in sel]
                mx = max(sc)
                w = [math.exp(x - mx) for x in sc]
                den = sum(w)
                for e in range(d):
                    out[bi, h, t, e] = sum(w[a] * float(v[bi, kv, s, e]) for a, s in enumerate(sel)) / den
    return out


@pytest.mark.parametrize("kind", KINDS)
@pytest.mark.parametrize("n,B", [(64, 8), (37, 4), (37, 8)])
def test_brute_force_tiny(kind, n, B):
    q, k, v = _qkv(1, 2, 1, n, 5, seed=5)
    rp, ci = R.route_csr(kind, n, B)
    got = A.attention(q, k, v, B, rp, ci)
    ref = _brute(q, k, v, B, kind, 1 / math.sqrt(5), 2)
    assert np.abs(got - ref).max() < 1e-12


@pytest.mark.parametrize("kind", KINDS)
def test_uniform_weights_when_k_is_zero(kind):
    # K = 0 makes every selected score 0, so O[t] is the plain mean of V over the selected keys.
    n, B = 300, 16
    q, _, _ = _qkv(1, 1, 1, n, 4, seed=6)
    k = torch.zeros(1, 1, n, 4, dtype=torch.float64)
    s = torch.arange(n, dtype=torch.float64)
    v = torch.stack([torch.ones(n), s, s * s, torch.zeros(n)], -1)[None, None]
    rp, ci = R.route_csr(kind, n, B)
    got, lse = A.attention(q, k, v, B, rp, ci, return_lse=True)
    for t in range(n):
        sel = [x for x in range(t + 1) if _member(kind, t // B, x // B)]
        assert abs(got[0, 0, t, 0] - 1.0) < 1e-12
        assert abs(got[0, 0, t, 1] - np.mean(sel)) < 1e-9
        assert abs(got[0, 0, t, 2] - np.mean(np.square(sel))) < 1e-6 * max(1.0, np.mean(np.square(sel)))
        assert abs(lse[0, 0, t] - math.log(len(sel))) < 1e-12


@pytest.mark.parametrize("kind", KINDS)
def test_first_row_reads_only_itself(kind):
    q, k, v = _qkv(2, 2, 2, 40, 8, seed=7)
    rp, ci = R.route_csr(kind, 40, 8)
    got = A.attention(q, k, v, 8, rp, ci)
    assert np.array_equal(got[:, :, 0], v[:, :, 0].numpy())


def test_gqa_equals_repeated_kv():
    q, k, v = _qkv(1, 6, 2, 48, 8, seed=8)
    rp, ci = R.route_csr(R.BF1, 48, 8)
    got = A.attention(q, k, v, 8, rp, ci)
    ref = A.attention(q, k.repeat_interleave(3, dim=1), v.repeat_interleave(3, dim=1), 8, rp, ci)
    assert np.array_equal(got, ref)
    # and not the tiled (h % Hkv) mapping
    alt = A.attention(q, k.repeat(1, 3, 1, 1), v.repeat(1, 3, 1, 1), 8, rp, ci)
    assert np.abs(alt - got).max() > 1e-3


def test_rows_subset_matches_full():
    q, k, v = _qkv(1, 2, 2, 130, 8, seed=9)
    rp, ci = R.route_csr(R.STATIC_RANDOM, 130, 16)
    full = A.attention(q, k, v, 16, rp, ci)
    rows = np.array([0, 5, 17, 64, 129])
    part = A.attention(q, k, v, 16, rp, ci, rows=rows)
    assert np.abs(part - full[:, :, rows]).max() < 1e-13  # same rows, different BLAS blocking


def test_bf16_inputs_are_read_exactly():
    q, k, v = _qkv(1, 1, 1, 32, 8, seed=10, dtype=torch.bfloat16)
    rp, ci = R.route_csr(R.BF1, 32, 8)
    a = A.attention(q, k, v, 8, rp, ci)
    b = A.attention(q.double(), k.double(), v.double(), 8, rp, ci)
    assert np.array_equal(a, b)


# --- selected-page decode ------------------------------------------------------------------

@pytest.mark.parametrize("kind", KINDS)
def test_decode_matches_masked_sdpa(kind):
    # one query per sequence against the library routine with an explicit token mask whose
    # membership is restated independently of oracle.routes
    n_max, B, hq, hkv, d = 90, 8, 4, 2, 8
    lens = [1, 8, 9, 57, 90]
    g = torch.Generator("cpu").manual_seed(21)
    q = torch.randn(len(lens), hq, d, generator=g, dtype=torch.float64)
    k = torch.randn(len(lens), hkv, n_max, d, generator=g, dtype=torch.float64)
    v = torch.randn(len(lens), hkv, n_max, d, generator=g, dtype=torch.float64)
    rp, ci = R.route_csr(kind, n_max, B)
    got, lse = A.decode_attention(q, k, v, lens, B, rp, ci, return_lse=True)
    for bi, ln in enumerate(lens):
        t = ln - 1
        mask = torch.tensor([[s <= t and _member(kind, t // B, s // B) for s in range(n_max)]])
        kk, vv = k[bi].repeat_interleave(2, 0), v[bi].repeat_interleave(2, 0)
        ref = F.scaled_dot_product_attention(q[bi][:, None], kk, vv, attn_mask=mask)[:, 0].numpy()
        assert np.abs(got[bi] - ref).max() < 1e-12
        sel = [s for s in range(n_max) if mask[0, s]]
        sc = (kk[:, sel] @ q[bi][:, :, None])[..., 0].numpy() / math.sqrt(d)  # [hq, |sel|]
        want_lse = np.log(np.exp(sc).sum(-1))
        assert np.abs(lse[bi] - want_lse).max() < 1e-12


@pytest.mark.parametrize("kind", KINDS)
def test_decode_agrees_with_prefill_row(kind):
    # decode-reference agreement: the decoded token t gives row t of the prefill output
    n, B = 120, 16
    q, k, v = _qkv(2, 4, 2, n, 8, seed=22)
    rp, ci = R.route_csr(kind, n, B)
    full = A.attention(q, k, v, B, rp, ci)
    for t in (0, 15, 16, 77, 119):
        got = A.decode_attention(q[:, :, t], k, v, [t + 1, t + 1], B, rp, ci)
        assert np.abs(got - full[:, :, t]).max() < 1e-12


def test_decode_closed_forms():
    # K = 0: uniform weights over the selected keys; a one-token cache returns v[0]; lengths are
    # clamped to [1, n_max]
    n_max, B = 200, 16
    s = torch.arange(n_max, dtype=torch.float64)
    v = torch.stack([torch.ones(n_max), s, s * s], -1)[None, None]
    k = torch.zeros(1, 1, n_max, 3, dtype=torch.float64)
    q = torch.randn(1, 1, 3, dtype=torch.float64)
    rp, ci = R.route_csr(R.BF1, n_max, B)
    for ln in (1, 17, 133, 200):
        t = ln - 1
        sel = [x for x in range(t + 1) if _member(R.BF1, t // B, x // B)]
        o, lse = A.decode_attention(q, k, v, [ln], B, rp, ci, return_lse=True)
        assert abs(o[0, 0, 1] - np.mean(sel)) < 1e-9 and abs(lse[0, 0] - math.log(len(sel))) < 1e-12
    o1 = A.decode_attention(q, torch.randn(1, 1, n_max, 3, dtype=torch.float64), v, [1], B, rp, ci)
    assert np.array_equal(o1[0, 0], v[0, 0, 0].numpy())
    assert np.array_equal(A.decode_attention(q, k, v, [0], B, rp, ci), A.decode_attention(q, k, v, [1], B, rp, ci))
    assert np.array_equal(A.decode_attention(q, k, v, [999], B, rp, ci),
                          A.decode_attention(q, k, v, [200], B, rp, ci))


# --- backward ------------------------------------------------------------------------------

def _autograd_ref(q, k, v, d_o, kind, B, nl=2):
    """torch autograd through the library attention with an independently restated mask."""
    n = q.shape[2]
    G = q.shape[1] // k.shape[1]
    mask = torch.tensor([[s <= t and _member(kind, t // B, s // B, nl) for s in range(n)] for t in range(n)])
    qq, kk, vv = (x.clone().requires_grad_(True) for x in (q, k, v))
    o = F.scaled_dot_product_attention(qq, kk.repeat_interleave(G, 1), vv.repeat_interleave(G, 1), attn_mask=mask)
    o.backward(d_o)
    return qq.grad.numpy(), kk.grad.numpy(), vv.grad.numpy()


@pytest.mark.parametrize("kind", KINDS)
@pytest.mark.parametrize("n,B", [(96, 16), (75, 8)])
def test_backward_matches_autograd(kind, n, B):
    q, k, v = _qkv(2, 4, 2, n, 8, seed=41)
    d_o = torch.randn(q.shape, generator=torch.Generator("cpu").manual_seed(42), dtype=torch.float64)
    rp, ci = R.route_csr(kind, n, B)
    dq, dk, dv = A.attention_backward(q, k, v, d_o, B, rp, ci)
    rq, rk, rv = _autograd_ref(q, k, v, d_o, kind, B)
    for got, ref in ((dq, rq), (dk, rk), (dv, rv)):
        assert np.abs(got - ref).max() < 1e-10


def test_backward_finite_differences():
    # central differences of f = sum(O * dO) on a tiny BF1 problem, every input element
    n, B, d = 20, 4, 3
    q, k, v = _qkv(1, 2, 1, n, d, seed=43)
    d_o = torch.randn(q.shape, generator=torch.Generator("cpu").manual_seed(44), dtype=torch.float64)
    rp, ci = R.route_csr(R.BF1, n, B)
    dq, dk, dv = A.attention_backward(q, k, v, d_o, B, rp, ci)

    def f(qq, kk, vv):
        return float((A.attention(qq, kk, vv, B, rp, ci) * d_o.numpy()).sum())

    h = 1e-6
    for t, g in ((q, dq), (k, dk), (v, dv)):
        for idx in np.ndindex(*t.shape):
            tp, tm = t.clone(), t.clone()
            tp[idx] += h
            tm[idx] -= h
            args_p = [tp if x is t else x for x in (q, k, v)]
            args_m = [tm if x is t else x for x in (q, k, v)]
            fd = (f(*args_p) - f(*args_m)) / (2 * h)
            assert abs(fd - g[idx]) < 1e-6 * max(1.0, abs(g[idx])), (idx, fd, g[idx])


def test_backward_gqa_sums_repeated_heads():
    q, k, v = _qkv(1, 6, 2, 64, 8, seed=45)
    d_o = torch.randn(q.shape, generator=torch.Generator("cpu").manual_seed(46), dtype=torch.float64)
    rp, ci = R.route_csr(R.STATIC_RANDOM, 64, 8)
    dq, dk, dv = A.attention_backward(q, k, v, d_o, 8, rp, ci)
    rq, rk, rv = A.attention_backward(q, k.repeat_interleave(3, 1), v.repeat_interleave(3, 1), d_o, 8, rp, ci)
    assert np.abs(dq - rq).max() < 1e-12
    assert np.abs(dk - rk.reshape(1, 2, 3, 64, 8).sum(2)).max() < 1e-12
    assert np.abs(dv - rv.reshape(1, 2, 3, 64, 8).sum(2)).max() < 1e-12


def test_backward_row_subsets_match_full():
    n, B = 200, 16
    q, k, v = _qkv(1, 2, 2, n, 8, seed=47)
    d_o = torch.randn(q.shape, generator=torch.Generator("cpu").manual_seed(48), dtype=torch.float64)
    rp, ci = R.route_csr(R.BF1, n, B)
    full = A.attention_backward(q, k, v, d_o, B, rp, ci)
    qr, kr = np.array([0, 17, 100, 199]), np.array([3, 64, 150, 199])
    sub = A.attention_backward(q, k, v, d_o, B, rp, ci, q_rows=qr, k_rows=kr)
    assert np.array_equal(sub[0], full[0][:, :, qr])
    assert np.abs(sub[1] - full[1][:, :, kr]).max() < 1e-12 and np.abs(sub[2] - full[2][:, :, kr]).max() < 1e-12


def test_backward_excluded_keys_get_no_gradient():
    # block-diagonal route: a key's gradient comes only from its own chunk's queries, so keys of
    # a chunk whose dO is zero get exactly zero dk, dv
    n, B = 64, 16
    q, k, v = _qkv(1, 1, 1, n, 4, seed=49)
    d_o = torch.randn(q.shape, generator=torch.Generator("cpu").manual_seed(50), dtype=torch.float64)
    d_o[:, :, 16:32] = 0
    rp, ci = R.route_csr(R.BLOCK_DIAGONAL, n, B)
    dq, dk, dv = A.attention_backward(q, k, v, d_o, B, rp, ci)
    assert (dk[:, :, 16:32] == 0).all() and (dv[:, :, 16:32] == 0).all() and (dq[:, :, 16:32] == 0).all()
