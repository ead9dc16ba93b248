"""Pins for the oracle's route sets (CPU only).

Each test ties oracle/routes.py to something other than itself: numbers the
pages print (tests/golden), closed forms derived from the definitions, an
independently written membership predicate, a published known-answer vector
for SplitMix64, and a uniformity test of the static-random sampler.
"""

import math

import numpy as np
import pytest

from oracle import routes as R


def _pow2(x: int) -> bool:
    return x > 0 and (x & (x - 1)) == 0


def _bf1_member(i: int, j: int, n_local: int, keep_first: bool) -> bool:
    """Independent restatement of BF1 membership as a predicate on the offset i - j."""
    if j > i or j < 0:
        return False
    off = i - j
    return off == 0 or off <= n_local or _pow2(off) or (keep_first and j == 0)


# --- pins from numbers printed on the pages -------------------------------------------

def test_bf1_selected_interaction_ratio_32k(golden):
    kv, _ = golden("bf1_selected_interactions_32k.txt")
    n, B, nl = int(kv["n"]), int(kv["block"]), int(kv["n_local"])
    sets = R.route_sets(R.BF1, R.num_blocks(n, B), n_local=nl)
    sel = R.selected_pairs(n, B, sets)
    dense = n * (n + 1) // 2
    assert dense == 536_887_296
    assert sel == 19_902_464
    assert round(dense / sel, 2) == float(kv["ratio_printed"])
    # dropping block 0 (a plausible misreading) would not reproduce the printed value
    sets_nofirst = R.route_sets(R.BF1, R.num_blocks(n, B), n_local=nl, keep_first=False)
    assert round(dense / R.selected_pairs(n, B, sets_nofirst), 2) != float(kv["ratio_printed"])
    # nor would block width 128 (the width of the GQA workload)
    sets128 = R.route_sets(R.BF1, R.num_blocks(n, 128), n_local=nl)
    assert round(dense / R.selected_pairs(n, 128, sets128), 2) != float(kv["ratio_printed"])


def test_bf1_max_shortest_path(golden):
    kv, _ = golden("bf1_depth.txt")
    nqb, nl = int(kv["nqb"]), int(kv["n_local"])
    assert R.max_shortest_path(R.route_sets(R.BF1, nqb, n_local=nl)) == int(kv["depth_printed"])


@pytest.mark.parametrize("nqb", [8, 64, 256])
def test_bf1_depth_closed_form(nqb):
    # every j -> i path: one hop through block 0 when j = 0; otherwise the dyadic offsets give
    # popcount(i - j) hops, maximised over 1 <= i - j <= nqb - 2 (j >= 1).
    want = max(bin(x).count("1") for x in range(1, nqb - 1)) if nqb > 2 else 1
    assert R.max_shortest_path(R.route_sets(R.BF1, nqb)) == want


# --- closed forms -----------------------------------------------------------------------

@pytest.mark.parametrize("n_local", [1, 2])
def test_bf1_row_length_closed_form(n_local):
    sets = R.route_sets(R.BF1, 600, n_local=n_local)
    assert len(sets[0]) == 1
    for i in range(1, 600):
        want = 2 + int(math.floor(math.log2(i))) + (0 if _pow2(i) else 1)
        if i == 1:
            want = 2
        assert len(sets[i]) == want, i


def test_bf1_tiny_rows_by_hand():
    # Derived by hand from the definition for 8 blocks (the tiny workload).
    want = [[0], [0, 1], [0, 1, 2], [0, 1, 2, 3], [0, 2, 3, 4], [0, 1, 3, 4, 5], [0, 2, 4, 5, 6],
            [0, 3, 5, 6, 7]]
    assert R.route_sets(R.BF1, 8, n_local=1) == want
    assert R.route_sets(R.BF1, 8, n_local=2) == want


@pytest.mark.parametrize("nqb,nnz", [(8, 29), (64, 442), (256, 2296), (512, 5111)])
def test_bf1_nnz(nqb, nnz):
    rp, ci = R.to_csr(R.route_sets(R.BF1, nqb))
    assert rp[-1] == nnz == len(ci)


def test_local_one_equals_local_two():
    # offset 2 is itself dyadic, so one and two local neighbours give the same route
    assert R.route_sets(R.BF1, 300, n_local=1) == R.route_sets(R.BF1, 300, n_local=2)
    assert R.route_sets(R.BF1, 300, n_local=3) != R.route_sets(R.BF1, 300, n_local=2)


@pytest.mark.parametrize("n_local,keep_first", [(0, True), (1, False), (2, True), (3, True), (5, False)])
def test_bf1_membership_predicate(n_local, keep_first):
    nqb = 80
    sets = R.route_sets(R.BF1, nqb, n_local=n_local, keep_first=keep_first)
    for i in range(nqb):
        want = [j for j in range(nqb) if _bf1_member(i, j, n_local, keep_first)]
        assert sets[i] == want


def test_dense_and_diagonal_closed_forms():
    for nqb in (1, 2, 7, 64, 256):
        rp, ci = R.to_csr(R.route_sets(R.DENSE_CAUSAL, nqb))
        assert rp[-1] == nqb * (nqb + 1) // 2
        rp, ci = R.to_csr(R.route_sets(R.BLOCK_DIAGONAL, nqb))
        assert list(ci) == list(range(nqb)) and list(rp) == list(range(nqb + 1))


def test_selected_pairs_closed_forms():
    for n, B in [(37, 8), (64, 8), (100, 16), (4096, 64)]:
        nqb = R.num_blocks(n, B)
        assert R.selected_pairs(n, B, R.route_sets(R.DENSE_CAUSAL, nqb)) == n * (n + 1) // 2
        diag = sum(m * (m + 1) // 2 for m in [min(B, n - b * B) for b in range(nqb)])
        assert R.selected_pairs(n, B, R.route_sets(R.BLOCK_DIAGONAL, nqb)) == diag


# --- static-random sampler -----------------------------------------------------------------

def test_splitmix64_known_answer(golden):
    _, vals = golden("splitmix64_seed0.txt")
    gamma, m64 = 0x9E3779B97F4A7C15, (1 << 64) - 1
    got = [R.splitmix64((k * gamma) & m64) for k in range(len(vals))]
    assert got == [int(v, 16) for v in vals]


def test_pair_hash_composition_known_answer(golden):
    """h(seed, i, j) = SM(seed XOR SM((i << 32) | j)) pinned by the same published vector: with i, j
    the high and low halves of the golden-ratio increment the inner call is SM(gamma), the second
    printed output; a seed equal to that output XOR 2 gamma turns the outer call into SM(2 gamma), the
    third.  A swapped (j, i) packing, a missing inner or outer step, or a sum in place of the XOR
    would each miss the printed value."""
    _, vals = golden("splitmix64_seed0.txt")
    ka = [int(v, 16) for v in vals]
    gamma, m64 = 0x9E3779B97F4A7C15, (1 << 64) - 1
    hi, lo = gamma >> 32, gamma & 0xFFFFFFFF
    assert R.pair_hash(ka[1] ^ ((2 * gamma) & m64), hi, lo) == ka[2]
    # i = j = 0: the inner call is SM(0), the first printed output
    assert R.pair_hash(ka[0] ^ gamma, 0, 0) == ka[1]
    assert R.pair_hash(ka[1] ^ ((2 * gamma) & m64), lo, hi) != ka[2]


@pytest.mark.parametrize("n_random,keep_first", [(14, True), (3, False)])
def test_static_random_structure(n_random, keep_first):
    nqb = 160
    sets = R.route_sets(R.STATIC_RANDOM, nqb, n_random=n_random, seed=17, keep_first=keep_first)
    for i, r in enumerate(sets):
        assert r == sorted(set(r)) and r[-1] == i
        n_cand = (i - 1 if keep_first else i) if i > 0 else 0
        assert len(r) == 1 + (1 if keep_first and i > 0 else 0) + min(n_random, max(n_cand, 0))
        if keep_first and i > 0:
            assert r[0] == 0
    if keep_first and n_random == 14:
        assert [len(r) for r in sets] == [min(i + 1, 16) for i in range(nqb)]


def test_static_random_seed_dependence():
    a = R.route_sets(R.STATIC_RANDOM, 128, seed=17)
    b = R.route_sets(R.STATIC_RANDOM, 128, seed=18)
    assert a != b
    assert [len(x) for x in a] == [len(x) for x in b]


def test_static_random_uniform():
    # chi-square test of the marginal position of drawn blocks within their candidate range
    nqb, K = 1200, 10
    counts = np.zeros(K)
    for i in range(100, nqb):
        r = R.static_random_set(i, 14, 17, True)
        for j in r - {0, i}:
            counts[((j - 1) * K) // (i - 1)] += 1
    exp = counts.sum() / K
    chi2 = float(((counts - exp) ** 2 / exp).sum())
    assert chi2 < 27.88  # 9 dof, p = 0.001


def test_csr_roundtrip_and_partial_block():
    n, B = 37, 8
    rp, ci = R.route_csr(R.BF1, n, B)
    assert len(rp) == R.num_blocks(n, B) + 1 == 6
    assert R.csr_to_sets(rp, ci) == R.route_sets(R.BF1, 5)


# --- local sliding band (BF1's equal-budget local control) ---------------------------------

@pytest.mark.parametrize("n_local", [0, 1, 3, 8])
def test_sliding_window_closed_forms(n_local):
    nqb = 200
    sets = R.route_sets(R.SLIDING_WINDOW, nqb, n_local=n_local)
    # membership predicate, written independently: 0 <= i - j <= n_local
    for i in range(nqb):
        assert sets[i] == [j for j in range(nqb) if 0 <= i - j <= n_local]
    # nnz = sum_i min(i + 1, n_local + 1) = W * nqb - W (W - 1) / 2 for W = n_local + 1 <= nqb
    W = n_local + 1
    rp, ci = R.to_csr(sets)
    assert rp[-1] == len(ci) == W * nqb - W * (W - 1) // 2


def test_sliding_window_degenerate_cases():
    nqb = 50
    assert R.route_sets(R.SLIDING_WINDOW, nqb, n_local=0) == R.route_sets(R.BLOCK_DIAGONAL, nqb)
    assert R.route_sets(R.SLIDING_WINDOW, nqb, n_local=nqb - 1) == R.route_sets(R.DENSE_CAUSAL, nqb)
    assert R.route_sets(R.SLIDING_WINDOW, nqb, n_local=10 * nqb) == R.route_sets(R.DENSE_CAUSAL, nqb)


@pytest.mark.parametrize("nqb,n_local", [(8, 1), (64, 2), (256, 8), (100, 7)])
def test_sliding_window_depth_closed_form(nqb, n_local):
    # a hop moves at most n_local blocks forward, and n_local-sized hops are always available:
    # the worst pair (0, nqb - 1) needs ceil((nqb - 1) / n_local) hops
    want = -(-(nqb - 1) // n_local)
    assert R.max_shortest_path(R.route_sets(R.SLIDING_WINDOW, nqb, n_local=n_local)) == want


def test_sliding_window_selected_pairs_closed_form():
    # full blocks of B tokens: a row with k off-diagonal blocks selects k B^2 + B (B + 1) / 2
    n, B, nl = 64 * 16, 16, 5
    nqb = n // B
    want = sum(min(i, nl) * B * B + B * (B + 1) // 2 for i in range(nqb))
    assert R.selected_pairs(n, B, R.route_sets(R.SLIDING_WINDOW, nqb, n_local=nl)) == want
