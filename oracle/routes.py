"""Route sets for causal block-sparse attention — oracle (test infrastructure only).

Vocabulary.  A sequence of ``n`` tokens is cut into query/key blocks of ``B``
tokens; block ``b`` holds tokens ``[b*B, min((b+1)*B, n))`` and there are
``nqb = ceil(n / B)`` blocks ("Block Sparse Attention in LLMs", section 3 "Why
block sparse?"; "Block-Sparse Attention", "How It Works").  A *route* gives,
for every query block ``i``, the set ``R(i)`` of key blocks it reads — the
block mask M_B of "Block-Sparse Attention" ("Math Or Compute Schema", the
block-sparse formula), stored as an adjacency list like the
``allowed_blocks`` dictionary of "Block Sparse Attention in LLMs" (section 6
"GPU implementation view").

Route kinds:

* BF1 ("BF1: A Causal Dyadic Sparse-Attention Retrofit ...", Method; section
  3.1 "Causal dyadic block graph"): the block itself, a small local
  neighbourhood of predecessors, the first block, and predecessors at dyadic
  offsets.  Reading used here: offsets are in blocks, the dyadic offsets are
  ``2**k`` for every ``k >= 0`` with ``2**k <= i``.
* Block-diagonal: the within-chunk term of BSBR ("bsbr", "Solution", the
  within-chunk causal mask M_in): every block reads only itself.
* Dense causal: every block reads all blocks ``0..i`` — dense causal
  attention expressed as a route.
* Static-random: BF1's topology control, a fixed random nonlocal graph at a
  matched pair budget drawn from a fixed seed ("BF1 ...", Abstract and
  section 5 "Topology control"; section 8 names seed 17).  The pages do not
  give the generator; the reading used here: the block itself, block 0, and
  ``m = min(n_random, #candidates)`` earlier blocks drawn uniformly without
  replacement, realised as the ``m`` candidates with the smallest key
  ``(h(seed, i, j), j)`` where ``h`` is built from the SplitMix64 output
  function (Steele, Lea & Flood, "Fast splittable pseudorandom number
  generators", OOPSLA 2014).
* Sliding window: BF1's equal-budget *local* control ("BF1 ...", Abstract:
  equal-budget local sliding; section 5 "Topology control" and
  "Communication depth": matched sliding).  Reading used here: a fixed band
  aligned to blocks, the block itself and its ``n_local`` predecessors — the
  fixed-band local pattern that "Block-Sparse Attention" compares against
  (sliding-window attention), at block granularity.  The pages do not give
  the band width of their matched control; a caller matches it to another
  route's budget.

Everything here is plain Python integers / sets; CSR conversion uses numpy.
"""

from __future__ import annotations

from collections import deque

import numpy as np

BF1 = 0
BLOCK_DIAGONAL = 1
DENSE_CAUSAL = 2
STATIC_RANDOM = 3
SLIDING_WINDOW = 4

KIND_NAMES = {BF1: "bf1", BLOCK_DIAGONAL: "block_diagonal",
              DENSE_CAUSAL: "dense_causal", STATIC_RANDOM: "static_random",
              SLIDING_WINDOW: "sliding_window"}

_MASK64 = (1 << 64) - 1
_GOLDEN_GAMMA = 0x9E3779B97F4A7C15


def num_blocks(n: int, B: int) -> int:
    """nqb = ceil(n / B): the number of (possibly partial) token blocks."""
    return -(-n // B)


# ---------------------------------------------------------------------------
# SplitMix64 (Steele, Lea & Flood 2014) — used only by the static-random route.
# ---------------------------------------------------------------------------

def splitmix64(x: int) -> int:
    """First output of a SplitMix64 generator whose state is ``x``.

    The generator advances its 64-bit state by the golden-ratio increment and
    returns the state passed through the variant-13 finaliser (xor-shift 30,
    multiply, xor-shift 27, multiply, xor-shift 31), all modulo 2**64.
    """
    z = (x + _GOLDEN_GAMMA) & _MASK64
    z = ((z ^ (z >> 30)) * 0xBF58476D1CE4E5B9) & _MASK64
    z = ((z ^ (z >> 27)) * 0x94D049BB133111EB) & _MASK64
    return z ^ (z >> 31)


def pair_hash(seed: int, i: int, j: int) -> int:
    """h(seed, i, j) = SM(seed XOR SM((i << 32) | j)) on unsigned 64-bit words."""
    return splitmix64((seed & _MASK64) ^ splitmix64(((i << 32) | j) & _MASK64))


# ---------------------------------------------------------------------------
# Route sets R(i)
# ---------------------------------------------------------------------------

def bf1_set(i: int, n_local: int = 2, keep_first: bool = True) -> set[int]:
    """BF1 key blocks of query block i.

    Follows "BF1: A Causal Dyadic Sparse-Attention Retrofit ...", Method and
    section 3.1: the block itself (read causally), ``n_local`` local
    predecessors, the first block, and predecessors at dyadic offsets
    ``i - 2**k`` (k >= 0).
    """
    s = {i}
    s |= {i - l for l in range(1, n_local + 1) if i - l >= 0}
    k = 0
    while (1 << k) <= i:
        s.add(i - (1 << k))
        k += 1
    if keep_first:
        s.add(0)
    return s


def block_diagonal_set(i: int) -> set[int]:
    """BSBR within-chunk term ("bsbr", Solution, mask M_in): block i reads itself."""
    return {i}


def dense_causal_set(i: int) -> set[int]:
    """Dense causal attention as a route: block i reads blocks 0..i."""
    return set(range(i + 1))


def static_random_set(i: int, n_random: int = 14, seed: int = 17,
                      keep_first: bool = True) -> set[int]:
    """Static-random nonlocal graph (BF1 topology control; seed 17 in section 8).

    Candidates are the earlier blocks not already kept: ``1..i-1`` when block 0
    is kept, else ``0..i-1``.  The ``m = min(n_random, #candidates)`` drawn
    blocks are the candidates with the smallest ``(pair_hash(seed, i, j), j)``.
    """
    s = {i}
    if i == 0:
        return s
    if keep_first:
        s.add(0)
        cands = range(1, i)
    else:
        cands = range(0, i)
    m = min(n_random, len(cands))
    ranked = sorted(cands, key=lambda j: (pair_hash(seed, i, j), j))
    s |= set(ranked[:m])
    return s


def sliding_window_set(i: int, n_local: int) -> set[int]:
    """Local sliding band (BF1's equal-budget local control): blocks i-n_local .. i, clipped at 0."""
    return {j for j in range(i - n_local, i + 1) if j >= 0}


def route_sets(kind: int, nqb: int, n_local: int = 2, keep_first: bool = True,
               n_random: int = 14, seed: int = 17) -> list[list[int]]:
    """All rows R(0..nqb-1), each sorted ascending (so the self block is last)."""
    out = []
    for i in range(nqb):
        if kind == BF1:
            s = bf1_set(i, n_local, keep_first)
        elif kind == BLOCK_DIAGONAL:
            s = block_diagonal_set(i)
        elif kind == DENSE_CAUSAL:
            s = dense_causal_set(i)
        elif kind == STATIC_RANDOM:
            s = static_random_set(i, n_random, seed, keep_first)
        elif kind == SLIDING_WINDOW:
            s = sliding_window_set(i, n_local)
        else:
            raise ValueError(f"unknown route kind {kind}")
        out.append(sorted(s))
    return out


def to_csr(sets: list[list[int]]) -> tuple[np.ndarray, np.ndarray]:
    """CSR encoding: row_ptr = exclusive prefix sum of |R(i)|, col_idx = rows concatenated."""
    row_ptr = np.zeros(len(sets) + 1, dtype=np.int64)
    for i, r in enumerate(sets):
        row_ptr[i + 1] = row_ptr[i] + len(r)
    col_idx = np.array([j for r in sets for j in r], dtype=np.int64)
    return row_ptr.astype(np.int32), col_idx.astype(np.int32)


def route_csr(kind: int, n: int, B: int, **params) -> tuple[np.ndarray, np.ndarray]:
    """CSR route for a sequence of n tokens at block width B."""
    return to_csr(route_sets(kind, num_blocks(n, B), **params))


def csr_to_sets(row_ptr, col_idx) -> list[list[int]]:
    rp = [int(x) for x in row_ptr]
    ci = [int(x) for x in col_idx]
    return [ci[rp[i]:rp[i + 1]] for i in range(len(rp) - 1)]


# ---------------------------------------------------------------------------
# Graph properties quoted on the pages
# ---------------------------------------------------------------------------

def selected_pairs(n: int, B: int, sets: list[list[int]]) -> int:
    """Selected causal token pairs (t, s), s <= t < n, with block(s) in R(block(t)).

    The counting convention of "BF1 ...", section 5 "Per-layer prefill
    scaling" (selected interactions vs dense causal): the diagonal is included,
    so the dense count is n(n+1)/2.
    """
    total = 0
    for i, r in enumerate(sets):
        t0, t1 = i * B, min((i + 1) * B, n)
        for t in range(t0, t1):
            for j in r:
                s0, s1 = j * B, min((j + 1) * B, n, t + 1)
                if s1 > s0:
                    total += s1 - s0
    return total


def max_shortest_path(sets: list[list[int]]) -> int:
    """Largest shortest-path length over ordered pairs j < i in the block graph.

    Edge j -> i whenever j is in R(i) (block i reads block j, so information
    moves from j to i in one attention layer) — the "communication depth" of
    "BF1 ...", sections 3.3 "Dyadic reachability" and 5 "Communication depth".
    Unreachable pairs raise.
    """
    nqb = len(sets)
    succ = [[] for _ in range(nqb)]
    for i, r in enumerate(sets):
        for j in r:
            if j != i:
                succ[j].append(i)
    worst = 0
    for src in range(nqb):
        dist = [-1] * nqb
        dist[src] = 0
        dq = deque([src])
        while dq:
            u = dq.popleft()
            for w in succ[u]:
                if dist[w] < 0:
                    dist[w] = dist[u] + 1
                    dq.append(w)
        for dst in range(src + 1, nqb):
            if dist[dst] < 0:
                raise ValueError(f"block {dst} unreachable from {src}")
            worst = max(worst, dist[dst])
    return worst
