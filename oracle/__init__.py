"""CPU oracle for causal block-sparse attention forward — TEST INFRASTRUCTURE ONLY.

This package is the plain, slow, obviously-correct definition of what the GPU
path computes, written in numpy float64 from the source pages:

* ``routes``  — the per-query-block key-block sets (BF1 causal dyadic route,
  the BSBR within-chunk block-diagonal route, the dense causal route, a
  seeded static-random nonlocal graph and the local sliding band), their CSR
  encoding, and graph properties (selected token pairs, shortest-path depth).
* ``attn``    — block-sparse attention as masked dense softmax attention:
  the route is expanded to an explicit token mask which is applied before the
  softmax, so excluded pairs get weight exactly zero.
* ``bsbr``    — the BSBR between-chunk retrieval term (chunk states K^T V,
  meta attention over strictly earlier chunks, read-out by each token's
  query), added to the within-chunk (block-diagonal) attention.

Who may use it: only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py``.  The product path (the C-ABI library and
its Python binding in ``long_context_block_amd``) never imports, calls or
links anything here, and nothing here imports the product path.  The two
share only the seeded input generators in ``synth.py`` (which hold none of the
method's arithmetic).

Pins (what ties this oracle to something other than itself) live in
``tests/test_oracle_routes.py``, ``tests/test_oracle_attn.py`` and
``tests/test_oracle_bsbr.py``; each function
below names the passage it follows.  Functions with no pin say "parity
unpinned" in their docstring.
"""

from . import routes, attn, bsbr  # noqa: F401
