"""Routes for the GPU parity tests: the kernels run on the route bsa_build_route writes on the
GPU, the oracle on the one oracle/routes.py builds from the same parameters, and the two are
checked equal entry by entry first (so no oracle input comes from the HIP path)."""

import functools

import numpy as np

import long_context_block_amd as bsa
from oracle import routes as R


@functools.lru_cache(maxsize=None)
def oracle_route(kind, n, B, n_local=2, keep_first=1, n_random=14, seed=17):
    rp, ci = R.route_csr(kind, n, B, n_local=n_local, keep_first=bool(keep_first), n_random=n_random, seed=seed)
    rp.flags.writeable = False
    ci.flags.writeable = False
    return rp, ci


def routes(kind, n, B, n_local=2, keep_first=1, n_random=14, seed=17):
    """((row_ptr, col_idx) on the GPU, (row_ptr, col_idx) from the oracle), checked equal."""
    rp, ci = bsa.build_route(bsa.route_spec(kind, n_local, keep_first, n_random, seed), n, B)
    orp, oci = oracle_route(kind, n, B, n_local, int(bool(keep_first)), n_random, seed)
    assert np.array_equal(rp.cpu().numpy(), orp) and np.array_equal(ci.cpu().numpy(), oci), \
        ("GPU route differs from the oracle's", kind, n, B)
    return (rp, ci), (orp, oci)


def workload_routes(w, kind=None):
    kind = w.route_kind if kind is None else kind
    return routes(kind, w.n, w.block, w.n_local, w.keep_first, w.n_random, w.route_seed)
