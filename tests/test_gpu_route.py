"""GPU route builder vs the oracle's route sets: row_ptr and col_idx must be identical arrays."""

import numpy as np
import pytest
import torch

import long_context_block_amd as bsa
from oracle import routes as R
import synth

pytestmark = pytest.mark.gpu


def _gpu_route(kind, n, B, n_local=2, keep_first=1, n_random=14, seed=17):
    spec = bsa.route_spec(kind, n_local, keep_first, n_random, seed)
    rp, ci = bsa.build_route(spec, n, B)
    torch.cuda.synchronize()
    return rp.cpu().numpy(), ci.cpu().numpy()


def _oracle_route(kind, n, B, n_local=2, keep_first=1, n_random=14, seed=17):
    return R.route_csr(kind, n, B, n_local=n_local, keep_first=bool(keep_first), n_random=n_random, seed=seed)


@pytest.mark.parametrize("name", list(synth.WORKLOADS))
def test_workload_routes_bit_exact(name):
    w = synth.WORKLOADS[name]
    print(f"route {name}: kind={w.route_kind} n={w.n} B={w.block}", flush=True)
    kinds = [w.route_kind] + ([R.DENSE_CAUSAL] if name == "qwen3_32k" else [])
    for kind in kinds:
        g_rp, g_ci = _gpu_route(kind, w.n, w.block, w.n_local, w.keep_first, w.n_random, w.route_seed)
        o_rp, o_ci = _oracle_route(kind, w.n, w.block, w.n_local, w.keep_first, w.n_random, w.route_seed)
        assert np.array_equal(g_rp, o_rp)
        assert np.array_equal(g_ci, o_ci)
        bsa.bsa_check_route(g_rp, g_ci)


SWEEP = [
    (R.BF1, dict(n_local=2, keep_first=1)), (R.BF1, dict(n_local=0, keep_first=0)),
    (R.BF1, dict(n_local=5, keep_first=1)), (R.BF1, dict(n_local=3, keep_first=0)),
    (R.BLOCK_DIAGONAL, {}), (R.DENSE_CAUSAL, {}),
    (R.STATIC_RANDOM, dict(n_random=14, keep_first=1, seed=17)),
    (R.STATIC_RANDOM, dict(n_random=5, keep_first=0, seed=3)),
    (R.STATIC_RANDOM, dict(n_random=70, keep_first=1, seed=12345678901234)),
    (R.STATIC_RANDOM, dict(n_random=0, keep_first=1, seed=17)),
    (R.SLIDING_WINDOW, dict(n_local=0)), (R.SLIDING_WINDOW, dict(n_local=8)),
    (R.SLIDING_WINDOW, dict(n_local=70)),
]


@pytest.mark.parametrize("kind,params", SWEEP)
@pytest.mark.parametrize("n,B", [(1, 64), (63, 64), (65, 64), (1000, 64), (4097, 128), (20000, 128)])
def test_route_sweep_bit_exact(kind, params, n, B):
    g = _gpu_route(kind, n, B, **params)
    o = _oracle_route(kind, n, B, **params)
    assert np.array_equal(g[0], o[0]) and np.array_equal(g[1], o[1])


def test_empty_route():
    spec = bsa.route_spec(R.BF1)
    rp = torch.full((1,), -7, dtype=torch.int32, device="cuda")
    ci = torch.empty(0, dtype=torch.int32, device="cuda")
    assert bsa.bsa_build_route(spec, 0, 64, rp, ci) == 0
    torch.cuda.synchronize()
    assert rp.item() == 0


def test_capacity_error_leaves_nnz():
    spec = bsa.route_spec(R.BF1)
    rp = torch.empty(9, dtype=torch.int32, device="cuda")
    ci = torch.empty(28, dtype=torch.int32, device="cuda")
    with pytest.raises(bsa.BsaError) as e:
        bsa.bsa_build_route(spec, 512, 64, rp, ci)
    assert e.value.status == bsa.BSA_ERR_CAPACITY
