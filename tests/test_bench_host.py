"""Host-side helpers of bench.py (CPU only): selected-pair counting and the communication-depth
BFS, checked against the oracle's definitions."""

import numpy as np
import pytest

import bench
from oracle import routes as R


@pytest.mark.parametrize("kind,params", [(R.BF1, {}), (R.SLIDING_WINDOW, dict(n_local=8)),
                                         (R.DENSE_CAUSAL, {}), (R.BLOCK_DIAGONAL, {}),
                                         (R.STATIC_RANDOM, dict(n_random=5))])
@pytest.mark.parametrize("n,B", [(4096, 64), (1000, 64), (777, 128)])
def test_selected_pairs_matches_oracle(kind, params, n, B):
    rp, ci = R.route_csr(kind, n, B, **params)
    assert bench.selected_pairs(rp, ci, n, B) == R.selected_pairs(n, B, R.csr_to_sets(rp, ci))


@pytest.mark.parametrize("kind,params,nqb", [(R.BF1, {}, 256), (R.BF1, {}, 64), (R.SLIDING_WINDOW, dict(n_local=8), 256),
                                             (R.DENSE_CAUSAL, {}, 40)])
def test_graph_depth_matches_oracle(kind, params, nqb):
    sets = R.route_sets(kind, nqb, **params)
    rp, ci = R.to_csr(sets)
    assert bench.graph_depth(rp, ci) == (R.max_shortest_path(sets), 0)


def test_graph_depth_counts_unreachable_pairs():
    # block-diagonal: no block reaches any other
    rp, ci = R.to_csr(R.route_sets(R.BLOCK_DIAGONAL, 10))
    assert bench.graph_depth(rp, ci) == (0, 45)


def test_algorithmic_bytes():
    import synth
    w = synth.WORKLOADS["qwen3_32k"]
    assert bench.algorithmic_bytes(w) == 2 * 32768 * 128 * (2 * 16 + 2 * 8)
    assert bench.algorithmic_bytes(synth.WORKLOADS["tiny"]) == 4 * 512 * 64 * 4


def test_multi_gpu_request_exits():
    import subprocess
    import sys
    r = subprocess.run([sys.executable, bench.__file__, "--gpus", "2"], capture_output=True, text=True)
    assert r.returncode == 2 and "one GPU" in r.stderr
