"""GPU forward parity: bsa_forward (through the C ABI) against the fp64 oracle.

Bars: bf16 inputs — max-abs <= 1e-2 and relative L2 <= 5e-3; fp32 inputs — both <= 1e-5.
Full outputs are compared at sizes the oracle finishes in seconds (several tiles and a ragged
tail); at the full workload sizes, in the launch configuration bench.py times, a sample of
query rows (first/last rows of blocks, every block's diagonal, random rows) is compared.
"""

import math

import numpy as np
import pytest
import torch

import long_context_block_amd as bsa
from oracle import attn as A
from oracle import routes as R
import synth
from route_ref import workload_routes

pytestmark = pytest.mark.gpu

BF16_MAXABS, BF16_RELL2 = 1e-2, 5e-3
FP32_TOL = 1e-5


def tol(dtype):
    return (FP32_TOL, FP32_TOL) if dtype == torch.float32 else (BF16_MAXABS, BF16_RELL2)


def errors(got, ref):
    got = np.asarray(got, dtype=np.float64)
    d = got - ref
    return float(np.abs(d).max()), float(np.linalg.norm(d) / np.linalg.norm(ref))


def route_for(w, kind=None):
    return workload_routes(w, kind)[0]


def run_gpu(w, q, k, v, kind=None, with_lse=False, stream=None):
    (rp, ci), oracle_rc = workload_routes(w, kind)
    qd, kd, vd = q.cuda(), k.cuda(), v.cuda()
    out = bsa.forward(qd, kd, vd, rp, ci, w.block, with_lse=with_lse, stream=stream)
    torch.cuda.synchronize()
    if not with_lse:
        out = (out, None)
    return out, oracle_rc


def sample_rows(n, B, rng, extra=24):
    nqb = -(-n // B)
    rows = {0, 1, n - 1, min(B - 1, n - 1)}
    for blk in rng.choice(nqb, size=min(nqb, 8), replace=False):
        rows |= {int(blk) * B, min(int(blk) * B + B - 1, n - 1), min(int(blk) * B + B // 2, n - 1)}
    rows |= set(int(x) for x in rng.integers(0, n, size=extra))
    return np.array(sorted(rows))


def check(w, kind=None, rows=None, with_lse=True):
    q, k, v = synth.make_qkv(w)
    (o, lse), (rp, ci) = run_gpu(w, q, k, v, kind, with_lse=True)
    ref, ref_lse = A.attention(q, k, v, w.block, rp, ci, rows=rows, return_lse=True)
    got = o.float().cpu().numpy()
    gl = lse.cpu().numpy()
    if rows is not None:
        got, gl = got[:, :, rows], gl[:, :, rows]
    mx, rl2 = errors(got, ref)
    lse_err = float(np.abs(gl - ref_lse).max())
    print(f"{w.name} kind={kind if kind is not None else w.route_kind}: max-abs {mx:.3e} rel-L2 {rl2:.3e} "
          f"lse {lse_err:.3e}", flush=True)
    ma, rt = tol(w.torch_dtype)
    assert mx <= ma and rl2 <= rt
    # the bf16 path sums the bf16-rounded weights, so LSE may be off by up to ln(1 + 2^-9) ~ 1.95e-3
    assert lse_err <= (1e-5 if w.dtype == "fp32" else 2.5e-3)
    return o


# ---- reduced sizes, full outputs (several tiles + a ragged tail) ------------------------------

REDUCED = [
    synth.WORKLOADS["tiny"],
    synth.WORKLOADS["tiny"].resized(name="tiny-ragged", n=500, heads_q=2, heads_kv=1),
    synth.WORKLOADS["tiny"].resized(name="tiny-d128-b128", n=700, d=128, block=128, heads_q=2, heads_kv=2),
    synth.WORKLOADS["bf1_4k"],
    synth.WORKLOADS["bf1_4k"].resized(name="bf1-ragged", n=1000, heads_q=4, heads_kv=4),
    synth.WORKLOADS["bsbr_chunk_8k"].resized(name="bsbr-ragged", n=1500, batch=2),
    synth.WORKLOADS["qwen3_32k"].resized(name="qwen3-reduced", n=2000),
    synth.WORKLOADS["qwen3_32k"].resized(name="qwen3-dense-reduced", n=2000, route_kind=R.DENSE_CAUSAL),
    synth.WORKLOADS["static_random_64k"].resized(name="static-random-reduced", n=3000, heads_q=4, heads_kv=4),
    synth.WORKLOADS["bf1_4k"].resized(name="gqa4-d64-b64", n=1100, d=64, heads_q=8, heads_kv=2),
    synth.WORKLOADS["bf1_4k"].resized(name="gqa3-d64-b128", n=900, d=64, block=128, heads_q=6, heads_kv=2),
    synth.WORKLOADS["bf1_4k"].resized(name="mqa-d128-b64", n=777, heads_q=4, heads_kv=1, batch=2),
    synth.WORKLOADS["qwen3_32k"].resized(name="sliding-reduced", n=2100, route_kind=R.SLIDING_WINDOW, n_local=3),
    synth.WORKLOADS["bf1_4k"].resized(name="sliding-d64-b64", n=1300, d=64, heads_q=4, heads_kv=4,
                                      route_kind=R.SLIDING_WINDOW, n_local=5),
]


@pytest.mark.parametrize("w", REDUCED, ids=[w.name for w in REDUCED])
def test_parity_full_output(w):
    check(w)


# ---- full workload sizes, sampled rows -------------------------------------------------------

FULL = ["bsbr_chunk_8k", "qwen3_32k", "static_random_64k"]


@pytest.mark.parametrize("name", FULL)
def test_parity_full_size_sampled(name):
    w = synth.WORKLOADS[name]
    rows = sample_rows(w.n, w.block, np.random.default_rng(7))
    check(w, rows=rows)


@pytest.mark.parametrize("kind,params", [(R.SLIDING_WINDOW, dict(n_local=8)), (R.STATIC_RANDOM, dict(n_random=7))])
def test_parity_full_size_topology_controls_sampled(kind, params):
    # the equal-budget controls of the topology sweep, at the 32K GQA shape
    w = synth.WORKLOADS["qwen3_32k"].resized(route_kind=kind, **params)
    rows = sample_rows(w.n, w.block, np.random.default_rng(9), extra=12)
    check(w, rows=rows)


def test_parity_full_size_dense_route_sampled():
    w = synth.WORKLOADS["qwen3_32k"]
    rows = sample_rows(w.n, w.block, np.random.default_rng(8), extra=8)
    check(w, kind=R.DENSE_CAUSAL, rows=rows)


# ---- edge cases ----------------------------------------------------------------------------

@pytest.mark.parametrize("n", [1, 2, 63, 64, 65, 129])
@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
def test_tiny_and_partial_blocks(n, dtype):
    w = synth.WORKLOADS["bf1_4k"].resized(name=f"n{n}", n=n, heads_q=2, heads_kv=1, d=64, dtype=dtype)
    check(w)


def test_empty_inputs():
    w = synth.WORKLOADS["bf1_4k"]
    q = torch.empty(1, 16, 0, 128, dtype=torch.bfloat16, device="cuda")
    rp = torch.zeros(1, dtype=torch.int32, device="cuda")
    ci = torch.empty(0, dtype=torch.int32, device="cuda")
    o = torch.empty_like(q)
    bsa.bsa_forward(q, q, q, o, rp, ci, w.block)
    qb = torch.empty(0, 16, 64, 128, dtype=torch.bfloat16, device="cuda")
    rp2, ci2 = route_for(w.resized(n=64))
    bsa.bsa_forward(qb, qb, qb, torch.empty_like(qb), rp2, ci2, 64)


def test_first_row_equals_v0():
    w = synth.WORKLOADS["qwen3_32k"].resized(n=1024)
    q, k, v = synth.make_qkv(w)
    (o, _), _ = run_gpu(w, q, k, v)
    G = w.heads_q // w.heads_kv
    ref = v[:, torch.arange(w.heads_q) // G, 0].float()
    assert torch.equal(o[:, :, 0].float().cpu(), ref)


@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
def test_uniform_weights_when_k_is_zero(dtype):
    # K = 0: every selected weight is exactly equal, so O[t] is the mean of V over sel(t); with
    # V[:, 0] = 1, V[:, 1] = s/n, V[:, 2] = (s/n)^2 this pins which tokens the kernel selects.
    for kind in (R.BF1, R.STATIC_RANDOM, R.BLOCK_DIAGONAL, R.DENSE_CAUSAL, R.SLIDING_WINDOW):
        w = synth.WORKLOADS["bf1_4k"].resized(n=777, heads_q=1, heads_kv=1, d=64, dtype=dtype, route_kind=kind)
        dt = w.torch_dtype
        q = torch.randn(1, 1, w.n, 64).to(dt)
        k = torch.zeros(1, 1, w.n, 64, dtype=dt)
        s = torch.arange(w.n, dtype=torch.float64) / w.n
        v = torch.zeros(1, 1, w.n, 64, dtype=torch.float64)
        v[..., 0], v[..., 1], v[..., 2] = 1.0, s, s * s
        v = v.to(dt)
        (o, _), (rp, ci) = run_gpu(w, q, k, v)
        sets = R.csr_to_sets(rp, ci)
        vv = v[0, 0].double().numpy()
        got = o[0, 0].double().cpu().numpy()
        for t in range(w.n):
            sel = [x for j in sets[t // w.block] for x in range(j * w.block, min((j + 1) * w.block, t + 1))]
            want = vv[sel, :3].mean(0)
            assert abs(got[t, 0] - 1.0) <= (1e-6 if dtype == "fp32" else 4e-3)
            assert np.abs(got[t, :3] - want).max() <= (1e-6 if dtype == "fp32" else 8e-3), (kind, t)


def test_future_leakage_is_zero():
    w = synth.WORKLOADS["qwen3_32k"].resized(n=3000)
    q, k, v = synth.make_qkv(w)
    (o1, _), _ = run_gpu(w, q, k, v)
    for t in (0, 700, 1919, 2000):
        k2, v2 = k.clone(), v.clone()
        k2[:, :, t + 1:] = torch.randn_like(k2[:, :, t + 1:].float()).to(k2.dtype) * 3
        v2[:, :, t + 1:] = torch.randn_like(v2[:, :, t + 1:].float()).to(v2.dtype) * 3
        (o2, _), _ = run_gpu(w, q, k2, v2)
        assert torch.equal(o1[:, :, :t + 1], o2[:, :, :t + 1]), t
        assert not torch.equal(o1[:, :, t + 1:], o2[:, :, t + 1:])


@pytest.mark.parametrize("d", [64, 128])
def test_gqa_equals_repeated_kv(d):
    # query head h reads key/value head h // G.  At d = 64 the GQA and the repeated-KV launches
    # run the same per-head arithmetic (bitwise equal); at d = 128 the GQA launch takes its
    # online-softmax steps over 32 keys instead of 64, so the two agree to rounding.
    w = synth.WORKLOADS["qwen3_32k"].resized(n=1500, d=d)
    q, k, v = synth.make_qkv(w)
    (o1, _), _ = run_gpu(w, q, k, v)
    G = w.heads_q // w.heads_kv
    wr = w.resized(heads_kv=w.heads_q)
    (o2, _), _ = run_gpu(wr, q, k.repeat_interleave(G, 1), v.repeat_interleave(G, 1))
    if d == 64:
        assert torch.equal(o1, o2)
    else:
        mx, rl2 = errors(o1.float().cpu().numpy(), o2.double().cpu().numpy())
        assert mx <= BF16_MAXABS and rl2 <= BF16_RELL2


def test_deterministic_and_non_default_stream():
    w = synth.WORKLOADS["static_random_64k"].resized(n=5000, heads_q=4, heads_kv=4)
    q, k, v = synth.make_qkv(w)
    (o1, _), _ = run_gpu(w, q, k, v)
    (o2, _), _ = run_gpu(w, q, k, v)
    assert torch.equal(o1, o2)
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        (o3, _), _ = run_gpu(w, q, k, v, stream=s)
    s.synchronize()
    assert torch.equal(o1, o3)


def test_dense_causal_ref_equals_forward_on_dense_route():
    w = synth.WORKLOADS["qwen3_32k"].resized(n=2500)
    q, k, v = synth.make_qkv(w)
    (o1, _), _ = run_gpu(w, q, k, v, kind=R.DENSE_CAUSAL)
    ws = torch.empty(bsa.bsa_dense_route_workspace_bytes(w.n, w.block) // 4, dtype=torch.int32, device="cuda")
    o2 = torch.empty_like(o1)
    bsa.bsa_dense_causal_ref(q.cuda(), k.cuda(), v.cuda(), o2, ws, w.block)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2)


def test_explicit_scale():
    w = synth.WORKLOADS["bf1_4k"].resized(n=600, heads_q=2, heads_kv=2)
    q, k, v = synth.make_qkv(w)
    (rp, ci), (orp, oci) = workload_routes(w)
    o = bsa.forward(q.cuda(), k.cuda(), v.cuda(), rp, ci, w.block, scale=0.05)
    torch.cuda.synchronize()
    ref = A.attention(q, k, v, w.block, orp, oci, scale=0.05)
    mx, rl2 = errors(o.float().cpu().numpy(), ref)
    assert mx <= BF16_MAXABS and rl2 <= BF16_RELL2


def test_validate_route_env(monkeypatch):
    w = synth.WORKLOADS["bf1_4k"].resized(n=512, heads_q=1, heads_kv=1)
    q, k, v = (x.cuda() for x in synth.make_qkv(w))
    rp, ci = route_for(w)
    monkeypatch.setenv("BSA_VALIDATE_ROUTE", "1")
    bsa.forward(q, k, v, rp, ci, w.block)
    bad = ci.clone()
    bad[1] = 5  # row 1 reads a future block
    with pytest.raises(bsa.BsaError) as e:
        bsa.forward(q, k, v, rp, bad, w.block)
    assert e.value.status == bsa.BSA_ERR_BAD_ROUTE
