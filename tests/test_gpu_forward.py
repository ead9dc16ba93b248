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
    # 64-token blocks with GQA pairs (the pipelined kernel with one 64-key step per chunk): rows of
    # odd and even lengths, ragged tails, both d
    synth.WORKLOADS["qwen3_32k"].resized(name="qwen3-b64-reduced", n=2000, block=64),
    synth.WORKLOADS["qwen3_32k"].resized(name="qwen3-b64-dense-reduced", n=1500, block=64, route_kind=R.DENSE_CAUSAL),
    synth.WORKLOADS["qwen3_32k"].resized(name="qwen3-b64-static-random", n=2500, block=64, route_kind=R.STATIC_RANDOM,
                                         n_random=5),
    synth.WORKLOADS["qwen3_32k"].resized(name="gqa2-d64-b64-sliding", n=999, d=64, block=64, heads_q=4, heads_kv=2,
                                         route_kind=R.SLIDING_WINDOW, n_local=3, batch=2),
    # multi-head d = 64 at 128-token blocks over rows of several blocks (the pipelined kernel with
    # 128-key chunks and one head per work-group), and odd GQA groups at d = 128
    synth.WORKLOADS["qwen3_32k"].resized(name="mha-d64-b128-bf1", n=1500, d=64, heads_q=3, heads_kv=3),
    synth.WORKLOADS["qwen3_32k"].resized(name="gqa3-d128-b128-bf1", n=1400, heads_q=6, heads_kv=2),
    # GQA pairs at d = 64 and 128-token blocks (the headline kernel's d = 64 instantiation)
    synth.WORKLOADS["qwen3_32k"].resized(name="gqa2-d64-b128-bf1", n=1300, d=64, heads_q=4, heads_kv=2, batch=2),
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


@pytest.mark.parametrize("kind", [R.BF1, R.DENSE_CAUSAL])
def test_parity_full_size_b64_sampled(kind):
    # the 32K GQA shape at 64-token blocks (the width the pages' 32K figures use)
    w = synth.WORKLOADS["qwen3_32k"].resized(name="qwen3_32k_b64", block=64)
    rows = sample_rows(w.n, w.block, np.random.default_rng(12), extra=8)
    check(w, kind=kind, rows=rows)


# Persistent launches whose items do not split evenly over the XCDs (the plain serpentine walk),
# several items per work-group, batch > 1 and a ragged last block, for the three pipelined
# instantiations that take the pages' shapes: 128-token blocks with GQA pairs, multi-head d = 128
# with 64-key chunks, 64-token blocks with GQA pairs.
MANY_ITEMS = [
    synth.WORKLOADS["qwen3_32k"].resized(name="gqa-pairs-b128-batch3-ragged", batch=3, heads_q=6, heads_kv=3, n=33000),
    synth.WORKLOADS["static_random_64k"].resized(name="mha-b128-batch2-ragged", batch=2, heads_q=5, heads_kv=5,
                                                 n=20000),
    synth.WORKLOADS["qwen3_32k"].resized(name="gqa-pairs-b64-batch2-ragged", batch=2, heads_q=6, heads_kv=3,
                                         n=17000, block=64),
]


@pytest.mark.parametrize("w", MANY_ITEMS, ids=[w.name for w in MANY_ITEMS])
def test_parity_many_items_per_workgroup_sampled(w):
    total = w.batch * (w.heads_q // 2 if (w.heads_q // w.heads_kv) % 2 == 0 else w.heads_q) * -(-w.n // w.block)
    assert total % 8 != 0 and total > 512  # the walk without XCD ranges, several items per work-group
    rows = sample_rows(w.n, w.block, np.random.default_rng(21), extra=12)
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


@pytest.mark.parametrize("block", [128, 64])
def test_future_leakage_is_zero(block):
    w = synth.WORKLOADS["qwen3_32k"].resized(n=3000, block=block)
    q, k, v = synth.make_qkv(w)
    (o1, _), _ = run_gpu(w, q, k, v)
    for t in (0, 700, 1919, 2000):
        k2, v2 = k.clone(), v.clone()
        k2[:, :, t + 1:] = torch.randn_like(k2[:, :, t + 1:].float()).to(k2.dtype) * 3
        v2[:, :, t + 1:] = torch.randn_like(v2[:, :, t + 1:].float()).to(v2.dtype) * 3
        (o2, _), _ = run_gpu(w, q, k2, v2)
        assert torch.equal(o1[:, :, :t + 1], o2[:, :, :t + 1]), t
        assert not torch.equal(o1[:, :, t + 1:], o2[:, :, t + 1:])


@pytest.mark.parametrize("d,block", [(64, 128), (128, 128), (64, 64), (128, 64)])
def test_gqa_equals_repeated_kv(d, block):
    # query head h reads key/value head h // G.  At d = 64 and 128-token blocks the GQA and the
    # repeated-KV launches run the same per-head arithmetic (bitwise equal); otherwise they run
    # on different kernels (the repeated-KV launch is multi-head) and agree to rounding.
    w = synth.WORKLOADS["qwen3_32k"].resized(n=1500, d=d, block=block)
    q, k, v = synth.make_qkv(w)
    (o1, _), _ = run_gpu(w, q, k, v)
    G = w.heads_q // w.heads_kv
    wr = w.resized(heads_kv=w.heads_q)
    (o2, _), _ = run_gpu(wr, q, k.repeat_interleave(G, 1), v.repeat_interleave(G, 1))
    if d == 64 and block == 128:
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


def test_dense_causal_ref_against_the_oracle_full_size_sampled():
    # bsa_dense_causal_ref (route built inside the call) against the oracle's dense causal
    # attention on sampled rows of the 32K GQA workload
    w = synth.WORKLOADS["qwen3_32k"]
    q, k, v = synth.make_qkv(w)
    ws = torch.empty(bsa.bsa_dense_route_workspace_bytes(w.n, w.block) // 4, dtype=torch.int32, device="cuda")
    o = torch.empty(q.shape, dtype=q.dtype, device="cuda")
    lse = torch.empty(q.shape[:3], dtype=torch.float32, device="cuda")
    bsa.bsa_dense_causal_ref(q.cuda(), k.cuda(), v.cuda(), o, ws, w.block, lse=lse)
    torch.cuda.synchronize()
    rows = sample_rows(w.n, w.block, np.random.default_rng(11), extra=8)
    orp, oci = R.route_csr(R.DENSE_CAUSAL, w.n, w.block)
    ref, ref_lse = A.attention(q, k, v, w.block, orp, oci, rows=rows, return_lse=True)
    mx, rl2 = errors(o.float().cpu().numpy()[:, :, rows], ref)
    lse_err = float(np.abs(lse.cpu().numpy()[:, :, rows] - ref_lse).max())
    print(f"dense_causal_ref 32K: max-abs {mx:.3e} rel-L2 {rl2:.3e} lse {lse_err:.3e}", flush=True)
    assert mx <= BF16_MAXABS and rl2 <= BF16_RELL2 and lse_err <= 2.5e-3


# ---- canary-padded outputs: no store outside O and LSE, and every element of both written ------

CANARY_CASES = [
    # (name, batch, heads_q, heads_kv, n, d, block, dtype)
    ("gqa2-d128-b128-n129", 1, 2, 1, 129, 128, 128, "bf16"),
    ("gqa2-d64-b128-n1000", 2, 4, 2, 1000, 64, 128, "bf16"),
    ("mha-d64-b64-n1", 1, 2, 2, 1, 64, 64, "bf16"),
    ("mha-d128-b64-n777", 1, 2, 2, 777, 128, 64, "bf16"),
    ("gqa4-d64-b64-n65", 1, 4, 1, 65, 64, 64, "bf16"),
    ("mha-d64-b128-n300", 2, 2, 2, 300, 64, 128, "bf16"),
    ("mha-d128-b128-n300-fp32", 1, 2, 2, 300, 128, 128, "fp32"),
    ("gqa2-d128-b64-n777", 1, 4, 2, 777, 128, 64, "bf16"),
    ("gqa2-d64-b64-n100-fp32", 1, 2, 1, 100, 64, 64, "fp32"),
]


@pytest.mark.parametrize("case", CANARY_CASES, ids=[c[0] for c in CANARY_CASES])
@pytest.mark.parametrize("dense_ref", [False, True])
def test_canary_padded_outputs(case, dense_ref):
    from canary import padded
    name, batch, hq, hkv, n, d, B, dtype = case
    w = synth.WORKLOADS["qwen3_32k"].resized(name=name, batch=batch, heads_q=hq, heads_kv=hkv, n=n, d=d,
                                             block=B, dtype=dtype)
    print(f"canary {name} dense_ref={dense_ref}", flush=True)
    q, k, v = synth.make_qkv(w)
    kind = R.DENSE_CAUSAL if dense_ref else w.route_kind
    (rp, ci), (orp, oci) = workload_routes(w, kind)
    o = padded(q.shape, q.dtype)
    lse = padded(q.shape[:3], torch.float32)
    qd, kd, vd = q.cuda(), k.cuda(), v.cuda()
    if dense_ref:
        ws = torch.empty(bsa.bsa_dense_route_workspace_bytes(n, B) // 4, dtype=torch.int32, device="cuda")
        bsa.bsa_dense_causal_ref(qd, kd, vd, o.t, ws, B, lse=lse.t)
    else:
        bsa.bsa_forward(qd, kd, vd, o.t, rp, ci, B, lse=lse.t)
    torch.cuda.synchronize()
    assert o.guards_intact() and lse.guards_intact()
    assert not o.untouched().any() and not lse.untouched().any()
    ref, ref_lse = A.attention(q, k, v, B, orp, oci, return_lse=True)
    mx, rl2 = errors(o.t.float().cpu().numpy(), ref)
    ma, rt = tol(w.torch_dtype)
    assert mx <= ma and rl2 <= rt
    assert float(np.abs(lse.t.cpu().numpy() - ref_lse).max()) <= (1e-5 if dtype == "fp32" else 2.5e-3)


# ---- NaN inputs reach only the rows that read them -------------------------------------------
# A NaN in q row r makes output row r NaN.  A NaN in element c of key j makes NaN every row whose
# selected keys include j (its score is NaN); a NaN in element c of value j makes element c NaN in
# those rows.  Rows of a query block whose route lists j's key block but that do not select j
# (within the diagonal block, the rows before j) may take the NaN as well: their zero weight
# multiplies value j in the same matrix product.  Every other output element, and the LSE of
# every row in the value case, is bit-identical to the run without the NaN.

NAN_CASES = [
    ("gqa2-d128-b128", 1, 4, 2, 700, 128, 128, "bf16"),
    ("mha-d128-b64", 1, 2, 2, 650, 128, 64, "bf16"),
    ("gqa2-d128-b64", 1, 4, 2, 650, 128, 64, "bf16"),
    ("gqa2-d64-b128-fp32", 1, 2, 1, 400, 64, 128, "fp32"),
]


@pytest.mark.parametrize("case", NAN_CASES, ids=[c[0] for c in NAN_CASES])
@pytest.mark.parametrize("which", ["q", "k", "v"])
def test_nan_reaches_only_the_rows_that_read_it(case, which):
    name, batch, hq, hkv, n, d, B, dtype = case
    w = synth.WORKLOADS["qwen3_32k"].resized(name=name, batch=batch, heads_q=hq, heads_kv=hkv, n=n, d=d,
                                             block=B, dtype=dtype)
    print(f"nan {name} in {which}", flush=True)
    q, k, v = synth.make_qkv(w)
    (rp, ci), (orp, oci) = workload_routes(w)
    sets = R.csr_to_sets(orp, oci)
    qd, kd, vd = q.cuda(), k.cuda(), v.cuda()
    o0, lse0 = bsa.forward(qd, kd, vd, rp, ci, B, with_lse=True)
    G = hq // hkv
    head, row, col = {"q": (1, n // 2, 5), "k": (hkv - 1, n // 3, 7), "v": (hkv - 1, (2 * n) // 3, 7)}[which]
    t = {"q": qd, "k": kd, "v": vd}[which].clone()
    t[0, head, row, col] = float("nan")
    args = {"q": (t, kd, vd), "k": (qd, t, vd), "v": (qd, kd, t)}[which]
    o1, lse1 = bsa.forward(*args, rp, ci, B, with_lse=True)
    torch.cuda.synchronize()
    a0, a1 = o0.float().cpu().numpy(), o1.float().cpu().numpy()
    l0, l1 = lse0.cpu().numpy(), lse1.cpu().numpy()
    must = np.zeros((batch, hq, n), dtype=bool)  # rows that select the NaN element
    may = np.zeros((batch, hq, n), dtype=bool)   # ... or share a matrix product with it
    if which == "q":
        must[0, head, row] = may[0, head, row] = True
    else:
        jb = row // B
        for h in range(head * G, head * G + G):
            for r in range(n):
                if jb in sets[r // B]:
                    may[0, h, r] = True
                    must[0, h, r] = r >= row

    def same(x, y):  # bit-identical
        return np.array_equal(np.ascontiguousarray(x, np.float32).view(np.uint32),
                              np.ascontiguousarray(y, np.float32).view(np.uint32))
    if which == "v":
        # element `col` of the rows that select value j is NaN; the other elements and the LSE are untouched
        assert np.isnan(a1[must][:, col]).all()
        other = np.ones(d, dtype=bool)
        other[col] = False
        assert same(a0[..., other], a1[..., other])
        assert same(a0[~may][:, col], a1[~may][:, col])
        mid0, mid1 = a0[may & ~must][:, col], a1[may & ~must][:, col]
        assert (np.isnan(mid1) | (mid1.view(np.uint32) == mid0.view(np.uint32))).all()
        assert same(l0, l1)
    else:
        assert np.isnan(a1[must]).all() and np.isnan(l1[must]).all()
        assert same(a0[~may], a1[~may]) and same(l0[~may], l1[~may])
        for r_ok in zip(*np.nonzero(may & ~must)):  # the rows before j in its diagonal block
            x0, x1 = a0[r_ok], a1[r_ok]
            assert np.isnan(x1).all() or same(x0, x1)


# ---- malformed routes: results undefined, every access in bounds -----------------------------

def malformed_route(nqb, nnz, seed):
    """A route that breaks every rule bsa_check_route enforces: row pointers that decrease, jump
    past nnz and repeat (empty rows), and entries that are negative, in the future or repeated."""
    rng = np.random.default_rng(seed)
    rp = np.sort(rng.integers(0, nnz + 1, size=nqb + 1))
    rp[0] = 0
    rp[1::3] = rp[1::3][::-1]           # non-monotone
    rp[-1] = nnz + 7                    # past the end
    rp[nqb // 2] = rp[nqb // 2 - 1]     # an empty row
    ci = rng.integers(-3, nqb + 3, size=nnz)
    return (torch.tensor(rp.astype(np.int32), device="cuda"), torch.tensor(ci.astype(np.int32), device="cuda"))


MALFORMED_CASES = [
    # (name, heads_q, heads_kv, n, d, block, dtype): each forward kernel family
    ("gqa2-d128-b128", 4, 2, 700, 128, 128, "bf16"),   # pipelined, 128-key chunks
    ("gqa2-d128-b64", 4, 2, 700, 128, 64, "bf16"),     # pipelined, one 64-key chunk per block
    ("mha-d128-b128", 2, 2, 700, 128, 128, "bf16"),    # pipelined, two 64-key chunks per block
    ("mha-d64-b128", 2, 2, 700, 64, 128, "bf16"),      # pipelined, multi-head d = 64
    ("mha-d128-b64", 2, 2, 700, 128, 64, "bf16"),      # unpipelined
    ("mha-d64-b128-fp32", 2, 2, 700, 64, 128, "fp32"), # fp32
]


@pytest.mark.parametrize("case", MALFORMED_CASES, ids=[c[0] for c in MALFORMED_CASES])
def test_malformed_route_stays_in_bounds(case):
    """Without BSA_VALIDATE_ROUTE a malformed route gives undefined output, but no store leaves the
    caller's O and LSE buffers, and the same buffers then serve a valid route correctly."""
    from canary import padded
    name, hq, hkv, n, d, B, dtype = case
    w = synth.WORKLOADS["qwen3_32k"].resized(name=name, heads_q=hq, heads_kv=hkv, n=n, d=d, block=B, dtype=dtype)
    q, k, v = (x.cuda() for x in synth.make_qkv(w))
    nqb = w.nqb
    for seed in (1, 2):
        rp, ci = malformed_route(nqb, 3 * nqb, seed)  # nnz > 1.5 nqb: the multi-head rows count as long
        print(f"malformed {name} seed={seed}: row_ptr={rp.tolist()}", flush=True)
        o = padded(q.shape, q.dtype)
        lse = padded(q.shape[:3], torch.float32)
        bsa.bsa_forward(q, k, v, o.t, rp, ci, B, lse=lse.t)
        torch.cuda.synchronize()
        assert o.guards_intact() and lse.guards_intact()
    # a valid route afterwards, through the same entry point
    (rp, ci), (orp, oci) = workload_routes(w)
    o = bsa.forward(q, k, v, rp, ci, B)
    torch.cuda.synchronize()
    ref = A.attention(*(x.cpu() for x in (q, k, v)), B, orp, oci)
    mx, rl2 = errors(o.float().cpu().numpy(), ref)
    ma, rt = tol(w.torch_dtype)
    assert mx <= ma and rl2 <= rt
