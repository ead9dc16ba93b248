"""GPU selected-page decode (bsa_decode through the C ABI) against the fp64 oracle.

Bars as for the prefill: bf16 — max-abs <= 1e-2 and relative L2 <= 5e-3; fp32 — both <= 1e-5.
Also checked on the GPU: decode-reference agreement (the decoded token equals row t of the
prefill kernel's output), length clamping, determinism and the error paths.
"""

import numpy as np
import pytest
import torch

import long_context_block_amd as bsa
from oracle import attn as A
from oracle import routes as R
import synth
from route_ref import routes

pytestmark = pytest.mark.gpu

KINDS = [R.BF1, R.BLOCK_DIAGONAL, R.DENSE_CAUSAL, R.STATIC_RANDOM, R.SLIDING_WINDOW]


def tol(dtype):
    return (1e-5, 1e-5) if dtype == torch.float32 else (1e-2, 5e-3)


def errors(got, ref):
    d = np.asarray(got, dtype=np.float64) - ref
    return float(np.abs(d).max()), float(np.linalg.norm(d) / np.linalg.norm(ref))


def make(batch, hq, hkv, n_max, d, dtype, seed):
    g = torch.Generator("cpu").manual_seed(seed)
    q = torch.randn(batch, hq, d, generator=g).to(dtype)
    k = torch.randn(batch, hkv, n_max, d, generator=g).to(dtype)
    v = torch.randn(batch, hkv, n_max, d, generator=g).to(dtype)
    return q, k, v


def run(q, k, v, lens, kind, B, n_local=2, n_random=14, with_lse=True):
    n_max = k.shape[2]
    (rp, ci), oracle_rc = routes(kind, n_max, B, n_local, 1, n_random, 17)
    sl = torch.tensor(lens, dtype=torch.int32, device="cuda")
    o, lse = bsa.decode(q.cuda(), k.cuda(), v.cuda(), sl, rp, ci, B, with_lse=True)
    torch.cuda.synchronize()
    return o.float().cpu().numpy(), lse.cpu().numpy(), oracle_rc


CASES = [
    # (name, batch, hq, hkv, n_max, d, B, dtype)
    ("gqa2-d128-b128-bf16", 3, 16, 8, 4096, 128, 128, torch.bfloat16),
    ("mha-d64-b64-fp32", 2, 2, 2, 700, 64, 64, torch.float32),
    ("gqa4-d64-b128-bf16", 2, 8, 2, 1500, 64, 128, torch.bfloat16),
    ("gqa3-d128-b64-bf16", 2, 6, 2, 999, 128, 64, torch.bfloat16),
    ("gqa8-d128-b64-fp32", 1, 8, 1, 513, 128, 64, torch.float32),
    ("mha-d128-b128-fp32", 2, 3, 3, 300, 128, 128, torch.float32),
]


@pytest.mark.parametrize("kind", KINDS)
@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_decode_parity(case, kind):
    name, batch, hq, hkv, n_max, d, B, dt = case
    q, k, v = make(batch, hq, hkv, n_max, d, dt, seed=31)
    lens = [n_max, 1, B + 1, B, n_max // 2 + 3][:batch]
    print(f"decode {name} kind={kind} lens={lens}", flush=True)
    got, lse, (rp, ci) = run(q, k, v, lens, kind, B)
    ref, ref_lse = A.decode_attention(q, k, v, lens, B, rp, ci, return_lse=True)
    mx, rl2 = errors(got, ref)
    ma, rt = tol(dt)
    assert mx <= ma and rl2 <= rt, (mx, rl2)
    assert np.abs(lse - ref_lse).max() <= (1e-5 if dt == torch.float32 else 1e-4)


@pytest.mark.parametrize("name,kind", [("qwen3_32k", R.BF1), ("qwen3_32k", R.DENSE_CAUSAL),
                                       ("static_random_64k", R.STATIC_RANDOM)])
def test_decode_full_size(name, kind):
    # the workloads' shapes as key/value caches, newest tokens at the end and in the middle
    w = synth.WORKLOADS[name]
    q, k, v = make(1, w.heads_q, w.heads_kv, w.n, w.d, w.torch_dtype, seed=32)
    for t in (w.n - 1, w.n // 2 + 77):
        print(f"decode {name} kind={kind} t={t}", flush=True)
        got, lse, (rp, ci) = run(q, k, v, [t + 1], kind, w.block, w.n_local, w.n_random)
        ref, ref_lse = A.decode_attention(q, k, v, [t + 1], w.block, rp, ci, return_lse=True)
        mx, rl2 = errors(got, ref)
        assert mx <= 1e-2 and rl2 <= 5e-3, (mx, rl2)
        assert np.abs(lse - ref_lse).max() <= 1e-4


@pytest.mark.parametrize("kind", [R.BF1, R.STATIC_RANDOM])
def test_decode_agrees_with_prefill_kernel(kind):
    # decode-reference agreement on the GPU: the decoded token t reproduces row t of bsa_forward
    w = synth.WORKLOADS["qwen3_32k"].resized(n=3000, route_kind=kind)
    q, k, v = synth.make_qkv(w)
    rp, ci = bsa.build_route(bsa.route_spec(kind, w.n_local, w.keep_first, w.n_random, w.route_seed), w.n, w.block)
    qd, kd, vd = q.cuda(), k.cuda(), v.cuda()
    full = bsa.forward(qd, kd, vd, rp, ci, w.block).float()
    ts = [0, 127, 128, 1500, 2999]
    qt = torch.stack([q[0, :, t] for t in ts]).cuda()  # [len(ts), Hq, d]
    kk = kd.expand(len(ts), -1, -1, -1).contiguous()
    vv = vd.expand(len(ts), -1, -1, -1).contiguous()
    sl = torch.tensor([t + 1 for t in ts], dtype=torch.int32, device="cuda")
    o = bsa.decode(qt, kk, vv, sl, rp, ci, w.block).float()
    torch.cuda.synchronize()
    for x, t in enumerate(ts):
        mx, rl2 = errors(o[x].cpu().numpy(), full[0, :, t].double().cpu().numpy())
        # both round their output to bf16 once; the prefill also rounds its weights to bf16
        assert mx <= 1e-2 and rl2 <= 5e-3, (t, mx, rl2)


def test_decode_length_clamping_and_determinism():
    q, k, v = make(4, 4, 2, 300, 64, torch.bfloat16, seed=33)
    a, _, _ = run(q, k, v, [0, -5, 300, 1000], R.BF1, 64)
    b, _, _ = run(q, k, v, [1, 1, 300, 300], R.BF1, 64)
    c, _, _ = run(q, k, v, [1, 1, 300, 300], R.BF1, 64)
    assert np.array_equal(a, b) and np.array_equal(b, c)
    # a one-token cache returns v[0]
    G = 2
    assert np.array_equal(a[0], v[0, np.arange(4) // G, 0].float().numpy())


def test_decode_errors():
    q = torch.zeros(1, 2, 64, dtype=torch.bfloat16, device="cuda")
    k = torch.zeros(1, 2, 128, 64, dtype=torch.bfloat16, device="cuda")
    rp, ci = bsa.build_route(bsa.route_spec(R.BF1), 128, 64)
    sl = torch.ones(1, dtype=torch.int32, device="cuda")
    small = torch.empty(8, dtype=torch.float32, device="cuda")
    with pytest.raises(bsa.BsaError) as e:
        bsa.bsa_decode(q, k, k, torch.empty_like(q), sl, rp, ci, 64, small)
    assert e.value.status == bsa.BSA_ERR_CAPACITY
    ws = torch.empty(bsa.bsa_decode_workspace_bytes(1, 2, 64) // 4, dtype=torch.float32, device="cuda")
    rp32, ci32 = bsa.build_route(bsa.route_spec(R.BF1), 128, 32)
    with pytest.raises(bsa.BsaError) as e:
        bsa.bsa_decode(q, k, k, torch.empty_like(q), sl, rp32, ci32, 32, ws)
    assert e.value.status == bsa.BSA_ERR_UNSUPPORTED
    with pytest.raises(ValueError):  # a route built for a shorter cache is refused by the binding
        bsa.bsa_decode(q, k, k, torch.empty_like(q), sl, *bsa.build_route(bsa.route_spec(R.BF1), 64, 64), 64, ws)


ROUTED_KINDS = [R.BF1, R.BLOCK_DIAGONAL, R.DENSE_CAUSAL, R.SLIDING_WINDOW]


def run_routed(q, k, v, lens, kind, B, n_local=2, keep_first=1):
    sl = torch.tensor(lens, dtype=torch.int32, device="cuda")
    spec = bsa.route_spec(kind, n_local, keep_first)
    o, lse = bsa.decode_routed(q.cuda(), k.cuda(), v.cuda(), sl, spec, B, with_lse=True)
    torch.cuda.synchronize()
    return o, lse


@pytest.mark.parametrize("kind", ROUTED_KINDS)
@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_decode_routed_parity(case, kind):
    # rows generated in the kernel from the route's closed form, against the oracle's route
    name, batch, hq, hkv, n_max, d, B, dt = case
    q, k, v = make(batch, hq, hkv, n_max, d, dt, seed=34)
    lens = [n_max, 1, B + 1, B, n_max // 2 + 3][:batch]
    print(f"decode_routed {name} kind={kind} lens={lens}", flush=True)
    o, lse = run_routed(q, k, v, lens, kind, B)
    rp, ci = R.route_csr(kind, n_max, B, n_local=2, keep_first=True)
    ref, ref_lse = A.decode_attention(q, k, v, lens, B, rp, ci, return_lse=True)
    mx, rl2 = errors(o.float().cpu().numpy(), ref)
    ma, rt = tol(dt)
    assert mx <= ma and rl2 <= rt, (mx, rl2)
    assert np.abs(lse.cpu().numpy() - ref_lse).max() <= (1e-5 if dt == torch.float32 else 1e-4)


@pytest.mark.parametrize("kind,n_local,keep_first", [(R.BF1, 2, 1), (R.BF1, 0, 0), (R.BF1, 5, 1),
                                                     (R.BLOCK_DIAGONAL, 2, 1), (R.DENSE_CAUSAL, 2, 1),
                                                     (R.SLIDING_WINDOW, 3, 1), (R.SLIDING_WINDOW, 0, 0)])
def test_decode_routed_bit_equal_to_the_csr_route(kind, n_local, keep_first):
    # 512 (sequence, kv head) units: both entry points use 2 key splits, so their sums run in the
    # same order and the outputs agree bit for bit (lengths from 1 to the full cache)
    batch, hq, hkv, n_max, d, B = 64, 8, 8, 700, 64, 64
    q, k, v = make(batch, hq, hkv, n_max, d, torch.bfloat16, seed=35)
    lens = [1 + (37 * x * x + 11 * x) % n_max for x in range(batch)]
    lens[:4] = [1, B, B + 1, n_max]
    print(f"decode_routed vs csr kind={kind} n_local={n_local} keep_first={keep_first}", flush=True)
    o1, l1 = run_routed(q, k, v, lens, kind, B, n_local, keep_first)
    (rp, ci), _ = routes(kind, n_max, B, n_local, keep_first)
    sl = torch.tensor(lens, dtype=torch.int32, device="cuda")
    o2, l2 = bsa.decode(q.cuda(), k.cuda(), v.cuda(), sl, rp, ci, B, with_lse=True)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


@pytest.mark.parametrize("kind", [R.BF1, R.SLIDING_WINDOW])
def test_decode_routed_full_size(kind):
    w = synth.WORKLOADS["qwen3_32k"]
    q, k, v = make(1, w.heads_q, w.heads_kv, w.n, w.d, w.torch_dtype, seed=36)
    rp, ci = R.route_csr(kind, w.n, w.block, n_local=w.n_local, keep_first=True)
    for t in (w.n - 1, w.n // 2 + 77, 2 ** 14 - 1):
        print(f"decode_routed qwen3_32k kind={kind} t={t}", flush=True)
        o, lse = run_routed(q, k, v, [t + 1], kind, w.block, w.n_local)
        ref, ref_lse = A.decode_attention(q, k, v, [t + 1], w.block, rp, ci, return_lse=True)
        mx, rl2 = errors(o.float().cpu().numpy(), ref)
        assert mx <= 1e-2 and rl2 <= 5e-3, (mx, rl2)
        assert np.abs(lse.cpu().numpy() - ref_lse).max() <= 1e-4


def test_decode_routed_errors():
    q = torch.zeros(1, 2, 64, dtype=torch.bfloat16, device="cuda")
    k = torch.zeros(1, 2, 128, 64, dtype=torch.bfloat16, device="cuda")
    sl = torch.ones(1, dtype=torch.int32, device="cuda")
    ws = torch.empty(bsa.bsa_decode_workspace_bytes(1, 2, 64) // 4, dtype=torch.float32, device="cuda")
    for spec, status in ((bsa.route_spec(R.STATIC_RANDOM), bsa.BSA_ERR_UNSUPPORTED),
                         (bsa.route_spec(7), bsa.BSA_ERR_INVALID_ARGUMENT),
                         (bsa.route_spec(R.BF1, n_local=-1), bsa.BSA_ERR_INVALID_ARGUMENT)):
        with pytest.raises(bsa.BsaError) as e:
            bsa.bsa_decode_routed(q, k, k, torch.empty_like(q), sl, spec, 64, ws)
        assert e.value.status == status
    with pytest.raises(bsa.BsaError) as e:
        bsa.bsa_decode_routed(q, k, k, torch.empty_like(q), sl, bsa.route_spec(R.BF1), 64, ws[:8])
    assert e.value.status == bsa.BSA_ERR_CAPACITY


@pytest.mark.parametrize("case", [CASES[0], CASES[1], CASES[3]], ids=[CASES[i][0] for i in (0, 1, 3)])
def test_decode_canary_padded(case):
    """No store outside o, lse or the workspace, and every output element written, with the plan
    from a CSR route and from the in-kernel rows."""
    from canary import padded, padded_workspace
    name, batch, hq, hkv, n_max, d, B, dt = case
    q, k, v = (x.cuda() for x in make(batch, hq, hkv, n_max, d, dt, seed=33))
    lens = torch.tensor([n_max, 1, B + 1][:batch], dtype=torch.int32, device="cuda")
    (rp, ci), _ = routes(R.BF1, n_max, B, 2, 1, 14, 17)
    for routed in (False, True):
        print(f"decode canary {name} routed={routed}", flush=True)
        o, lse = padded(q.shape, q.dtype), padded((batch, hq), torch.float32)
        ws = padded_workspace(bsa.bsa_decode_workspace_bytes(batch, hq, d), torch.float32)
        if routed:
            bsa.bsa_decode_routed(q, k, v, o.t, lens, bsa.route_spec(R.BF1), B, ws.t, lse=lse.t)
        else:
            bsa.bsa_decode(q, k, v, o.t, lens, rp, ci, B, ws.t, lse=lse.t)
        torch.cuda.synchronize()
        for x in (o, lse, ws):
            assert x.guards_intact()
        assert not o.untouched().any() and not lse.untouched().any()
        # the same entry point on plain buffers (the two entry points may split the keys differently)
        if routed:
            ref, ref_lse = bsa.decode_routed(q, k, v, lens, bsa.route_spec(R.BF1), B, with_lse=True)
        else:
            ref, ref_lse = bsa.decode(q, k, v, lens, rp, ci, B, with_lse=True)
        torch.cuda.synchronize()
        assert torch.equal(o.t, ref) and torch.equal(lse.t, ref_lse)
