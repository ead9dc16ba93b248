"""GPU backward (bsa_backward and bsa_build_route_transpose through the C ABI) against the fp64
oracle.

Transposed routes must be identical arrays.  Gradient bars (bf16 inputs and outputs): relative L2
<= 1e-2 and max-abs <= 1e-2 * max|reference| per tensor.  Derivation: the kernels round three
quantities to bf16 on the way (the weights P or the scores' gradient dS before each product, and
the output), each with relative error <= 2^-9 ~ 1.95e-3, so a gradient formed as a sum of many such
terms keeps a relative L2 error below about 3 x 1.95e-3 ~ 5.9e-3; 1e-2 leaves margin for the
cancellation in dP - D.
"""

import numpy as np
import pytest
import torch

import long_context_block_amd as bsa
from oracle import attn as A
from oracle import routes as R
import synth
from route_ref import routes, workload_routes

pytestmark = pytest.mark.gpu

KINDS = [R.BF1, R.BLOCK_DIAGONAL, R.DENSE_CAUSAL, R.STATIC_RANDOM, R.SLIDING_WINDOW]
RELL2, MAXREL = 1e-2, 1e-2


def transpose_sets(rp, ci):
    sets = R.csr_to_sets(rp, ci)
    out = [[] for _ in sets]
    for i, r in enumerate(sets):
        for j in r:
            out[j].append(i)
    return out


@pytest.mark.parametrize("kind", KINDS)
@pytest.mark.parametrize("n,B", [(1, 64), (1000, 64), (4097, 128), (32768, 128)])
def test_route_transpose_bit_exact(kind, n, B):
    (rp, ci), (orp, oci) = routes(kind, n, B)
    trp, tci = bsa.build_route_transpose(rp, ci)
    torch.cuda.synchronize()
    want_rp, want_ci = R.to_csr(transpose_sets(orp, oci))
    assert np.array_equal(trp.cpu().numpy(), want_rp) and np.array_equal(tci.cpu().numpy(), want_ci)


CANARY = -123456789


@pytest.mark.parametrize("row_ptr,col_idx", [
    ([0, 2, 0, 2], [0, 2]),            # overlapping rows: 4 memberships counted for 2 entries
    ([0, 3, 1, 3], [0, 1, 2]),         # a row that starts inside the previous one
    ([0, 1, 9, 9], [0, 1, 1, 2]),      # a row pointer past nnz (clamped on read)
])
def test_route_transpose_malformed_stays_in_bounds(row_ptr, col_idx):
    """The transpose of a malformed route is meaningless, but every write stays inside the caller's
    buffers: canaries right after t_col_idx[nnz - 1] survive and every t_row_ptr value is <= nnz."""
    nqb, nnz = len(row_ptr) - 1, len(col_idx)
    print(f"malformed transpose: row_ptr={row_ptr} col_idx={col_idx}", flush=True)
    rp = torch.tensor(row_ptr, dtype=torch.int32, device="cuda")
    ci = torch.tensor(col_idx, dtype=torch.int32, device="cuda")
    trp_buf = torch.full((nqb + 1 + 64,), CANARY, dtype=torch.int32, device="cuda")
    tci_buf = torch.full((nnz + 64,), CANARY, dtype=torch.int32, device="cuda")
    bsa.bsa_build_route_transpose(rp, ci, trp_buf[:nqb + 1], tci_buf[:nnz])
    torch.cuda.synchronize()
    trp = trp_buf.cpu().numpy()
    tci = tci_buf.cpu().numpy()
    assert (trp[nqb + 1:] == CANARY).all() and (tci[nnz:] == CANARY).all()
    assert trp[0] == 0 and (np.diff(trp[:nqb + 1]) >= 0).all() and trp[nqb] <= nnz


def grad_errors(got, ref):
    got = got.double().cpu().numpy() if hasattr(got, "cpu") else got
    d = got - ref
    return float(np.linalg.norm(d) / max(np.linalg.norm(ref), 1e-300)), float(np.abs(d).max() / max(np.abs(ref).max(), 1e-300))


def run_backward(w, kind=None, seed=61, q_rows=None, k_rows=None):
    kind = w.route_kind if kind is None else kind
    q, k, v = synth.make_qkv(w)
    g = torch.Generator("cpu").manual_seed(seed)
    d_o = torch.randn(q.shape, generator=g).to(q.dtype)
    (rp, ci), (orp, oci) = workload_routes(w, kind)
    qd, kd, vd, dod = q.cuda(), k.cuda(), v.cuda(), d_o.cuda()
    o, lse = bsa.forward(qd, kd, vd, rp, ci, w.block, with_lse=True)
    dq, dk, dv = bsa.backward(qd, kd, vd, o, dod, lse, rp, ci, w.block)
    torch.cuda.synchronize()
    rq, rk, rv = A.attention_backward(q, k, v, d_o, w.block, orp, oci,
                                      q_rows=q_rows, k_rows=k_rows)
    if q_rows is not None:
        dq = dq[:, :, q_rows]
    if k_rows is not None:
        dk, dv = dk[:, :, k_rows], dv[:, :, k_rows]
    return (dq, rq), (dk, rk), (dv, rv)


REDUCED = [
    synth.WORKLOADS["qwen3_32k"].resized(name="gqa2-d128-b128", n=1000),
    synth.WORKLOADS["bf1_4k"].resized(name="mha-d128-b64", n=777, heads_q=2, heads_kv=2),
    synth.WORKLOADS["bsbr_chunk_8k"].resized(name="mha-d64-b128", n=700, batch=2, heads_q=2, heads_kv=2),
    synth.WORKLOADS["bf1_4k"].resized(name="gqa4-d64-b64", n=600, d=64, heads_q=4, heads_kv=1),
    synth.WORKLOADS["qwen3_32k"].resized(name="gqa2-ragged", n=1, heads_q=2, heads_kv=1),
    synth.WORKLOADS["qwen3_32k"].resized(name="gqa2-ragged-129", n=129, heads_q=2, heads_kv=1),
    # batch > 1 with GQA pairs and a ragged last block (the transposed rows and the segment table
    # are per key/value head of each batch entry)
    synth.WORKLOADS["qwen3_32k"].resized(name="gqa2-d128-b128-batch2-ragged", n=1100, batch=2, heads_q=4, heads_kv=2),
    synth.WORKLOADS["bf1_4k"].resized(name="gqa2-d128-b64-batch3-ragged", n=650, batch=3, heads_q=4, heads_kv=2),
]


@pytest.mark.parametrize("kind", KINDS)
@pytest.mark.parametrize("w", REDUCED, ids=[w.name for w in REDUCED])
def test_backward_parity(w, kind):
    print(f"backward {w.name} kind={kind}", flush=True)
    for name, (got, ref) in zip(("dq", "dk", "dv"), run_backward(w, kind)):
        rl2, mx = grad_errors(got, ref)
        print(f"  {name}: rel-L2 {rl2:.3e} max-abs/max {mx:.3e}", flush=True)
        assert rl2 <= RELL2 and mx <= MAXREL, (name, rl2, mx)


def test_backward_long_reader_list_is_split():
    # block 0 of a BF1 route is read by every query block: at 96 blocks its readers span several
    # segments of the dK/dV pass, which are summed in order afterwards
    w = synth.WORKLOADS["qwen3_32k"].resized(name="bf1-12k", n=12288)
    rows = np.array([0, 1, 63, 127, 128, 4000, 12287])
    for name, (got, ref) in zip(("dq", "dk", "dv"), run_backward(w, q_rows=rows, k_rows=rows)):
        rl2, mx = grad_errors(got, ref)
        print(f"  {name}: rel-L2 {rl2:.3e} max-abs/max {mx:.3e}", flush=True)
        assert rl2 <= RELL2 and mx <= MAXREL, (name, rl2, mx)


def test_backward_deterministic_and_no_future_gradient():
    w = synth.WORKLOADS["qwen3_32k"].resized(n=900)
    q, k, v = (x.cuda() for x in synth.make_qkv(w))
    d_o = torch.randn(q.shape, device="cuda").to(q.dtype)
    rp, ci = bsa.build_route(bsa.route_spec(w.route_kind), w.n, w.block)
    o, lse = bsa.forward(q, k, v, rp, ci, w.block, with_lse=True)
    g1 = bsa.backward(q, k, v, o, d_o, lse, rp, ci, w.block)
    g2 = bsa.backward(q, k, v, o, d_o, lse, rp, ci, w.block)
    torch.cuda.synchronize()
    for a, b in zip(g1, g2):
        assert torch.equal(a, b)
    # an upstream gradient on the last 100 rows only: keys before every one of those rows' route
    # blocks get none, and dq of the other rows is exactly zero
    d_o2 = torch.zeros_like(d_o)
    d_o2[:, :, 800:] = d_o[:, :, 800:]
    dq, dk, dv = bsa.backward(q, k, v, o, d_o2, lse, rp, ci, w.block)
    torch.cuda.synchronize()
    assert (dq[:, :, :800] == 0).all()
    # keys and values read by none of those rows get exactly zero gradient; the ones they read get
    # some (rows 800 .. 899 lie in query blocks 6 and 7, which read their routes' key blocks, and
    # within block 6 only the keys up to row 899)
    sets = R.csr_to_sets(rp.cpu().numpy(), ci.cpu().numpy())
    read = np.zeros(w.n, dtype=bool)
    for i in (800 // w.block, (w.n - 1) // w.block):
        for j in sets[i]:
            read[j * w.block:(j + 1) * w.block] = True
    read_t = torch.from_numpy(read).cuda()
    for g in (dk, dv):
        assert (g[:, :, ~read_t] == 0).all()
        assert (g[:, :, read_t].abs().amax(dim=-1) > 0).all()


def test_backward_errors():
    q = torch.zeros(1, 2, 128, 64, dtype=torch.float32, device="cuda")
    rp, ci = bsa.build_route(bsa.route_spec(R.BF1), 128, 64)
    trp, tci = bsa.build_route_transpose(rp, ci)
    lse = torch.zeros(1, 2, 128, device="cuda")
    ws = torch.empty(1 << 20, dtype=torch.uint8, device="cuda")
    with pytest.raises(bsa.BsaError) as e:
        bsa.bsa_backward(q, q, q, q, q, lse, q.clone(), q.clone(), q.clone(), rp, ci, trp, tci, 64, ws)
    assert e.value.status == bsa.BSA_ERR_UNSUPPORTED
    qb = q.to(torch.bfloat16)
    small = torch.empty(16, dtype=torch.uint8, device="cuda")
    with pytest.raises(bsa.BsaError) as e:
        bsa.bsa_backward(qb, qb, qb, qb, qb, lse, qb.clone(), qb.clone(), qb.clone(), rp, ci, trp, tci, 64, small)
    assert e.value.status == bsa.BSA_ERR_CAPACITY


@pytest.mark.parametrize("wname,n", [("qwen3_32k", 1000), ("bf1_4k", 777)])
def test_backward_transposed_rows_in_any_order(wname, n):
    # The dK/dV pass masks only a leading run of diagonal-block work when the transposed rows are
    # sorted (as bsa_build_route_transpose writes them); given the same readers in reverse order it
    # must fall back to masking every step of the affected segments and still match the oracle.
    w = synth.WORKLOADS[wname].resized(n=n, heads_q=2, heads_kv=2 if wname == "bf1_4k" else 1)
    q, k, v = synth.make_qkv(w)
    g = torch.Generator("cpu").manual_seed(62)
    d_o = torch.randn(q.shape, generator=g).to(q.dtype)
    (rp, ci), (orp, oci) = workload_routes(w)
    trp, tci = bsa.build_route_transpose(rp, ci)
    trp_h, tci_h = trp.cpu().numpy(), tci.cpu().numpy().copy()
    for j in range(len(trp_h) - 1):
        tci_h[trp_h[j]:trp_h[j + 1]] = tci_h[trp_h[j]:trp_h[j + 1]][::-1].copy()
    tci_rev = torch.from_numpy(tci_h).cuda()
    qd, kd, vd, dod = q.cuda(), k.cuda(), v.cuda(), d_o.cuda()
    o, lse = bsa.forward(qd, kd, vd, rp, ci, w.block, with_lse=True)
    grads = []
    for t_ci in (tci, tci_rev):
        dq, dk, dv = torch.empty_like(qd), torch.empty_like(kd), torch.empty_like(vd)
        ws = torch.empty(bsa.bsa_backward_workspace_bytes(w.batch, w.heads_q, w.heads_kv, w.n, w.d, w.block, ci.numel()),
                         dtype=torch.uint8, device="cuda")
        bsa.bsa_backward(qd, kd, vd, o, dod, lse, dq, dk, dv, rp, ci, trp, t_ci, w.block, ws)
        grads.append((dq, dk, dv))
    torch.cuda.synchronize()
    ref = A.attention_backward(q, k, v, d_o, w.block, orp, oci)
    for name, got, r in zip(("dq", "dk", "dv"), grads[1], ref):
        rl2, mx = grad_errors(got, r)
        print(f"  reversed rows {name}: rel-L2 {rl2:.3e} max-abs/max {mx:.3e}", flush=True)
        assert rl2 <= RELL2 and mx <= MAXREL, (name, rl2, mx)
    assert torch.equal(grads[0][0], grads[1][0])  # dQ walks the forward route: unaffected


def test_canary_padded_gradients_and_workspace():
    """No store outside dq, dk, dv or the workspace, and every gradient element written, at partial
    final blocks for both kernels' block widths."""
    from canary import padded, padded_workspace
    for w in (synth.WORKLOADS["qwen3_32k"].resized(name="gqa2-d128-b128-n1000", n=1000, heads_q=4, heads_kv=2),
              synth.WORKLOADS["bf1_4k"].resized(name="mha-d128-b64-n129", n=129, heads_q=2, heads_kv=2),
              synth.WORKLOADS["bf1_4k"].resized(name="gqa4-d64-b64-n70", n=70, d=64, heads_q=4, heads_kv=1)):
        print(f"canary backward {w.name}", flush=True)
        q, k, v = (x.cuda() for x in synth.make_qkv(w))
        d_o = torch.randn(q.shape, device="cuda").to(q.dtype)
        (rp, ci), _ = workload_routes(w)
        o, lse = bsa.forward(q, k, v, rp, ci, w.block, with_lse=True)
        trp, tci = bsa.build_route_transpose(rp, ci)
        b, hq, n, d = q.shape
        dq, dk, dv = padded(q.shape, q.dtype), padded(k.shape, k.dtype), padded(v.shape, v.dtype)
        ws = padded_workspace(bsa.bsa_backward_workspace_bytes(b, hq, k.shape[1], n, d, w.block, ci.numel()))
        bsa.bsa_backward(q, k, v, o, d_o, lse, dq.t, dk.t, dv.t, rp, ci, trp, tci, w.block, ws.t)
        torch.cuda.synchronize()
        for x in (dq, dk, dv, ws):
            assert x.guards_intact()
        for x in (dq, dk, dv):
            assert not x.untouched().any()
        ref = bsa.backward(q, k, v, o, d_o, lse, rp, ci, w.block)
        torch.cuda.synchronize()
        for x, r in zip((dq, dk, dv), ref):
            assert torch.equal(x.t, r)
