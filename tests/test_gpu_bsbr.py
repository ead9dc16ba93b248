"""GPU BSBR attention (bsa_bsbr_forward through the C ABI) against the fp64 oracle.

Bar (relative, because the retrieval term is a sum of unnormalised chunk states and far from unit
scale): rel-L2 <= 5e-3 and max-abs <= 1e-2 * max|reference|.  The kernels form the chunk states
from exact bf16 products in fp32, mix and apply them in fp32, and round the output to bf16 after
the within-chunk term and again after adding the retrieval term (<= 2^-8 relative per element).
"""

import numpy as np
import pytest
import torch

import long_context_block_amd as bsa
from oracle import attn as A
from oracle import bsbr as OB
from oracle import routes as R
import synth

pytestmark = pytest.mark.gpu

RELL2, MAXREL = 5e-3, 1e-2


def errors(got, ref):
    d = np.asarray(got, dtype=np.float64) - ref
    return float(np.linalg.norm(d) / np.linalg.norm(ref)), float(np.abs(d).max() / np.abs(ref).max())


def run(w, rows=None):
    q, k, v = synth.make_qkv(w)
    r, h = synth.make_meta(w)
    o = bsa.bsbr_forward(q.cuda(), k.cuda(), v.cuda(), r.cuda(), h.cuda(), w.block)
    torch.cuda.synchronize()
    got = o.float().cpu().numpy()
    ref = OB.bsbr_forward(q, k, v, r, h, w.block, rows=rows)
    if rows is not None:
        got = got[:, :, rows]
    return got, ref, (q, k, v, r, h, o)


C3 = synth.WORKLOADS["bsbr_chunk_8k"]
CASES = [
    C3.resized(name="c3-d64-c128", n=700),
    C3.resized(name="gqa2-d128-c128", n=1000, d=128, heads_q=4, heads_kv=2, batch=1),
    C3.resized(name="d128-c64", n=333, d=128, block=64, heads_q=2, heads_kv=1, batch=1),
    C3.resized(name="d64-c64-exact", n=320, block=64, heads_q=1, heads_kv=1, batch=1),
    C3.resized(name="two-chunks-one-token", n=129, heads_q=2, heads_kv=2, batch=1),
    C3.resized(name="single-token", n=1, heads_q=2, heads_kv=1, batch=1),
]


@pytest.mark.parametrize("w", CASES, ids=[w.name for w in CASES])
def test_bsbr_parity(w):
    print(f"bsbr {w.name}", flush=True)
    got, ref, _ = run(w)
    rl2, mx = errors(got, ref)
    print(f"  rel-L2 {rl2:.3e} max-abs/max {mx:.3e}", flush=True)
    assert rl2 <= RELL2 and mx <= MAXREL, (rl2, mx)


def test_bsbr_first_chunk_is_within_chunk_attention_and_retrieval_term_alone():
    # chunk 0 retrieves nothing: its rows are the within-chunk attention alone, held to the
    # forward's bf16 bar; the rest minus the oracle's within-chunk term is the retrieval term
    w = C3.resized(n=1000, batch=1, heads_q=2, heads_kv=1)
    got, ref, (q, k, v, r, h, o) = run(w)
    rp, ci = R.route_csr(R.BLOCK_DIAGONAL, w.n, w.block)
    within = A.attention(q, k, v, w.block, rp, ci)
    d0 = got[:, :, :w.block] - within[:, :, :w.block]
    assert np.abs(d0).max() <= 1e-2 and np.linalg.norm(d0) / np.linalg.norm(within[:, :, :w.block]) <= 5e-3
    term = got - within
    ref_term = OB.retrieval(q, k, v, r, h, w.block)
    rl2, mx = errors(term[:, :, w.block:], ref_term[:, :, w.block:])
    print(f"  retrieval term: rel-L2 {rl2:.3e} max-abs/max {mx:.3e}", flush=True)
    assert rl2 <= RELL2 and mx <= MAXREL, (rl2, mx)


def test_bsbr_full_size_sampled_rows():
    # the bsbr_chunk_8k workload (2 x 8 heads, n 8192, d 64, chunks of 128), rows spread over the
    # chunks including the first and the last
    w = C3
    rows = np.array([0, 127, 128, 129, 1000, 4095, 4096, 6000, 8064, 8191])
    got, ref, _ = run(w, rows=rows)
    rl2, mx = errors(got, ref)
    print(f"  full size sampled rows: rel-L2 {rl2:.3e} max-abs/max {mx:.3e}", flush=True)
    assert rl2 <= RELL2 and mx <= MAXREL, (rl2, mx)


@pytest.mark.parametrize("w,rows", [
    # 1024 chunks of 64 (the largest count): the meta weights of a 32-chunk tile span 1024 chunks
    (C3.resized(name="c1024-d64-c64", n=65536, block=64, heads_q=1, heads_kv=1, batch=1),
     [0, 63, 64, 2047, 2048, 2049, 33000, 65471, 65472, 65535]),
    # 100 chunks, the last one partial and the last 32-chunk tile short; GQA at d = 128
    (C3.resized(name="c100-gqa2-d128-c64", n=6370, block=64, d=128, heads_q=4, heads_kv=2, batch=1),
     [0, 64, 2047, 2048, 4000, 6143, 6335, 6336, 6369]),
])
def test_bsbr_many_chunks_sampled_rows(w, rows):
    print(f"bsbr {w.name}", flush=True)
    got, ref, _ = run(w, rows=np.array(rows))
    rl2, mx = errors(got, ref)
    print(f"  rel-L2 {rl2:.3e} max-abs/max {mx:.3e}", flush=True)
    assert rl2 <= RELL2 and mx <= MAXREL, (rl2, mx)


def test_bsbr_deterministic():
    w = C3.resized(n=2000, batch=1)
    q, k, v = (x.cuda() for x in synth.make_qkv(w))
    r, h = (x.cuda() for x in synth.make_meta(w))
    a = bsa.bsbr_forward(q, k, v, r, h, w.block)
    b = bsa.bsbr_forward(q, k, v, r, h, w.block)
    torch.cuda.synchronize()
    assert torch.equal(a, b)


def test_bsbr_errors():
    q = torch.zeros(1, 2, 256, 64, dtype=torch.float32, device="cuda")
    r = torch.zeros(1, 2, 2, 64, dtype=torch.float32, device="cuda")
    ws = torch.empty(1 << 20, dtype=torch.uint8, device="cuda")
    with pytest.raises(bsa.BsaError) as e:
        bsa.bsa_bsbr_forward(q, q, q, r, r, q.clone(), 128, ws)
    assert e.value.status == bsa.BSA_ERR_UNSUPPORTED
    qb, rb = q.to(torch.bfloat16), r.to(torch.bfloat16)
    small = torch.empty(16, dtype=torch.uint8, device="cuda")
    with pytest.raises(bsa.BsaError) as e:
        bsa.bsa_bsbr_forward(qb, qb, qb, rb, rb, qb.clone(), 128, small)
    assert e.value.status == bsa.BSA_ERR_CAPACITY
    with pytest.raises(ValueError):  # meta tensors must have one row per chunk
        bsa.bsa_bsbr_forward(qb, qb, qb, rb[:, :, :1], rb, qb.clone(), 128, ws)


@pytest.mark.parametrize("w", [CASES[1], CASES[2], CASES[4]], ids=[CASES[i].name for i in (1, 2, 4)])
def test_bsbr_canary_padded(w):
    """No store outside o or the workspace, and every output element written, at partial final
    chunks."""
    from canary import padded, padded_workspace
    print(f"bsbr canary {w.name}", flush=True)
    q, k, v = (x.cuda() for x in synth.make_qkv(w))
    r, h = (x.cuda() for x in synth.make_meta(w))
    o = padded(q.shape, q.dtype)
    ws = padded_workspace(bsa.bsa_bsbr_workspace_bytes(w.batch, w.heads_q, w.heads_kv, w.n, w.d, w.block))
    bsa.bsa_bsbr_forward(q, k, v, r, h, o.t, w.block, ws.t)
    torch.cuda.synchronize()
    assert o.guards_intact() and ws.guards_intact()
    assert not o.untouched().any()
    ref = bsa.bsbr_forward(q, k, v, r, h, w.block)
    torch.cuda.synchronize()
    assert torch.equal(o.t, ref)
