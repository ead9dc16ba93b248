"""C-ABI tests that need no GPU: the library loads, exports every declared symbol, validates
arguments before any HIP call, and its host-side route logic (closed-form nnz, route checker)
agrees with the oracle."""

import ctypes
import os
import re

import numpy as np
import pytest

import long_context_block_amd as bsa
from oracle import routes as R

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "bsa.h")

pytestmark = pytest.mark.skipif(not os.path.exists(bsa.LIB_PATH), reason="libbsa.so not built")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(bsa_[a-z_]+)\s*\(", text)))


def test_header_declares_expected_calls():
    assert set(declared_functions()) == set(bsa.EXPORTS)


def test_library_exports_every_declared_symbol():
    L = bsa.lib()
    for name in declared_functions():
        assert hasattr(L, name), name


def test_status_strings():
    assert bsa.bsa_status_string(0) == "BSA_OK"
    assert bsa.bsa_status_string(4) == "BSA_ERR_CAPACITY"
    assert bsa.bsa_status_string(99) == "BSA_ERR_UNKNOWN"


def _raw_forward(**kw):
    args = dict(q=16, k=16, v=16, o=16, lse=None, batch=1, hq=2, hkv=1, n=256, d=64, block=64, dtype=0,
                scale=0.0, rp=16, ci=16, nnz=8, stream=None)
    args.update(kw)
    return bsa.lib().bsa_forward(args["q"], args["k"], args["v"], args["o"], args["lse"], args["batch"],
                                 args["hq"], args["hkv"], args["n"], args["d"], args["block"], args["dtype"],
                                 args["scale"], args["rp"], args["ci"], args["nnz"], args["stream"])


@pytest.mark.parametrize("kw,status", [
    (dict(hq=3, hkv=2), bsa.BSA_ERR_INVALID_ARGUMENT),
    (dict(batch=-1), bsa.BSA_ERR_INVALID_ARGUMENT),
    (dict(n=-5), bsa.BSA_ERR_INVALID_ARGUMENT),
    (dict(hkv=0), bsa.BSA_ERR_INVALID_ARGUMENT),
    (dict(d=96), bsa.BSA_ERR_UNSUPPORTED),
    (dict(block=32), bsa.BSA_ERR_UNSUPPORTED),
    (dict(dtype=7), bsa.BSA_ERR_UNSUPPORTED),
    (dict(q=None), bsa.BSA_ERR_INVALID_ARGUMENT),
    (dict(o=24), bsa.BSA_ERR_INVALID_ARGUMENT),      # misaligned
    (dict(lse=18), bsa.BSA_ERR_INVALID_ARGUMENT),    # misaligned lse
    (dict(rp=None), bsa.BSA_ERR_INVALID_ARGUMENT),
    (dict(nnz=3), bsa.BSA_ERR_INVALID_ARGUMENT),     # fewer entries than blocks
    (dict(scale=float("inf")), bsa.BSA_ERR_INVALID_ARGUMENT),
])
def test_forward_rejects_bad_arguments(kw, status):
    assert _raw_forward(**kw) == status
    assert bsa.bsa_last_error() != ""


def test_forward_empty_inputs_are_noops():
    # no device work, so this runs without a GPU
    assert _raw_forward(n=0, q=None, k=None, v=None, o=None, rp=None, ci=None, nnz=0) == bsa.BSA_OK
    assert _raw_forward(batch=0, q=None, k=None, v=None, o=None) == bsa.BSA_OK


def _raw_decode(**kw):
    args = dict(q=16, k=16, v=16, o=16, lse=None, sl=16, batch=2, hq=4, hkv=2, n_max=1000, d=128, block=128,
                dtype=0, scale=0.0, rp=16, ci=16, nnz=8, ws=16, wsb=None, stream=None)
    args.update(kw)
    if args["wsb"] is None:
        args["wsb"] = bsa.bsa_decode_workspace_bytes(args["batch"], args["hq"], args["d"])
    return bsa.lib().bsa_decode(args["q"], args["k"], args["v"], args["o"], args["lse"], args["sl"], args["batch"],
                                args["hq"], args["hkv"], args["n_max"], args["d"], args["block"], args["dtype"],
                                args["scale"], args["rp"], args["ci"], args["nnz"], args["ws"], args["wsb"],
                                args["stream"])


@pytest.mark.parametrize("kw,status", [
    (dict(hq=3, hkv=2), bsa.BSA_ERR_INVALID_ARGUMENT),
    (dict(n_max=0), bsa.BSA_ERR_INVALID_ARGUMENT),
    (dict(d=96), bsa.BSA_ERR_UNSUPPORTED),
    (dict(block=32), bsa.BSA_ERR_UNSUPPORTED),
    (dict(dtype=7), bsa.BSA_ERR_UNSUPPORTED),
    (dict(sl=None), bsa.BSA_ERR_INVALID_ARGUMENT),
    (dict(ws=None), bsa.BSA_ERR_INVALID_ARGUMENT),
    (dict(q=24), bsa.BSA_ERR_INVALID_ARGUMENT),      # misaligned
    (dict(nnz=7), bsa.BSA_ERR_INVALID_ARGUMENT),     # fewer entries than blocks (8)
    (dict(wsb=100), bsa.BSA_ERR_CAPACITY),
    (dict(scale=float("nan")), bsa.BSA_ERR_INVALID_ARGUMENT),
])
def test_decode_rejects_bad_arguments(kw, status):
    assert _raw_decode(**kw) == status
    assert bsa.bsa_last_error() != ""


def test_decode_workspace_and_empty_batch():
    assert bsa.bsa_decode_workspace_bytes(3, 16, 128) == 3 * 16 * 64 * 130 * 4
    assert bsa.bsa_decode_workspace_bytes(-1, 16, 128) == 0
    assert _raw_decode(batch=0, q=None, k=None, v=None, o=None, sl=None, ws=None) == bsa.BSA_OK


def _raw_decode_routed(spec=None, **kw):
    args = dict(q=16, k=16, v=16, o=16, lse=None, sl=16, batch=2, hq=4, hkv=2, n_max=1000, d=128, block=128,
                dtype=0, scale=0.0, ws=16, wsb=None, stream=None)
    args.update(kw)
    if args["wsb"] is None:
        args["wsb"] = bsa.bsa_decode_workspace_bytes(args["batch"], args["hq"], args["d"])
    sp = ctypes.byref(spec) if spec is not None else None
    return bsa.lib().bsa_decode_routed(args["q"], args["k"], args["v"], args["o"], args["lse"], args["sl"],
                                       args["batch"], args["hq"], args["hkv"], args["n_max"], args["d"],
                                       args["block"], args["dtype"], args["scale"], sp, args["ws"], args["wsb"],
                                       args["stream"])


@pytest.mark.parametrize("spec,kw,status", [
    (None, {}, bsa.BSA_ERR_INVALID_ARGUMENT),
    (bsa.route_spec(bsa.BSA_ROUTE_STATIC_RANDOM), {}, bsa.BSA_ERR_UNSUPPORTED),
    (bsa.route_spec(bsa.BSA_ROUTE_STATIC_RANDOM), dict(batch=0), bsa.BSA_ERR_UNSUPPORTED),
    (bsa.route_spec(9), {}, bsa.BSA_ERR_INVALID_ARGUMENT),
    (bsa.route_spec(-1), {}, bsa.BSA_ERR_INVALID_ARGUMENT),
    (bsa.route_spec(bsa.BSA_ROUTE_BF1, n_local=-2), {}, bsa.BSA_ERR_INVALID_ARGUMENT),
    (bsa.route_spec(bsa.BSA_ROUTE_BF1), dict(hq=3, hkv=2), bsa.BSA_ERR_INVALID_ARGUMENT),
    (bsa.route_spec(bsa.BSA_ROUTE_BF1), dict(d=96), bsa.BSA_ERR_UNSUPPORTED),
    (bsa.route_spec(bsa.BSA_ROUTE_BF1), dict(block=32), bsa.BSA_ERR_UNSUPPORTED),
    (bsa.route_spec(bsa.BSA_ROUTE_BF1), dict(sl=None), bsa.BSA_ERR_INVALID_ARGUMENT),
    (bsa.route_spec(bsa.BSA_ROUTE_BF1), dict(q=24), bsa.BSA_ERR_INVALID_ARGUMENT),
    (bsa.route_spec(bsa.BSA_ROUTE_DENSE_CAUSAL), dict(wsb=100), bsa.BSA_ERR_CAPACITY),
    (bsa.route_spec(bsa.BSA_ROUTE_SLIDING_WINDOW), dict(scale=float("inf")), bsa.BSA_ERR_INVALID_ARGUMENT),
])
def test_decode_routed_rejects_bad_arguments(spec, kw, status):
    assert _raw_decode_routed(spec, **kw) == status
    assert bsa.bsa_last_error() != ""


def test_decode_routed_empty_batch_and_no_route_pointers():
    # no CSR arrays at all: the closed-form kinds validate and an empty batch is a no-op
    for kind in (bsa.BSA_ROUTE_BF1, bsa.BSA_ROUTE_BLOCK_DIAGONAL, bsa.BSA_ROUTE_DENSE_CAUSAL,
                 bsa.BSA_ROUTE_SLIDING_WINDOW):
        assert _raw_decode_routed(bsa.route_spec(kind), batch=0, q=None, k=None, v=None, o=None, sl=None,
                                  ws=None) == bsa.BSA_OK


def test_decode_routed_noalloc_rejects_before_device_work():
    L = bsa.lib()
    spec = bsa.route_spec(bsa.BSA_ROUTE_BF1)
    # 512 x 64 (batch, query head) pairs of single-split partials at d = 128 need 17 MB, more
    # than the static scratch array holds: refused before any device call (this runs without a GPU)
    st = L.bsa_decode_routed_noalloc(16, 16, 16, 16, None, 16, 512, 64, 64, 65536, 128, 128, 0, 0.0,
                                     ctypes.byref(spec), None)
    assert st == bsa.BSA_ERR_CAPACITY and "static scratch" in bsa.bsa_last_error()
    assert L.bsa_decode_routed_noalloc(16, 16, 16, 16, None, 16, 2, 4, 2, 1000, 128, 128, 0, 0.0, None,
                                       None) == bsa.BSA_ERR_INVALID_ARGUMENT
    st = L.bsa_decode_routed_noalloc(None, None, None, None, None, None, 0, 4, 2, 1000, 128, 128, 0, 0.0,
                                     ctypes.byref(spec), None)
    assert st == bsa.BSA_OK  # empty batch: nothing to do


def test_dense_ref_rejects_small_workspace():
    L = bsa.lib()
    need = bsa.bsa_dense_route_workspace_bytes(4096, 64)
    assert need == (65 + 64 * 65 // 2) * 4
    st = L.bsa_dense_causal_ref(16, 16, 16, 16, None, 1, 1, 1, 4096, 64, 64, 0, 0.0, 16, need - 4, None)
    assert st == bsa.BSA_ERR_CAPACITY
    st = L.bsa_dense_causal_ref(16, 16, 16, 16, None, 1, 1, 1, 4096, 64, 64, 0, 0.0, None, need, None)
    assert st == bsa.BSA_ERR_INVALID_ARGUMENT


def _raw_bsbr(**kw):
    args = dict(q=16, k=16, v=16, r=16, h=16, o=16, batch=1, hq=2, hkv=1, n=1000, d=64, chunk=128, dtype=0,
                scale=0.0, ws=16, wsb=None, stream=None)
    args.update(kw)
    if args["wsb"] is None:
        args["wsb"] = bsa.bsa_bsbr_workspace_bytes(max(args["batch"], 0), args["hq"], max(args["hkv"], 1),
                                                   max(args["n"], 1), args["d"], max(args["chunk"], 1))
    return bsa.lib().bsa_bsbr_forward(args["q"], args["k"], args["v"], args["r"], args["h"], args["o"],
                                      args["batch"], args["hq"], args["hkv"], args["n"], args["d"], args["chunk"],
                                      args["dtype"], args["scale"], args["ws"], args["wsb"], args["stream"])


@pytest.mark.parametrize("kw,status", [
    (dict(hq=3, hkv=2), bsa.BSA_ERR_INVALID_ARGUMENT),
    (dict(batch=-1), bsa.BSA_ERR_INVALID_ARGUMENT),
    (dict(chunk=0), bsa.BSA_ERR_INVALID_ARGUMENT),
    (dict(dtype=1), bsa.BSA_ERR_UNSUPPORTED),
    (dict(d=96), bsa.BSA_ERR_UNSUPPORTED),
    (dict(chunk=32), bsa.BSA_ERR_UNSUPPORTED),
    (dict(n=128 * 1024 + 1), bsa.BSA_ERR_UNSUPPORTED),
    (dict(r=None), bsa.BSA_ERR_INVALID_ARGUMENT),
    (dict(h=24), bsa.BSA_ERR_INVALID_ARGUMENT),
    (dict(ws=None), bsa.BSA_ERR_INVALID_ARGUMENT),
    (dict(wsb=100), bsa.BSA_ERR_CAPACITY),
    (dict(scale=float("inf")), bsa.BSA_ERR_INVALID_ARGUMENT),
])
def test_bsbr_rejects_bad_arguments(kw, status):
    assert _raw_bsbr(**kw) == status
    assert bsa.bsa_last_error() != ""


def test_bsbr_workspace_and_empty_batch():
    # fp32 states per kv head and retrieved states per query head
    nch, d, hq, hkv = 8, 64, 3, 1
    align = lambda x: -(-x // 256) * 256  # noqa: E731
    want = align(hkv * nch * d * d * 4) + hq * nch * d * d * 4
    assert bsa.bsa_bsbr_workspace_bytes(1, 3, 1, 1000, 64, 128) == want
    assert bsa.bsa_bsbr_workspace_bytes(1, 3, 2, 1000, 64, 128) == 0
    assert _raw_bsbr(batch=0, q=None, k=None, v=None, r=None, h=None, o=None, ws=None) == bsa.BSA_OK


ROUTE_CASES = [
    (R.BF1, dict(n_local=2, keep_first=1)), (R.BF1, dict(n_local=1, keep_first=1)),
    (R.BF1, dict(n_local=0, keep_first=0)), (R.BF1, dict(n_local=5, keep_first=1)),
    (R.BF1, dict(n_local=3, keep_first=0)),
    (R.BLOCK_DIAGONAL, {}), (R.DENSE_CAUSAL, {}),
    (R.STATIC_RANDOM, dict(n_random=14, keep_first=1)), (R.STATIC_RANDOM, dict(n_random=3, keep_first=0)),
    (R.STATIC_RANDOM, dict(n_random=0, keep_first=1)),
    (R.SLIDING_WINDOW, dict(n_local=0)), (R.SLIDING_WINDOW, dict(n_local=8)),
    (R.SLIDING_WINDOW, dict(n_local=100)),
]


@pytest.mark.parametrize("kind,params", ROUTE_CASES)
@pytest.mark.parametrize("n,B", [(512, 64), (4096, 64), (8192, 128), (32768, 128), (1000, 64), (1, 64), (0, 64)])
def test_route_size_query_matches_oracle(kind, params, n, B):
    spec = bsa.route_spec(kind, params.get("n_local", 2), params.get("keep_first", 1),
                          params.get("n_random", 14), 17)
    nnz = bsa.bsa_build_route(spec, n, B)  # col_idx None: host-only size query
    oparams = dict(n_local=params.get("n_local", 2), keep_first=bool(params.get("keep_first", 1)),
                   n_random=params.get("n_random", 14), seed=17)
    nqb = R.num_blocks(n, B)
    if kind == R.STATIC_RANDOM and nqb > 600:
        want = sum(min(params.get("n_random", 14), (i - 1 if params.get("keep_first", 1) else i)) +
                   1 + (1 if params.get("keep_first", 1) else 0) if i > 0 else 1 for i in range(nqb))
    else:
        want = int(R.to_csr(R.route_sets(kind, nqb, **oparams))[0][-1])
    assert nnz == want


def test_route_spec_rejected():
    with pytest.raises(bsa.BsaError) as e:
        bsa.bsa_build_route(bsa.route_spec(9), 100, 64)
    assert e.value.status == bsa.BSA_ERR_INVALID_ARGUMENT
    with pytest.raises(bsa.BsaError):
        bsa.bsa_build_route(bsa.route_spec(0, n_local=-1), 100, 64)


@pytest.mark.parametrize("kind", [R.BF1, R.BLOCK_DIAGONAL, R.DENSE_CAUSAL, R.STATIC_RANDOM, R.SLIDING_WINDOW])
def test_check_route_accepts_oracle_routes(kind):
    rp, ci = R.route_csr(kind, 3000, 64)
    bsa.bsa_check_route(rp, ci)


@pytest.mark.parametrize("mutate,msg", [
    (lambda rp, ci: ci.__setitem__(3, 2), "outside"),          # row 2 reads block ... non-causal / order
    (lambda rp, ci: ci.__setitem__(0, 1), "outside"),          # row 0 reads block 1
    (lambda rp, ci: ci.__setitem__(slice(4, 6), ci[4:6][::-1].copy()), "ascending"),
    (lambda rp, ci: rp.__setitem__(0, 1), "row_ptr[0]"),
])
def test_check_route_rejects_malformed(mutate, msg):
    rp, ci = R.route_csr(R.BF1, 512, 64)
    rp, ci = rp.copy(), ci.copy()
    mutate(rp, ci)
    with pytest.raises(bsa.BsaError) as e:
        bsa.bsa_check_route(rp, ci)
    assert e.value.status == bsa.BSA_ERR_BAD_ROUTE


def test_check_route_rejects_missing_self_and_empty_rows():
    rp = np.array([0, 1, 2], dtype=np.int32)
    ci = np.array([0, 0], dtype=np.int32)  # row 1 lacks block 1
    with pytest.raises(bsa.BsaError):
        bsa.bsa_check_route(rp, ci)
    rp = np.array([0, 1, 1], dtype=np.int32)
    with pytest.raises(bsa.BsaError):
        bsa.bsa_check_route(rp, np.array([0], dtype=np.int32))
    # the non-causal toy adjacency of "Block Sparse Attention in LLMs" (section 6) is rejected
    rp = np.array([0, 2, 5, 8], dtype=np.int32)
    ci = np.array([0, 1, 0, 1, 2, 1, 2, 3], dtype=np.int32)
    with pytest.raises(bsa.BsaError):
        bsa.bsa_check_route(rp, ci)


def test_no_cpu_fallback_when_library_missing(monkeypatch, tmp_path):
    monkeypatch.setattr(bsa, "LIB_PATH", str(tmp_path / "libbsa.so"))
    monkeypatch.setattr(bsa, "_lib", None)
    with pytest.raises(RuntimeError):
        bsa.lib()
