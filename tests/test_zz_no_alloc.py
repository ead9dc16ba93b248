"""bsa_decode_routed_noalloc (partials in the library's static scratch array, no workspace) against
bsa_decode_routed with a caller workspace: the same kernels and split count, so the outputs and
LSEs must be equal bit for bit.  Two calls in a row on one device, the second smaller than the
first, so a result that read the previous call's leftovers would differ."""

import pytest
import torch

import long_context_block_amd as bsa

pytestmark = pytest.mark.gpu

CASES = [  # (batch, heads_q, heads_kv, n_max, d, block, dtype, route kind, n_local, seed)
    (8, 16, 8, 8192, 128, 128, torch.bfloat16, bsa.BSA_ROUTE_BF1, 2, 71),
    (3, 4, 2, 2000, 64, 64, torch.bfloat16, bsa.BSA_ROUTE_SLIDING_WINDOW, 5, 72),
    (2, 2, 1, 700, 64, 64, torch.float32, bsa.BSA_ROUTE_DENSE_CAUSAL, 0, 73),
]


def _inputs(batch, hq, hkv, n_max, d, dtype, seed):
    g = torch.Generator("cpu").manual_seed(seed)
    q = torch.randn(batch, hq, d, generator=g).to(dtype).cuda()
    k = torch.randn(batch, hkv, n_max, d, generator=g).to(dtype).cuda()
    v = torch.randn(batch, hkv, n_max, d, generator=g).to(dtype).cuda()
    lens = torch.randint(1, n_max + 1, (batch,), generator=g, dtype=torch.int32)
    lens[0] = n_max
    return q, k, v, lens.cuda()


def _both(case):
    batch, hq, hkv, n_max, d, block, dtype, kind, n_local, seed = case
    print(f"no-alloc decode: batch={batch} hq={hq} hkv={hkv} n_max={n_max} d={d} block={block} "
          f"dtype={dtype} kind={kind}", flush=True)
    q, k, v, lens = _inputs(batch, hq, hkv, n_max, d, dtype, seed)
    spec = bsa.route_spec(kind, n_local)
    o_ref, lse_ref = bsa.decode_routed(q, k, v, lens, spec, block, with_lse=True)
    o = torch.full_like(q, float("nan"))
    lse = torch.full((batch, hq), float("nan"), dtype=torch.float32, device=q.device)
    bsa.bsa_decode_routed_noalloc(q, k, v, o, lens, spec, block, lse=lse)
    torch.cuda.synchronize()
    return o, lse, o_ref, lse_ref


def test_noalloc_decode_equals_workspace_decode_two_calls_in_a_row():
    outs = [_both(CASES[0]), _both(CASES[1])]  # the second call is smaller than the first
    for o, lse, o_ref, lse_ref in outs:
        assert torch.equal(o, o_ref)
        assert torch.equal(lse, lse_ref)


def test_noalloc_decode_fp32_and_repeat():
    for case in (CASES[2], CASES[0], CASES[2]):
        o, lse, o_ref, lse_ref = _both(case)
        assert torch.equal(o, o_ref)
        assert torch.equal(lse, lse_ref)
