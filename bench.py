#!/usr/bin/env python3
"""Benchmark: causal block-sparse attention forward (prefill) on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload qwen3_32k] [--no-cpu-baseline]
                    [--no-others] [--only backward|bsbr|decode]

Workload (default): the Qwen3-0.6B-shaped layer at 32K tokens — batch 1, 16 query / 8 key-value
heads, d = 128, block 128, bf16, BF1 route — the geometry the BF1 summary quotes its 32K
per-layer prefill speedup on.  Inputs are seeded N(0, 1) synthetic tensors already resident in
HBM when timing starts.

One step = one pass of the hot path: build the BF1 route (integer kernels) and run the
block-sparse forward over it.  W untimed warmup steps, then exactly K steps between HIP events
on the launch stream, bracketed by torch.cuda.synchronize().  Separately timed on the same
inputs: the forward alone (the dominant kernel, for the roofline: K launches right before and right
after the timed steps, the faster of the two), and the same kernel over the dense causal route
(the speedup denominator), in both orders sparse->dense and dense->sparse.

Also reported, outside the timed region: the backward pass (BF1 and dense route), selected-page decode of the newest token over the same
tensors as a key/value cache (batch 1 and 16; persistent plan, plan per token, dense route), the
topology sweep (BF1 against the local sliding band
and the static-random graph at the nearest selected-pair count, same inputs, with each graph's
communication depth), the forward alone on the other workloads, each against the roofline
that bounds it (HBM bytes, matrix-core flops or vector flops), and BSBR attention (within-chunk
term plus the retrieval over earlier chunks' states) on the 8K-token block-diagonal workload.

Prints ONE JSON line.  value = selected-interaction TFLOP/s of the step, where selected FLOPs =
4 * d * batch * heads_q * S and S counts the causal token pairs the route selects (QK^T and PV
only, the diagonal included).
"""

from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

BF16_PEAK_TFLOPS = 2500.0      # MI355X dense bf16 matrix peak (published)
FP32_VALU_PEAK_TFLOPS = 157.3  # MI355X fp32 vector peak (published)
HBM_PEAK_GBS = 8000.0          # MI355X HBM3E (published)


def selected_pairs(row_ptr: np.ndarray, col_idx: np.ndarray, n: int, B: int) -> int:
    """Causal token pairs selected by a CSR route (closed form per block pair)."""
    total = 0
    nqb = len(row_ptr) - 1
    for i in range(nqb):
        ti = min(B, n - i * B)
        for j in col_idx[row_ptr[i]:row_ptr[i + 1]]:
            j = int(j)
            if j < i:
                total += ti * min(B, n - j * B)
            elif j == i:
                total += ti * (ti + 1) // 2
    return total


def kernel_source_hash() -> str:
    """sha256 over the forward kernel sources (the traffic counters are tied to them)."""
    import hashlib
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "long_context_block_amd", "csrc")
    for name in ("fwd_common.hpp", "fwd_bf16.hip"):
        with open(os.path.join(csrc, name), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def time_loop(fn, steps: int, warmup: int):
    """Average ms per call over `steps` calls, timed with events on torch's current stream."""
    import torch
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    start, stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    start.record()
    for _ in range(steps):
        fn()
    stop.record()
    torch.cuda.synchronize()
    return start.elapsed_time(stop) / steps


def per_call_samples(fn, reps: int):
    """Per-call durations (ms) from event pairs around each call: median/p10/p90 reporting."""
    import torch
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(reps)]
    for a, b in evs:
        a.record()
        fn()
        b.record()
    torch.cuda.synchronize()
    return np.array([a.elapsed_time(b) for a, b in evs])


def gemm_reference(dev, size: int = 8192, reps: int = 20) -> dict:
    """A plain bf16 GEMM through torch (hipBLASLt) on random N(0,1) operands, timed like the
    forward: the matrix-core rate this GPU sustains under its power limit on realistic data,
    reported beside the published dense peak for context."""
    import torch
    g = torch.Generator(device=dev).manual_seed(0)
    a = torch.randn(size, size, dtype=torch.bfloat16, device=dev, generator=g)
    b = torch.randn(size, size, dtype=torch.bfloat16, device=dev, generator=g)
    c = torch.empty(size, size, dtype=torch.bfloat16, device=dev)
    ms = time_loop(lambda: torch.matmul(a, b, out=c), reps, 5)
    return {"what": f"torch.matmul bf16 {size}x{size}x{size}, random N(0,1) operands",
            "tflops": round(2.0 * size ** 3 / (ms * 1e-3) / 1e12, 1), "ms": round(ms, 4)}


def graph_depth(row_ptr: np.ndarray, col_idx: np.ndarray) -> tuple[int, int]:
    """Largest shortest-path hop count over ordered block pairs j < i, edges j -> i for j in R(i)
    (the communication depth the BF1 summary compares topologies by, section 5), over the pairs
    that are connected, and the number of pairs j < i with no path."""
    from collections import deque
    nqb = len(row_ptr) - 1
    succ = [[] for _ in range(nqb)]
    for i in range(nqb):
        for j in col_idx[row_ptr[i]:row_ptr[i + 1]]:
            if int(j) != i:
                succ[int(j)].append(i)
    worst, unreachable = 0, 0
    for src in range(nqb):
        dist = np.full(nqb, -1, dtype=np.int64)
        dist[src] = 0
        dq = deque([src])
        while dq:
            u = dq.popleft()
            for x in succ[u]:
                if dist[x] < 0:
                    dist[x] = dist[u] + 1
                    dq.append(x)
        tail = dist[src + 1:]
        unreachable += int((tail < 0).sum())
        if len(tail):
            worst = max(worst, int(tail.max()))
    return worst, unreachable


def topology_sweep(w, qd, kd, vd, steps: int) -> dict:
    """BF1 against its two equal-budget controls on the same inputs ("BF1 ...", section 5,
    "Topology control" and "Communication depth": at a matched pair count the page finds the three
    topologies' sparse kernel times close together, and compares their depths): the local sliding
    band and the static-random graph whose parameter gives the selected-pair count nearest to
    BF1's."""
    import torch
    import long_context_block_amd as bsa
    od = torch.empty_like(qd)

    def build(kind, **kw):
        spec = bsa.route_spec(kind, kw.get("n_local", w.n_local), w.keep_first, kw.get("n_random", w.n_random),
                              w.route_seed)
        rp, ci = bsa.build_route(spec, w.n, w.block)
        torch.cuda.synchronize()
        return rp, ci

    def pairs(rp, ci):
        return selected_pairs(rp.cpu().numpy(), ci.cpu().numpy(), w.n, w.block)

    rp0, ci0 = build(bsa.BSA_ROUTE_BF1)
    target = pairs(rp0, ci0)
    best = {}
    for kind, key in ((bsa.BSA_ROUTE_SLIDING_WINDOW, "n_local"), (bsa.BSA_ROUTE_STATIC_RANDOM, "n_random")):
        cands = []
        for val in range(0, 64):
            rp, ci = build(kind, **{key: val})
            cands.append((abs(pairs(rp, ci) - target), val))
        best[kind] = (key, min(cands)[1])
    out = {}
    routes = [("bf1", bsa.BSA_ROUTE_BF1, {}),
              ("sliding_window", bsa.BSA_ROUTE_SLIDING_WINDOW, {best[bsa.BSA_ROUTE_SLIDING_WINDOW][0]:
                                                               best[bsa.BSA_ROUTE_SLIDING_WINDOW][1]}),
              ("static_random", bsa.BSA_ROUTE_STATIC_RANDOM, {best[bsa.BSA_ROUTE_STATIC_RANDOM][0]:
                                                             best[bsa.BSA_ROUTE_STATIC_RANDOM][1]})]
    built = [(name, kw) + build(kind, **kw) for name, kind, kw in routes]
    fns = [(lambda rp=rp, ci=ci: bsa.bsa_forward(qd, kd, vd, od, rp, ci, w.block)) for _, _, rp, ci in built]
    t0 = time.perf_counter()
    while time.perf_counter() - t0 < 0.3:  # steady clock before the sweep
        for f in fns:
            f()
        torch.cuda.synchronize()
    best_ms = [float("inf")] * len(fns)
    for _ in range(3):  # interleaved rounds, best of three per route
        for x, f in enumerate(fns):
            best_ms[x] = min(best_ms[x], time_loop(f, steps, 3))
    for (name, kw, rp, ci), ms in zip(built, best_ms):
        S = pairs(rp, ci)
        depth, unreachable = graph_depth(rp.cpu().numpy(), ci.cpu().numpy())
        out[name] = {"params": kw, "nnz": int(ci.numel()), "selected_pairs_per_head": int(S),
                     "forward_ms": round(ms, 5),
                     "selected_tflops": round(4.0 * w.d * w.batch * w.heads_q * S / (ms * 1e-3) / 1e12, 2),
                     "depth_hops": depth, "unreachable_block_pairs": unreachable}
    return out


def decode_bench(w, kd, vd, steps: int, batch: int = 1) -> dict:
    """Selected-page decode on the workload's key/value tensors as a cache (newest token at the
    last position): with the route built once for the cache (persistent plan), with the plan
    rebuilt for every token (the pages' per-token accounting, "BF1 ...", section 5), with the
    row generated in the kernel (bsa_decode_routed: no plan at all), and over the dense causal
    route (the speedup denominator).  Algorithmic bytes: the selected key and
    value rows, q and o."""
    import torch
    import long_context_block_amd as bsa
    hq, d = w.heads_q, w.d
    e = 2 if w.dtype == "bf16" else 4
    g = torch.Generator(device=kd.device).manual_seed(7)
    q = torch.randn(batch, hq, d, device=kd.device, generator=g).to(kd.dtype)
    kc = kd.expand(batch, -1, -1, -1).contiguous() if batch > 1 else kd
    vc = vd.expand(batch, -1, -1, -1).contiguous() if batch > 1 else vd
    o = torch.empty_like(q)
    ws = torch.empty(bsa.bsa_decode_workspace_bytes(batch, hq, d) // 4, dtype=torch.float32, device=kd.device)
    sl = torch.full((batch,), w.n, dtype=torch.int32, device=kd.device)
    out = {"batch": batch, "token": w.n - 1}
    for name, kind in (("bf1", w.route_kind), ("dense_causal", bsa.BSA_ROUTE_DENSE_CAUSAL)):
        spec = bsa.route_spec(kind, w.n_local, w.keep_first, w.n_random, w.route_seed)
        rp, ci = bsa.build_route(spec, w.n, w.block)
        torch.cuda.synchronize()
        rph, cih = rp.cpu().numpy(), ci.cpu().numpy()
        i = (w.n - 1) // w.block
        sel = sum(min(w.block, w.n - int(j) * w.block) for j in cih[rph[i]:rph[i + 1]])
        nbytes = batch * (2 * w.heads_kv * sel * d * e + 2 * hq * d * e)
        fn = lambda: bsa.bsa_decode(q, kc, vc, o, sl, rp, ci, w.block, ws)  # noqa: E731
        ms = time_loop(fn, max(50, steps), 10)
        rec = {"selected_keys": int(sel), "ms": round(ms, 5), "algorithmic_bytes": int(nbytes),
               "GBs": round(nbytes / (ms * 1e-3) / 1e9, 1),
               "roofline": {"bound": "hbm", "peak": HBM_PEAK_GBS, "unit": "GB/s",
                            "frac": round(nbytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)}}
        # the same decode with the row generated inside the kernel from the route's closed form
        # (no route in memory, no planning launch)
        routed = lambda: bsa.bsa_decode_routed(q, kc, vc, o, sl, spec, w.block, ws)  # noqa: E731
        rec["ms_routed"] = round(time_loop(routed, max(50, steps), 10), 5)
        if name == "bf1":
            def planned():
                bsa.bsa_build_route(spec, w.n, w.block, rp, ci)
                fn()
            rec["ms_with_plan_per_token"] = round(time_loop(planned, max(50, steps), 10), 5)
        out[name] = rec
    out["speedup_vs_dense"] = round(out["dense_causal"]["ms"] / out["bf1"]["ms"], 3)
    return out


def backward_bench(w, qd, kd, vd, steps: int) -> dict:
    """The gradients (bsa_backward) of the workload's forward, BF1 route and dense causal route,
    with the transposed route built once.  FLOPs use the usual count for attention gradients,
    2.5x the forward's (five products of 2*d flops per selected pair: the recomputed scores, dP,
    dQ, dK, dV); the kernels also recompute the scores and dP once more (seven products)."""
    import torch
    import long_context_block_amd as bsa
    g = torch.Generator(device=qd.device).manual_seed(11)
    d_o = torch.randn(qd.shape, device=qd.device, generator=g).to(qd.dtype)
    out = {}
    for name, kind in (("bf1", w.route_kind), ("dense_causal", bsa.BSA_ROUTE_DENSE_CAUSAL)):
        spec = bsa.route_spec(kind, w.n_local, w.keep_first, w.n_random, w.route_seed)
        rp, ci = bsa.build_route(spec, w.n, w.block)
        trp, tci = bsa.build_route_transpose(rp, ci)
        o, lse = bsa.forward(qd, kd, vd, rp, ci, w.block, with_lse=True)
        dq, dk, dv = torch.empty_like(qd), torch.empty_like(kd), torch.empty_like(vd)
        nbytes = bsa.bsa_backward_workspace_bytes(w.batch, w.heads_q, w.heads_kv, w.n, w.d, w.block, ci.numel())
        ws = torch.empty(nbytes, dtype=torch.uint8, device=qd.device)
        torch.cuda.synchronize()
        S = selected_pairs(rp.cpu().numpy(), ci.cpu().numpy(), w.n, w.block)
        fn = lambda: bsa.bsa_backward(qd, kd, vd, o, d_o, lse, dq, dk, dv, rp, ci, trp, tci, w.block, ws)  # noqa: E731
        ms = time_loop(fn, max(5, steps // (1 if name == "bf1" else 10)), 2)
        flops = 10.0 * w.d * w.batch * w.heads_q * S
        out[name] = {"ms": round(ms, 5), "tflops": round(flops / (ms * 1e-3) / 1e12, 2),
                     "roofline": {"bound": "mfma", "peak": BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                                  "frac": round(flops / (ms * 1e-3) / 1e12 / BF16_PEAK_TFLOPS, 4)},
                     "workspace_bytes": int(nbytes)}
        del ws, dq, dk, dv, o, lse
        torch.cuda.empty_cache()
    out["speedup_vs_dense"] = round(out["dense_causal"]["ms"] / out["bf1"]["ms"], 3)
    return out


def algorithmic_bytes(w) -> int:
    """Q, K, V read once and O written once, in the workload's dtype."""
    e = 4 if w.dtype == "fp32" else 2
    return e * w.batch * w.n * w.d * (2 * w.heads_q + 2 * w.heads_kv)


def other_workloads(names, steps: int) -> dict:
    """The forward alone on the other workloads (parity cases of the same path), each against the
    roofline that bounds it: HBM bytes for the streaming cases (bf1_4k, the block-diagonal
    route), matrix-core flops for the 64K static-random graph, fp32 vector flops for the tiny
    fp32 case (launch-latency bound in practice)."""
    import torch
    import long_context_block_amd as bsa
    import synth
    out = {}
    for name in names:
        w = synth.WORKLOADS[name]
        q, k, v = (x.cuda() for x in synth.make_qkv(w))
        o = torch.empty_like(q)
        rp, ci = bsa.build_route(bsa.route_spec(w.route_kind, w.n_local, w.keep_first, w.n_random, w.route_seed),
                                 w.n, w.block)
        S = selected_pairs(rp.cpu().numpy(), ci.cpu().numpy(), w.n, w.block)
        fn = lambda: bsa.bsa_forward(q, k, v, o, rp, ci, w.block)  # noqa: E731
        ms = time_loop(fn, max(10, steps), 5)
        # the same kernel over the dense causal route on the same inputs (the speedup denominator)
        drp, dci = bsa.build_route(bsa.route_spec(bsa.BSA_ROUTE_DENSE_CAUSAL), w.n, w.block)
        ms_dense = time_loop(lambda: bsa.bsa_forward(q, k, v, o, drp, dci, w.block), max(3, steps // 10), 2)
        flops = 4.0 * w.d * w.batch * w.heads_q * S
        nbytes = algorithmic_bytes(w)
        tflops, gbs = flops / (ms * 1e-3) / 1e12, nbytes / (ms * 1e-3) / 1e9
        if w.dtype == "fp32":
            roof = {"bound": "alu", "achieved": round(tflops, 4), "peak": FP32_VALU_PEAK_TFLOPS, "unit": "TFLOP/s",
                    "frac": round(tflops / FP32_VALU_PEAK_TFLOPS, 6)}
        elif flops / nbytes < BF16_PEAK_TFLOPS * 1e12 / (HBM_PEAK_GBS * 1e9):
            roof = {"bound": "hbm", "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                    "frac": round(gbs / HBM_PEAK_GBS, 4)}
        else:
            roof = {"bound": "mfma", "achieved": round(tflops, 2), "peak": BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                    "frac": round(tflops / BF16_PEAK_TFLOPS, 4)}
        out[name] = {"forward_ms": round(ms, 5), "selected_tflops": round(tflops, 3),
                     "algorithmic_bytes": nbytes, "algorithmic_GBs": round(gbs, 1), "nnz": int(ci.numel()),
                     "selected_pairs_per_head": int(S), "dense_route_ms": round(ms_dense, 5),
                     "speedup_vs_dense": round(ms_dense / ms, 3), "roofline": roof}
        del q, k, v, o
        torch.cuda.empty_cache()
    return out


def bsbr_bench(steps: int) -> dict:
    """BSBR attention on the bsbr_chunk_8k workload (2 x 8 heads, n 8192, d 64, chunks of 128):
    the within-chunk term alone (the forward over the block-diagonal route) and the whole operator
    with the retrieval over earlier chunks' states.  HBM-bound by its algorithmic bytes (Q, K, V, O,
    meta queries and keys once); the retrieval's flops are the chunk states (2 n d^2 per key/value
    head), the mix (nch (nch - 1) d^2 per query head) and the read-out (2 n d^2 per query head)."""
    import torch
    import long_context_block_amd as bsa
    import synth
    w = synth.WORKLOADS["bsbr_chunk_8k"]
    q, k, v = (x.cuda() for x in synth.make_qkv(w))
    r, h = (x.cuda() for x in synth.make_meta(w))
    o = torch.empty_like(q)
    ws = torch.empty(bsa.bsa_bsbr_workspace_bytes(w.batch, w.heads_q, w.heads_kv, w.n, w.d, w.block),
                     dtype=torch.uint8, device=q.device)
    rp, ci = bsa.build_route(bsa.route_spec(bsa.BSA_ROUTE_BLOCK_DIAGONAL), w.n, w.block)
    steps = max(20, steps)
    ms_within = time_loop(lambda: bsa.bsa_forward(q, k, v, o, rp, ci, w.block), steps, 5)
    ms = time_loop(lambda: bsa.bsa_bsbr_forward(q, k, v, r, h, o, w.block, ws), steps, 5)
    nch = -(-w.n // w.block)
    nbytes = algorithmic_bytes(w) + 2 * w.batch * nch * w.d * (w.heads_q + w.heads_kv)
    flops_ret = (2.0 * w.n * w.d * w.d * w.batch * w.heads_kv + nch * (nch - 1) * w.d * w.d * w.batch * w.heads_q
                 + 2.0 * w.n * w.d * w.d * w.batch * w.heads_q)
    gbs = nbytes / (ms * 1e-3) / 1e9
    out = {"workload": w.name, "chunks": nch, "ms": round(ms, 5), "within_chunk_ms": round(ms_within, 5),
           "retrieval_ms": round(ms - ms_within, 5), "retrieval_flops": flops_ret,
           "algorithmic_bytes": int(nbytes), "algorithmic_GBs": round(gbs, 1),
           "roofline": {"bound": "hbm", "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                        "frac": round(gbs / HBM_PEAK_GBS, 4)},
           "workspace_bytes": int(ws.numel())}
    del q, k, v, r, h, o, ws
    torch.cuda.empty_cache()
    return out


def cpu_baseline(w, q, k, v, target_s: float = 15.0):
    """Time the fp64 oracle on the host over a bounded sample of query blocks of the workload, on
    the route oracle/routes.py builds from the workload's parameters (nothing from the GPU)."""
    from oracle import attn as A
    from oracle import routes as OR
    try:
        from threadpoolctl import threadpool_info
        blas_threads = max((d.get("num_threads", 1) for d in threadpool_info()), default=1)
    except Exception:
        blas_threads = os.cpu_count() or 1
    rp, ci = OR.route_csr(w.route_kind, w.n, w.block, **w.route_params())
    nqb = w.nqb
    order = np.linspace(0, nqb - 1, num=min(nqb, 64)).round().astype(int)
    done_rows, sel_pairs, t_used, blocks = 0, 0, 0.0, 0
    for blk in order:
        rows = np.arange(blk * w.block, min((blk + 1) * w.block, w.n))
        t0 = time.perf_counter()
        A.attention(q, k, v, w.block, rp, ci, rows=rows)
        t_used += time.perf_counter() - t0
        sel = 0
        ti = len(rows)
        for j in ci[rp[blk]:rp[blk + 1]]:
            sel += ti * min(w.block, w.n - int(j) * w.block) if j < blk else ti * (ti + 1) // 2
        sel_pairs += sel
        done_rows += ti
        blocks += 1
        if t_used >= target_s:
            break
    flops = 4.0 * w.d * w.batch * w.heads_q * sel_pairs
    return {"value": flops / t_used / 1e12, "unit": "TFLOP/s", "cores": int(blas_threads), "kind": "oracle",
            "sample": f"{w.name}: {blocks} of {nqb} query blocks ({done_rows} query rows x {w.batch * w.heads_q} "
                      f"heads, spread evenly over the sequence), fp64 masked-dense numpy on the oracle's own "
                      f"route, {t_used:.1f} s", "seconds": round(t_used, 2)}


def crossover(steps: int) -> dict:
    """BF1 against the dense causal route on the same inputs at the Qwen3 layer geometry (batch 1,
    16 query / 8 key-value heads, d 128) for n = 2K .. 32K at block widths 64 and 128: the forward
    time of each, the speedup, and the ratio of selected causal pairs (dense / BF1).  "BF1 ...",
    section 5 (per-layer prefill scaling) reports the crossover between 2K and 4K tokens and
    2.84x / 5.50x / 10.91x at 8K / 16K / 32K on its own hardware (context, not a target)."""
    import torch
    import long_context_block_amd as bsa
    import synth
    base = synth.WORKLOADS["qwen3_32k"]
    rows = []
    for n in (2048, 4096, 8192, 16384, 32768):
        w0 = base.resized(name=f"qwen3_{n // 1024}k", n=n)
        q, k, v = (x.cuda() for x in synth.make_qkv(w0))
        o = torch.empty_like(q)
        for B in (64, 128):
            w = w0.resized(block=B)
            rp, ci = bsa.build_route(bsa.route_spec(bsa.BSA_ROUTE_BF1, w.n_local, w.keep_first), n, B)
            drp, dci = bsa.build_route(bsa.route_spec(bsa.BSA_ROUTE_DENSE_CAUSAL), n, B)
            torch.cuda.synchronize()
            S = selected_pairs(rp.cpu().numpy(), ci.cpu().numpy(), n, B)
            S_dense = n * (n + 1) // 2
            f_bf1 = lambda: bsa.bsa_forward(q, k, v, o, rp, ci, B)  # noqa: E731
            f_dense = lambda: bsa.bsa_forward(q, k, v, o, drp, dci, B)  # noqa: E731
            reps = max(5, steps // (4 if n >= 16384 else 1))
            ms_bf1 = min(time_loop(f_bf1, reps, 3), time_loop(f_bf1, reps, 1))
            ms_dense = min(time_loop(f_dense, max(3, reps // 4), 2), time_loop(f_dense, max(3, reps // 4), 1))
            fl = 4.0 * w.d * w.batch * w.heads_q
            rows.append({"n": n, "block": B, "bf1_ms": round(ms_bf1, 5), "dense_ms": round(ms_dense, 5),
                         "speedup": round(ms_dense / ms_bf1, 3), "pair_ratio": round(S_dense / S, 3),
                         "bf1_selected_tflops": round(fl * S / (ms_bf1 * 1e-3) / 1e12, 1),
                         "dense_tflops": round(fl * S_dense / (ms_dense * 1e-3) / 1e12, 1),
                         "nnz_bf1": int(ci.numel())})
        del q, k, v, o
        torch.cuda.empty_cache()
    return {"geometry": "batch 1, 16/8 heads, d 128, BF1 n_local 2 with block 0, bf16", "rows": rows,
            "pages_speedup_context": {"8192": 2.84, "16384": 5.50, "32768": 10.91},
            "pages_crossover_context": "between 2K and 4K tokens"}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="qwen3_32k")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-others", action="store_true", help="skip the other workloads' forward timings")
    ap.add_argument("--cpu-seconds", type=float, default=15.0)
    ap.add_argument("--only", choices=["backward", "bsbr", "decode"], default=None,
                    help="run only this secondary section on the workload's inputs and print it (for profiling)")
    ap.add_argument("--copy-probe", type=int, default=0, metavar="MB",
                    help="run only a plain device-to-device copy of MB MiB (calibrates rocprofv3 "
                         "FETCH_SIZE/WRITE_SIZE against a known byte count) and exit")
    args = ap.parse_args()
    if args.copy_probe:
        import torch
        src = torch.ones(args.copy_probe * 2**20 // 4, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(5):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_probe_bytes": src.numel() * 4, "dispatches": 5}))
        return
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported (the path shards by "
              f"(batch, kv-head) with no collective and is measured on one GPU's share).", file=sys.stderr)
        sys.exit(2)

    import torch
    import long_context_block_amd as bsa
    import synth

    w = synth.WORKLOADS[args.workload]
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    q, k, v = synth.make_qkv(w)
    qd, kd, vd = q.to(dev), k.to(dev), v.to(dev)
    od = torch.empty_like(qd)
    if args.only:
        sect = {"backward": lambda: backward_bench(w, qd, kd, vd, args.steps),
                "bsbr": lambda: bsbr_bench(args.steps),
                "decode": lambda: [decode_bench(w, kd, vd, args.steps, batch) for batch in (1, 16)]}[args.only]
        print(json.dumps({"workload": w.name, args.only: sect()}), flush=True)
        return

    spec = bsa.route_spec(w.route_kind, w.n_local, w.keep_first, w.n_random, w.route_seed)
    nnz = bsa.bsa_build_route(spec, w.n, w.block)
    rp = torch.empty(w.nqb + 1, dtype=torch.int32, device=dev)
    ci = torch.empty(nnz, dtype=torch.int32, device=dev)
    ws = torch.empty(bsa.bsa_dense_route_workspace_bytes(w.n, w.block) // 4, dtype=torch.int32, device=dev)
    od_dense = torch.empty_like(qd)

    def route_step():
        bsa.bsa_build_route(spec, w.n, w.block, rp, ci)

    def fwd():
        bsa.bsa_forward(qd, kd, vd, od, rp, ci, w.block)

    def step():
        route_step()
        fwd()

    def dense():
        bsa.bsa_dense_causal_ref(qd, kd, vd, od_dense, ws, w.block)

    route_step()
    torch.cuda.synchronize()
    rp_h, ci_h = rp.cpu().numpy(), ci.cpu().numpy()
    S = selected_pairs(rp_h, ci_h, w.n, w.block)
    S_dense = w.n * (w.n + 1) // 2  # the dense causal route selects every causal pair
    flops = 4.0 * w.d * w.batch * w.heads_q * S
    flops_dense = 4.0 * w.d * w.batch * w.heads_q * S_dense

    # bring the GPU to its steady clock first (a few hundred ms of the forward, untimed)
    t0 = time.perf_counter()
    while time.perf_counter() - t0 < 0.3:
        for _ in range(10):
            fwd()
        torch.cuda.synchronize()
    # the dominant kernel alone, and the dense baseline, in both orders
    ms_fwd_a = time_loop(fwd, args.steps, 3)
    ms_dense_a = time_loop(dense, max(5, args.steps // 4), 2)
    ms_dense_b = time_loop(dense, max(5, args.steps // 4), 2)
    ms_fwd_b = time_loop(fwd, args.steps, 3)
    ms_route = time_loop(route_step, args.steps, 3)
    fwd_samples = per_call_samples(fwd, max(20, args.steps))
    # the timed region: W warmup steps, then K steps (route build + forward), bracketed by the
    # forward alone, K launches each, so that the kernel's time and the step's are taken under the
    # same clock conditions
    ms_fwd_c = time_loop(fwd, args.steps, 3)
    ms_step = time_loop(step, args.steps, args.warmup)
    ms_fwd_d = time_loop(fwd, args.steps, 3)
    ms_fwd = min(ms_fwd_c, ms_fwd_d)
    ms_dense = min(ms_dense_a, ms_dense_b)

    tflops_step = flops / (ms_step * 1e-3) / 1e12
    tflops_fwd = flops / (ms_fwd * 1e-3) / 1e12
    tflops_dense = flops_dense / (ms_dense * 1e-3) / 1e12
    peak = BF16_PEAK_TFLOPS if w.dtype == "bf16" else FP32_VALU_PEAK_TFLOPS

    # HBM traffic of the dominant kernel from committed rocprofv3 counters (profiles/), valid only
    # while the kernel source is the one that was profiled
    traffic = None
    tfile = os.path.join(ROOT, "profiles", f"traffic_{w.name}.json")
    if os.path.exists(tfile):
        with open(tfile) as f:
            rec = json.load(f)
        if rec.get("kernel_source_sha256") == kernel_source_hash():
            traffic = rec.get("traffic_bytes_per_launch")

    out = {
        "metric": "selected-interaction TFLOP/s (block-sparse attention forward, bf16 MFMA)",
        "value": round(tflops_step, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype,
        "data": "synthetic (seeded N(0,1) Q/K/V)",
        "config": {"workload": w.name, "batch": w.batch, "heads_q": w.heads_q, "heads_kv": w.heads_kv,
                   "seq_len": w.n, "head_dim": w.d, "block": w.block,
                   "route": {0: "bf1", 1: "block_diagonal", 2: "dense_causal", 3: "static_random",
                             4: "sliding_window"}[w.route_kind],
                   "nnz": int(nnz), "selected_pairs_per_head": int(S)},
        "pct_bf16_peak": round(100.0 * tflops_step / BF16_PEAK_TFLOPS, 2),
        "forward_ms": round(ms_fwd, 5),
        "forward_tflops": round(tflops_fwd, 2),
        "forward_ms_median_p10_p90": [round(float(np.median(fwd_samples)), 5),
                                      round(float(np.percentile(fwd_samples, 10)), 5),
                                      round(float(np.percentile(fwd_samples, 90)), 5)],
        "route_build_ms": round(ms_route, 5),
        "dense_route_ms": round(ms_dense, 5),
        "dense_route_tflops": round(tflops_dense, 2),
        "dense_ms_orders": {"sparse_then_dense": round(ms_dense_a, 5), "dense_then_sparse": round(ms_dense_b, 5)},
        "sparse_ms_orders": {"sparse_then_dense": round(ms_fwd_a, 5), "dense_then_sparse": round(ms_fwd_b, 5),
                             "before_step": round(ms_fwd_c, 5), "after_step": round(ms_fwd_d, 5)},
        "step_minus_forward_ms": round(ms_step - ms_fwd, 5),
        "speedup_vs_dense": round(ms_dense / ms_fwd, 3),
        "ideal_speedup_vs_dense": round(S_dense / S, 3),
        "roofline": {"bound": "mfma" if w.dtype == "bf16" else "alu", "achieved": round(tflops_fwd, 2),
                     "peak": peak, "unit": "TFLOP/s", "frac": round(tflops_fwd / peak, 4), "traffic": traffic,
                     "kernel": "fwd_bf16_kernel" if w.dtype == "bf16" else "fwd_f32_kernel"},
    }
    if w.dtype == "bf16":
        out["roofline"]["gemm_reference"] = gemm_reference(dev)
    if not args.no_others:
        out["topology_sweep"] = topology_sweep(w, qd, kd, vd, args.steps)
        out["decode"] = [decode_bench(w, kd, vd, args.steps, batch) for batch in (1, 16)]
        out["backward"] = backward_bench(w, qd, kd, vd, args.steps)
        out["other_workloads"] = other_workloads([x for x in synth.WORKLOADS if x != w.name], args.steps)
        out["bsbr"] = bsbr_bench(args.steps)
    if not args.no_others:
        out["crossover"] = crossover(args.steps)
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(w, q, k, v, args.cpu_seconds)
        if not args.no_others:
            out["cpu_baseline_other_workloads"] = {
                x: {key: val for key, val in cpu_baseline(synth.WORKLOADS[x], *synth.make_qkv(synth.WORKLOADS[x]),
                                                        target_s=max(1.0, args.cpu_seconds / 5)).items()
                    if key in ("value", "unit", "cores", "sample", "seconds")}
                for x in synth.WORKLOADS if x != w.name}
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
