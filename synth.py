"""Seeded synthetic inputs and the workload table — shared by tests, bench and smoke.

This module holds no arithmetic of the attention method: it only names the
workloads (shapes, dtypes, route parameters) and draws seeded N(0, 1) inputs.
Both the CPU oracle and the GPU path read the very same host tensors it
returns, so the generator choice cannot affect parity.

Input recipe: ``torch.Generator('cpu').manual_seed(seed)``, then Q, K, V are
drawn in that order with ``torch.randn`` in float32 and cast to the workload's
dtype (round-to-nearest-even for bfloat16).

Workloads (sizes of the prefill measurements on the pages: the BF1 summary
times Qwen3-0.6B-shaped attention layers at batch 1 from 2K to 32K tokens; the
block-diagonal case is the BSBR within-chunk term; the static-random case is
BF1's nonlocal topology control at 64K tokens):
"""

from __future__ import annotations

from dataclasses import dataclass

import torch

ROUTE_BF1 = 0
ROUTE_BLOCK_DIAGONAL = 1
ROUTE_DENSE_CAUSAL = 2
ROUTE_STATIC_RANDOM = 3
ROUTE_SLIDING_WINDOW = 4


@dataclass(frozen=True)
class Workload:
    name: str
    batch: int
    heads_q: int
    heads_kv: int
    n: int
    d: int
    block: int
    dtype: str            # "fp32" or "bf16"
    route_kind: int
    n_local: int = 2
    keep_first: int = 1
    n_random: int = 14
    route_seed: int = 17
    input_seed: int = 1

    @property
    def torch_dtype(self):
        return torch.float32 if self.dtype == "fp32" else torch.bfloat16

    @property
    def nqb(self) -> int:
        return -(-self.n // self.block)

    def route_params(self) -> dict:
        return dict(n_local=self.n_local, keep_first=bool(self.keep_first),
                    n_random=self.n_random, seed=self.route_seed)

    def with_route(self, kind: int, name: str | None = None) -> "Workload":
        d = dict(self.__dict__)
        d["route_kind"] = kind
        d["name"] = name or f"{self.name}-{kind}"
        return Workload(**d)

    def resized(self, **kw) -> "Workload":
        d = dict(self.__dict__)
        d.update(kw)
        return Workload(**d)


WORKLOADS = {
    # tiny fp32 BF1 case: self (causal), 1 previous block, block 0, dyadic predecessors
    "tiny": Workload("tiny", 1, 1, 1, 512, 64, 64, "fp32", ROUTE_BF1, n_local=1, input_seed=1),
    # BF1 with 2 local neighbours at 4K
    "bf1_4k": Workload("bf1_4k", 1, 16, 16, 4096, 128, 64, "bf16", ROUTE_BF1, n_local=2, input_seed=2),
    # BSBR within-chunk term: block-diagonal route
    "bsbr_chunk_8k": Workload("bsbr_chunk_8k", 2, 8, 8, 8192, 64, 128, "bf16",
                              ROUTE_BLOCK_DIAGONAL, input_seed=3),
    # Qwen3-0.6B-shaped layer, GQA 16/8, BF1 at 32K (and the dense causal route on the same inputs)
    "qwen3_32k": Workload("qwen3_32k", 1, 16, 8, 32768, 128, 128, "bf16", ROUTE_BF1, n_local=2, input_seed=4),
    # static-random nonlocal graph at 64K: self + block 0 + 14 drawn earlier blocks, seed 17
    "static_random_64k": Workload("static_random_64k", 1, 32, 32, 65536, 128, 128, "bf16",
                                  ROUTE_STATIC_RANDOM, n_random=14, route_seed=17, input_seed=5),
}


def make_qkv(w: Workload, seed: int | None = None):
    """Seeded host tensors (q, k, v) of the workload's shape and dtype."""
    g = torch.Generator("cpu").manual_seed(w.input_seed if seed is None else seed)
    q = torch.randn(w.batch, w.heads_q, w.n, w.d, generator=g, dtype=torch.float32)
    k = torch.randn(w.batch, w.heads_kv, w.n, w.d, generator=g, dtype=torch.float32)
    v = torch.randn(w.batch, w.heads_kv, w.n, w.d, generator=g, dtype=torch.float32)
    dt = w.torch_dtype
    return q.to(dt), k.to(dt), v.to(dt)


def make_meta(w: Workload, seed: int | None = None):
    """Seeded host tensors (r, h) for the BSBR retrieval term: one meta query per chunk and query
    head, one meta key per chunk and key/value head, N(0, 1) in the workload's dtype (chunk width =
    the workload's block)."""
    g = torch.Generator("cpu").manual_seed((w.input_seed if seed is None else seed) + 1000)
    nch = -(-w.n // w.block)
    r = torch.randn(w.batch, w.heads_q, nch, w.d, generator=g, dtype=torch.float32)
    h = torch.randn(w.batch, w.heads_kv, nch, w.d, generator=g, dtype=torch.float32)
    dt = w.torch_dtype
    return r.to(dt), h.to(dt)
