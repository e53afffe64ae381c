"""Seeded synthetic inputs for the MoE grouped-GEMM workloads.

This module is shared by the oracle tests, the GPU parity tests and the
benchmark, and it holds none of the method's arithmetic: it only draws
random numbers and turns router logits into top-k expert ids and gate
weights, which the workloads define as *input generation*.  The expert
histogram, offsets, gather/scatter indices and every GEMM are computed
elsewhere (by the oracle on the CPU, by the HIP library on the GPU) from
what this module returns.

All draws use CPU ``torch.Generator`` objects with fixed seeds, so the oracle
and the GPU receive the very same bytes.  bf16 values are fp32 normal draws
rounded to nearest-even by ``Tensor.to(torch.bfloat16)``.

Workloads (shapes of the pages' MoE layers; no dataset is involved):
  tiny          T=128, K=256, N=512, E=8, k=2; X, W ~ N(0, 0.02);
                routing = top-2 of softmax over N(0,1) logits; permute_x.
  dual          two groups X0[512,1024] @ W0[1024,2048], X1[256,1024] @
                W1[1024,4096]; entries N(0,1)/sqrt(1024); W stored [K, N].
  mixtral       T=4096, K=4096, N=28672 (2 x 14336), E=8, k=2; W ~ N(0,0.02),
                X ~ N(0,1); top-2 of softmax over N(0,1) logits; permute_x.
  fine_down     T=8192, E=128, k=8, K=768, N=2048; X ~ N(0,1) [T*k, K] already
                in expert order; W ~ N(0,0.02); Zipf(s=1.2) expert popularity
                with the 8 least popular experts never chosen; gate weights
                renormalised over the 8 chosen experts; permute_y +
                fuse_mul_post.
  fine_decode   the same layer with T=64 (same popularity order, fresh seed).
  fine_bwd      fine_down plus dY ~ N(0, 0.01) [T*k, N] in slot order.
"""

from __future__ import annotations

import math
from dataclasses import dataclass, field

import numpy as np
import torch

PERMUTE_X = 1
PERMUTE_Y = 2
FUSE_MUL_POST = 4

# Seeds: 1000 + the workload's number; the decode slice and dY have their own.
SEEDS = {"tiny": 1001, "dual": 1002, "mixtral": 1003, "fine_down": 1004,
         "fine_bwd_dy": 1005, "fine_decode": 1041, "mixtral_bwd_dy": 2003, "combine_y": 1046,
         "dense": 1007}


def generator(seed: int) -> torch.Generator:
    g = torch.Generator(device="cpu")
    g.manual_seed(int(seed))
    return g


def normal_bf16(shape, std: float, g: torch.Generator) -> torch.Tensor:
    """bf16 CPU tensor of N(0, std^2) draws (fp32 draw, round-to-nearest-even)."""
    return (torch.randn(*shape, generator=g, dtype=torch.float32) * std).to(torch.bfloat16)


def bits(t: torch.Tensor) -> np.ndarray:
    """Raw uint16 bit patterns of a bf16 CPU tensor (what the oracle takes)."""
    assert t.dtype == torch.bfloat16
    return t.contiguous().view(torch.int16).numpy().view(np.uint16)


def _topk_desc(scores: torch.Tensor, k: int) -> torch.Tensor:
    """Indices of the k largest scores per row; equal scores keep the lower id first."""
    order = torch.sort(scores, dim=-1, descending=True, stable=True).indices
    return order[:, :k]


def route_softmax_topk(T: int, E: int, k: int, g: torch.Generator):
    """Top-k of softmax over N(0,1) logits: ids int32 [T, k], weights fp32 [T, k]."""
    logits = torch.randn(T, E, generator=g, dtype=torch.float32)
    probs = torch.softmax(logits, dim=-1)
    ids = _topk_desc(probs, k)
    w = torch.gather(probs, 1, ids)
    return ids.to(torch.int32), w.contiguous()


def zipf_rank(E: int, g: torch.Generator) -> torch.Tensor:
    """rank[e] in 1..E: a seeded permutation giving each expert its popularity rank."""
    return torch.randperm(E, generator=g).to(torch.float64) + 1.0


def route_zipf(T: int, E: int, k: int, s: float, rank: torch.Tensor, g: torch.Generator,
               n_never: int = 8):
    """Zipf-popularity routing (expert popularity p_e proportional to rank_e^-s).

    Each token draws logits log p_e + Gumbel(0,1) and keeps the top k, which
    samples k distinct experts without replacement in proportion to p.  The
    n_never least popular experts are never chosen, so some experts are
    empty as the workload asks (pure Zipf over 65,536 slots leaves none
    empty).  Gate weights are the softmax over the k chosen logits, i.e. the
    renormalised top-k of the softmax over all experts.
    """
    logp = -s * torch.log(rank)
    u = torch.rand(T, E, generator=g, dtype=torch.float64).clamp_(1e-300, 1.0 - 1e-16)
    gumbel = -torch.log(-torch.log(u))
    logits = logp.unsqueeze(0) + gumbel
    logits[:, rank > (E - n_never)] = -math.inf
    ids = _topk_desc(logits, k)
    chosen = torch.gather(logits, 1, ids)
    w = torch.softmax(chosen, dim=-1).to(torch.float32)
    return ids.to(torch.int32), w.contiguous()


@dataclass
class Workload:
    name: str
    T: int = 0
    K: int = 0
    N: int = 0
    E: int = 0
    topk: int = 1
    flags: int = 0
    ids: torch.Tensor | None = None       # int32 [T, topk]
    weights: torch.Tensor | None = None   # fp32 [T, topk]
    X: torch.Tensor | None = None         # bf16 [T, K] (permute_x) or [T*topk, K]
    W: torch.Tensor | None = None         # bf16 [E, N, K]
    dY: torch.Tensor | None = None        # bf16 [T*topk, N]
    groups: list = field(default_factory=list)  # dual: [(X [m,k], W [k,n]), ...]

    @property
    def S(self) -> int:
        return self.T * self.topk


def tiny(T=128, K=256, N=512, E=8, topk=2, seed=SEEDS["tiny"]) -> Workload:
    g = generator(seed)
    ids, w = route_softmax_topk(T, E, topk, g)
    X = normal_bf16((T, K), 0.02, g)
    W = normal_bf16((E, N, K), 0.02, g)
    return Workload("tiny", T, K, N, E, topk, PERMUTE_X, ids, w, X, W)


def dual(seed=SEEDS["dual"], shapes=((512, 1024, 2048), (256, 1024, 4096))) -> Workload:
    g = generator(seed)
    xs = [normal_bf16((m, k), 1.0 / math.sqrt(k), g) for (m, k, n) in shapes]
    ws = [normal_bf16((k, n), 1.0 / math.sqrt(k), g) for (m, k, n) in shapes]
    return Workload("dual", groups=list(zip(xs, ws)))


def mixtral(T=4096, K=4096, N=28672, E=8, topk=2, seed=SEEDS["mixtral"]) -> Workload:
    g = generator(seed)
    ids, w = route_softmax_topk(T, E, topk, g)
    X = normal_bf16((T, K), 1.0, g)
    W = normal_bf16((E, N, K), 0.02, g)
    return Workload("mixtral", T, K, N, E, topk, PERMUTE_X, ids, w, X, W)


def dense(T=8192, K=4096, N=28672, seed=SEEDS["dense"]) -> Workload:
    """The Mixtral gate_up FLOPs as one dense product (a single expert, every
    row routed to it, no permutation): the shape on which the grouped kernels
    are compared with a vendor GEMM."""
    g = generator(seed)
    ids = torch.zeros(T, 1, dtype=torch.int32)
    w = torch.ones(T, 1, dtype=torch.float32)
    X = normal_bf16((T, K), 1.0, g)
    W = normal_bf16((1, N, K), 0.02, g)
    return Workload("dense", T, K, N, 1, 1, 0, ids, w, X, W)


def _fine(name, T, K, N, E, topk, s, seed, rank_seed, with_dy):
    rank = zipf_rank(E, generator(rank_seed))
    g = generator(seed)
    ids, w = route_zipf(T, E, topk, s, rank, g)
    X = normal_bf16((T * topk, K), 1.0, g)
    W = normal_bf16((E, N, K), 0.02, g)
    dY = normal_bf16((T * topk, N), 0.01, generator(SEEDS["fine_bwd_dy"])) if with_dy else None
    return Workload(name, T, K, N, E, topk, PERMUTE_Y | FUSE_MUL_POST, ids, w, X, W, dY)


def fine_down(T=8192, K=768, N=2048, E=128, topk=8, s=1.2, with_dy=False) -> Workload:
    """Popularity order comes from the fine_down seed; routing and X/W from the same stream."""
    return _fine("fine_down", T, K, N, E, topk, s, SEEDS["fine_down"], SEEDS["fine_down"], with_dy)


def fine_decode(T=64, K=768, N=2048, E=128, topk=8, s=1.2) -> Workload:
    """Decode slice: fine_down's popularity order, a fresh seed for routing and X/W."""
    return _fine("fine_decode", T, K, N, E, topk, s, SEEDS["fine_decode"], SEEDS["fine_down"],
                 False)


def fine_bwd(**kw) -> Workload:
    wl = fine_down(with_dy=True, **kw)
    wl.name = "fine_bwd"
    wl.flags = PERMUTE_Y   # the backward never carries the gate multiply
    return wl


def fine_decode_bwd(T=64, K=768, N=2048, E=128, topk=8, s=1.2) -> Workload:
    """The decode slice with an output gradient: the decode-shaped backward."""
    wl = _fine("fine_decode_bwd", T, K, N, E, topk, s, SEEDS["fine_decode"], SEEDS["fine_down"],
               True)
    wl.flags = PERMUTE_Y
    return wl


def random_routing(T: int, E: int, topk: int, g: torch.Generator, empty=()):
    """Uniform random top-k routing (distinct experts per token) avoiding `empty` experts."""
    allowed = torch.tensor([e for e in range(E) if e not in set(empty)], dtype=torch.int64)
    assert allowed.numel() >= topk
    scores = torch.rand(T, allowed.numel(), generator=g)
    pick = _topk_desc(scores, topk)
    ids = allowed[pick].to(torch.int32)
    w = torch.rand(T, topk, generator=g, dtype=torch.float32) + 0.1
    w = w / w.sum(-1, keepdim=True)
    return ids, w


def random_case(T: int, K: int, N: int, E: int, topk: int, flags: int, seed: int,
                empty=(), x_std=1.0, w_std=0.05, with_dy=False) -> Workload:
    """Small random MoE GEMM case for parity sweeps (ragged groups, empty experts)."""
    g = generator(seed)
    ids, w = random_routing(T, E, topk, g, empty)
    rows = T if (flags & PERMUTE_X) else T * topk
    X = normal_bf16((rows, K), x_std, g)
    W = normal_bf16((E, N, K), w_std, g)
    dY = normal_bf16((T * topk, N), 0.05, g) if with_dy else None
    return Workload(f"random_{seed}", T, K, N, E, topk, flags, ids, w, X, W, dY)


BUILDERS = {"tiny": tiny, "dual": dual, "mixtral": mixtral, "fine_down": fine_down,
            "fine_decode": fine_decode, "fine_bwd": fine_bwd, "fine_decode_bwd": fine_decode_bwd}
