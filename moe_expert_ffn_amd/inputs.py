"""Seeded synthetic workloads for the MegaMoE expert pipeline.

This module only draws random inputs; it holds none of the method's arithmetic.
Both the HIP path and the CPU oracle are fed from here.

Workload shapes follow the MegaMoE pages' operator signature (pto-isa MegaMoE
overview, stage overview: x[M, K], expert_idx[M, topK], probs, weight1 producing
N = 2I columns, weight2 [N/2 -> K]).  Draw order is fixed: x, routing, logits,
w1, scale1, w2, scale2, all from one ``numpy.random.default_rng(seed)``.
"""
from __future__ import annotations

import dataclasses

import numpy as np


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    M: int          # tokens
    K: int          # hidden size
    E: int          # local experts
    top_k: int
    I: int          # SwiGLU output width; GMM1 produces 2*I columns
    routing: str = "uniform"   # "uniform" | "zipf" | "zipf_empty"

    @property
    def R(self) -> int:
        return self.M * self.top_k

    @property
    def N1(self) -> int:
        return 2 * self.I

    def describe(self) -> str:
        return (f"{self.name}: M={self.M} K={self.K} E={self.E} topK={self.top_k} "
                f"I={self.I} routing={self.routing}")


WORKLOADS = {
    # tiny forward: every stage fits in a handful of tiles
    "tiny": Workload("tiny", M=16, K=256, E=4, top_k=2, I=128),
    # decode-size: weight-streaming bound
    "decode": Workload("decode", M=128, K=7168, E=32, top_k=8, I=2048),
    "mid": Workload("mid", M=512, K=7168, E=32, top_k=8, I=2048),
    # large: compute-bound grouped GEMMs
    "large": Workload("large", M=2048, K=7168, E=32, top_k=8, I=2048),
    # skewed routing with Zipf(1.2) expert popularity
    "skewed": Workload("skewed", M=4096, K=4096, E=64, top_k=6, I=1408, routing="zipf"),
    # skewed routing with experts 48..63 never chosen (empty groups)
    "skewed_empty": Workload("skewed_empty", M=4096, K=4096, E=64, top_k=6, I=1408,
                             routing="zipf_empty"),
}


def zipf_popularity(E: int, s: float = 1.2, empty_from: int | None = None) -> np.ndarray:
    p = (np.arange(E, dtype=np.float64) + 1.0) ** (-s)
    if empty_from is not None:
        p[empty_from:] = 0.0
    return p / p.sum()


def draw_routing(rng: np.random.Generator, M: int, E: int, top_k: int, routing: str) -> np.ndarray:
    """Expert ids [M, top_k] int32, distinct within a token."""
    if routing == "uniform":
        return np.argsort(rng.random((M, E)), axis=1)[:, :top_k].astype(np.int32)
    if routing in ("zipf", "zipf_empty"):
        p = zipf_popularity(E, empty_from=(3 * E) // 4 if routing == "zipf_empty" else None)
        # Sampling top_k experts without replacement with probabilities p:
        # keys log(p_e) + Gumbel noise, take the top_k keys (Gumbel-top-k).
        with np.errstate(divide="ignore"):
            logp = np.log(p)
        g = -np.log(-np.log(rng.random((M, E))))
        keys = logp[None, :] + g
        return np.argsort(-keys, axis=1, kind="stable")[:, :top_k].astype(np.int32)
    raise ValueError(f"unknown routing {routing!r}")


def generate(w: Workload, seed: int = 0) -> dict[str, np.ndarray]:
    """All inputs of one forward, as numpy arrays.

    x        float16 [M, K]            ~ N(0, 1)
    expert_idx int32 [M, topK]
    probs    float32 [M, topK]         softmax of N(0, 1) logits
    w1       int8    [E, K, 2I]        uniform [-127, 127]; columns [0, I) feed silu
    scale1   float32 [E, 2I]           uniform [1e-3, 1e-2)
    w2       int8    [E, I, K]
    scale2   float32 [E, K]
    """
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((w.M, w.K), dtype=np.float32).astype(np.float16)
    expert_idx = draw_routing(rng, w.M, w.E, w.top_k, w.routing)
    logits = rng.standard_normal((w.M, w.top_k), dtype=np.float32)
    z = np.exp(logits - logits.max(axis=1, keepdims=True))
    probs = (z / z.sum(axis=1, keepdims=True)).astype(np.float32)
    w1 = rng.integers(-127, 128, (w.E, w.K, w.N1), dtype=np.int8)
    scale1 = rng.uniform(1e-3, 1e-2, (w.E, w.N1)).astype(np.float32)
    w2 = rng.integers(-127, 128, (w.E, w.I, w.K), dtype=np.int8)
    scale2 = rng.uniform(1e-3, 1e-2, (w.E, w.K)).astype(np.float32)
    return dict(x=x, expert_idx=expert_idx, probs=probs, w1=w1, scale1=scale1, w2=w2,
                scale2=scale2)


def custom(M: int, K: int, E: int, top_k: int, I: int, routing: str = "uniform",
           name: str | None = None) -> Workload:
    return Workload(name or f"M{M}_K{K}_E{E}_k{top_k}_I{I}_{routing}", M, K, E, top_k, I, routing)
