"""Seeded synthetic workloads for MoE token dispatch and combine.

This module only draws inputs: token activations, router choices and router
weights. It holds none of the dispatch/combine arithmetic, so both the HIP path
and the CPU oracle can be fed from it without sharing any of the method.

Workload shapes follow the problem statement of the expert-parallel buffer API
(NeMo AutoModel ``uccl_ep.buffer``: ``Buffer.dispatch`` takes ``x`` as
``[num_tokens, hidden]`` bf16, ``topk_idx`` as ``[num_tokens, num_topk]`` int64
with ``-1`` for "no selection", and ``topk_weights`` as ``[num_tokens,
num_topk]`` float32). The batch sizes of the low-latency sweep are those of the
"Full dispatch benchmark table" on the NIXL EP page "nixl_ep: Optimize
low-latency NVLink path" (16 ... 512 tokens per rank).

Recipe (every draw comes from ``numpy.random.Generator(PCG64(seed))`` in the
order x, routing, weight logits):

* activations: f32 draws cast to bf16 with round-to-nearest-even by torch's CPU
  conversion; returned as raw ``uint16`` bit patterns;
* uniform routing: per token the first ``K`` entries of ``argsort`` of
  ``U[0,1)`` keys over the experts (a uniform random ``K``-subset, in random
  order);
* Zipf routing: ``p_i ~ (i+1)^-s`` over a seeded permutation of the experts,
  ``K`` draws without replacement taken as Gumbel-top-k on ``log p`` (the
  draw order is the ``k`` order);
* router weights: softmax of ``N(0,1)`` f32 logits over the chosen ``K``.
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import Optional

import numpy as np

__all__ = [
    "Workload",
    "to_bf16_bits",
    "bf16_bits_to_f32",
    "config_c1",
    "config_c2",
    "config_c3",
    "config_c4",
    "config_c5",
    "C3_SWEEP",
    "random_case",
    "by_name",
]

C3_SWEEP = (16, 32, 64, 128, 256, 512)


@dataclass
class Workload:
    """One batch of synthetic input.

    ``x`` holds bf16 bit patterns (``uint16``), row-major ``[T, H]``;
    ``topk_idx`` is int64 ``[T, K]``; ``topk_weights`` is float32 ``[T, K]``.
    ``A`` is the expert alignment, ``M`` the low-latency per-rank token
    capacity (or None), ``src_rank`` the logical rank this GPU plays in the
    low-latency layout, ``replicas`` the number of extra physical replicas
    for the replica-expanded routing (0 = none).
    """

    name: str
    T: int
    H: int
    E: int
    R: int
    K: int
    A: int
    x: np.ndarray
    topk_idx: np.ndarray
    topk_weights: np.ndarray
    M: Optional[int] = None
    src_rank: int = 0
    replicas: int = 0
    seed: int = 0
    meta: dict = field(default_factory=dict)

    @property
    def L(self) -> int:
        return self.E // self.R

    @property
    def P(self) -> int:
        return self.T * self.K


def to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """f32 array -> bf16 bit patterns (uint16), rounded by torch's CPU cast."""
    import torch

    t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32))
    return t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16).copy()


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """bf16 bit patterns (uint16) -> exact f32 values."""
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def _softmax_f32(logits: np.ndarray) -> np.ndarray:
    z = logits.astype(np.float32)
    z = z - z.max(axis=1, keepdims=True)
    e = np.exp(z, dtype=np.float32)
    return (e / e.sum(axis=1, keepdims=True, dtype=np.float32)).astype(np.float32)


def _uniform_subsets(rng: np.random.Generator, T: int, E: int, K: int) -> np.ndarray:
    keys = rng.random((T, E))
    return np.argsort(keys, axis=1, kind="stable")[:, :K].astype(np.int64)


def _zipf_without_replacement(rng: np.random.Generator, T: int, E: int, K: int, s: float):
    perm = rng.permutation(E)
    logp = -s * np.log(np.arange(1, E + 1, dtype=np.float64))
    scores = logp[None, :] + rng.gumbel(size=(T, E))
    order = np.argsort(-scores, axis=1, kind="stable")[:, :K]
    return perm[order].astype(np.int64), perm


def config_c1(seed: int = 1) -> Workload:
    """Tiny case: 64 tokens, hidden 256, 16 experts on 4 ranks, top-2 by logit."""
    T, H, E, R, K = 64, 256, 16, 4, 2
    rng = np.random.Generator(np.random.PCG64(seed))
    x = to_bf16_bits(rng.uniform(-1.0, 1.0, size=(T, H)).astype(np.float32))
    logits = rng.standard_normal((T, E)).astype(np.float32)
    # top-k by logit, descending; ties go to the lower expert id
    idx = np.argsort(-logits, axis=1, kind="stable")[:, :K].astype(np.int64)
    chosen = np.take_along_axis(logits, idx, axis=1)
    w = _softmax_f32(chosen)
    return Workload("c1_tiny", T, H, E, R, K, 1, x, idx, w, seed=seed)


def config_c2(seed: int = 2) -> Workload:
    """Standard shape: 128 tokens x 7168 hidden, 256 experts on 8 ranks, top-8 uniform."""
    T, H, E, R, K = 128, 7168, 256, 8, 8
    rng = np.random.Generator(np.random.PCG64(seed))
    x = to_bf16_bits(rng.standard_normal((T, H), dtype=np.float32))
    idx = _uniform_subsets(rng, T, E, K)
    w = _softmax_f32(rng.standard_normal((T, K), dtype=np.float32))
    return Workload("c2_standard", T, H, E, R, K, 1, x, idx, w, seed=seed)


def config_c3(M: int, seed: Optional[int] = None, src_rank: int = 0) -> Workload:
    """Low-latency padded layout: T = M tokens per rank, 8 ranks, hidden 7168, 256E top-8."""
    T, H, E, R, K = M, 7168, 256, 8, 8
    seed = 3000 + M if seed is None else seed
    rng = np.random.Generator(np.random.PCG64(seed))
    x = to_bf16_bits(rng.standard_normal((T, H), dtype=np.float32))
    idx = _uniform_subsets(rng, T, E, K)
    w = _softmax_f32(rng.standard_normal((T, K), dtype=np.float32))
    return Workload(f"c3_ll_m{M}", T, H, E, R, K, 1, x, idx, w, M=M, src_rank=src_rank, seed=seed)


def config_c4(seed: int = 4) -> Workload:
    """Skewed routing: 4096 tokens x 4096 hidden, 64 experts on 8 ranks, top-6 Zipf(1.2)."""
    T, H, E, R, K = 4096, 4096, 64, 8, 6
    rng = np.random.Generator(np.random.PCG64(seed))
    x = to_bf16_bits(rng.standard_normal((T, H), dtype=np.float32))
    idx, perm = _zipf_without_replacement(rng, T, E, K, 1.2)
    w = _softmax_f32(rng.standard_normal((T, K), dtype=np.float32))
    return Workload("c4_skewed", T, H, E, R, K, 1, x, idx, w, seed=seed, meta={"perm": perm})


def config_c5(seed: int = 5, T: int = 8192, H: int = 7168) -> Workload:
    """Replica-expanded routing: 8192 tokens x 7168, 256 logical experts top-8 Zipf(1.0), +32 replicas."""
    E, R, K = 256, 8, 8
    rng = np.random.Generator(np.random.PCG64(seed))
    x = to_bf16_bits(rng.standard_normal((T, H), dtype=np.float32))
    idx, perm = _zipf_without_replacement(rng, T, E, K, 1.0)
    w = _softmax_f32(rng.standard_normal((T, K), dtype=np.float32))
    return Workload("c5_replica", T, H, E, R, K, 1, x, idx, w, replicas=32, seed=seed,
                    meta={"perm": perm})


def random_case(seed: int, T: int, H: int, E: int, R: int, K: int, A: int = 1,
                neg_frac: float = 0.0, dup_frac: float = 0.0, bad_frac: float = 0.0,
                distinct: bool = False, M: Optional[int] = None, src_rank: int = 0,
                x_dist: str = "normal") -> Workload:
    """Edge-case generator: ids uniform in [0, E) with optional -1 entries,
    repeated ids inside a token's row, and out-of-range ids (``bad_frac``:
    values >= E or < -1)."""
    rng = np.random.Generator(np.random.PCG64(seed))
    if x_dist == "normal":
        xf = rng.standard_normal((T, H), dtype=np.float32)
    else:
        xf = rng.uniform(-1.0, 1.0, size=(T, H)).astype(np.float32)
    x = to_bf16_bits(xf)
    if distinct:
        if K > E:
            raise ValueError("distinct ids need K <= E")
        idx = _uniform_subsets(rng, T, E, K)
    else:
        idx = rng.integers(0, E, size=(T, K), dtype=np.int64)
    if dup_frac > 0 and K > 1:
        m = rng.random((T, K)) < dup_frac
        m[:, 0] = False
        idx = np.where(m, idx[:, :1], idx)
    if neg_frac > 0:
        idx = np.where(rng.random((T, K)) < neg_frac, -1, idx)
    if bad_frac > 0:
        bad = rng.choice(np.array([E, E + 7, -2, -100, 1 << 40], dtype=np.int64), size=(T, K))
        idx = np.where(rng.random((T, K)) < bad_frac, bad, idx)
    w = _softmax_f32(rng.standard_normal((T, K), dtype=np.float32)) if K > 0 else \
        np.zeros((T, 0), np.float32)
    return Workload(f"rand_s{seed}_T{T}_H{H}_E{E}_R{R}_K{K}_A{A}", T, H, E, R, K, A,
                    x, idx.astype(np.int64), w, M=M, src_rank=src_rank, seed=seed)


def by_name(name: str) -> Workload:
    if name in ("c1", "c1_tiny"):
        return config_c1()
    if name in ("c2", "c2_standard"):
        return config_c2()
    if name.startswith("c3"):
        return config_c3(int(name.split("m")[-1]))
    if name in ("c4", "c4_skewed"):
        return config_c4()
    if name in ("c5", "c5_replica"):
        return config_c5()
    raise KeyError(name)
