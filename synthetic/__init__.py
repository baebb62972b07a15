"""Seeded synthetic workloads for the MoE dispatch/combine path.

This module is shared by the tests, the benchmark and the smoke check. It
only draws random numbers and lays them out in the shapes of the workloads;
it holds none of the routing, layout, permutation or combine arithmetic, so
neither the oracle nor the HIP library depends on anything here beyond the
arrays it returns.

Workload shapes follow the regimes the pages describe:
  * decode vs prefill sizes: aicassindra "gpu_moe_all_to_all", section
    "Latency-bound at decode, bandwidth-bound at prefill";
  * capacity factor 1.2: "MoE All-to-All Dispatch and Ragged Routing",
    section "Fixed Capacity vs. Ragged Routing";
  * 6 local experts out of 384: same page, section "Why MoE Token Dispatch is
    All-to-All";
  * 512 experts, 10 routed + 1 shared: ai-from-scratch "19. All-to-all",
    section "Why Qwen3.8's 512 experts is a systems statement";
  * the uniform round-robin assignment used as a diagnostic input:
    aicassindra "gpu_moe_all_to_all", section "How to tell whether the
    all-to-all is your bottleneck".

Random streams: one numpy PCG64 generator per tensor, seeded with
SeedSequence([seed, stream]) where stream is 0 logits, 1 bias, 2 x,
3 residual, 4 shared, 5 the stand-in expert weights. bf16 tensors are drawn as float32 normals and rounded
to bf16 by torch's CPU conversion; they are returned as uint16 bit patterns.
"""

from __future__ import annotations

import dataclasses
import math
from typing import Optional

import numpy as np

STREAM_LOGITS = 0
STREAM_BIAS = 1
STREAM_X = 2
STREAM_RESIDUAL = 3
STREAM_SHARED = 4
STREAM_EXPERT_W = 5


@dataclasses.dataclass(frozen=True)
class Workload:
    """Shape and distribution of one synthetic batch on one rank."""

    name: str
    T: int                      # tokens on this rank
    H: int                      # hidden width (bf16 elements per row)
    E: int                      # routed experts
    k: int                      # routed experts per token
    R: int                      # logical destination ranks (E % R == 0)
    bias: str = "none"          # "none" | "zeros" | "uniform" (+-bias_range)
    bias_range: float = 0.1
    skew: float = 0.0           # logits += skew * log(1 / (e + 1))
    capacity_factor: Optional[float] = None   # None: dropless
    shared: bool = False        # one always-on shared expert (dense input)
    residual: bool = True

    @property
    def local_experts(self) -> int:
        return self.E // self.R

    @property
    def capacity(self) -> int:
        """Integer per-expert row limit on this sender, -1 when dropless.

        Reading of "capacity factor": factor times the mean number of
        assignments per expert on this sender, T*k/E, rounded up. Each of a
        token's k replicas takes its own slot.
        """
        if self.capacity_factor is None:
            return -1
        return int(math.ceil(self.capacity_factor * self.T * self.k / self.E))

    def describe(self) -> str:
        parts = [f"T={self.T}", f"H={self.H}", f"E={self.E}",
                 f"k={self.k}" + ("+1 shared" if self.shared else ""),
                 f"R={self.R}"]
        if self.capacity_factor is not None:
            parts.append(f"capacity {self.capacity_factor} (C={self.capacity})")
        else:
            parts.append("dropless")
        if self.skew:
            parts.append(f"Zipf skew {self.skew}")
        if self.bias == "uniform":
            parts.append(f"selection bias U(-{self.bias_range},{self.bias_range})")
        return f"{self.name}: " + ", ".join(parts)


WORKLOADS = {
    1: Workload("tiny", T=256, H=512, E=16, k=2, R=4, bias="zeros"),
    2: Workload("decode", T=128, H=7168, E=256, k=8, R=32, bias="uniform"),
    3: Workload("prefill_capacity", T=16384, H=4096, E=64, k=2, R=8,
                skew=1.0, capacity_factor=1.2),
    4: Workload("ragged_dropless", T=4096, H=7168, E=384, k=8, R=64),
    5: Workload("fine_grained", T=32768, H=2048, E=512, k=10, R=64,
                skew=0.5, shared=True),
}


def rng(seed: int, stream: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, stream])))


def bf16_bits_from_f32(a: np.ndarray) -> np.ndarray:
    """Round float32 values to bf16 (torch's CPU conversion) and return the bits."""
    import torch
    t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32))
    return t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16).copy()


def normal_bf16(seed: int, stream: int, shape) -> np.ndarray:
    return bf16_bits_from_f32(rng(seed, stream).standard_normal(shape, dtype=np.float32))


def make_logits(w: Workload, seed: int = 0, T: Optional[int] = None) -> np.ndarray:
    T = w.T if T is None else T
    logits = rng(seed, STREAM_LOGITS).standard_normal((T, w.E), dtype=np.float32)
    if w.skew:
        ranks = np.arange(1, w.E + 1, dtype=np.float64)
        logits += (w.skew * np.log(1.0 / ranks)).astype(np.float32)
    return logits


def make_bias(w: Workload, seed: int = 0) -> Optional[np.ndarray]:
    if w.bias == "none":
        return None
    if w.bias == "zeros":
        return np.zeros(w.E, dtype=np.float32)
    if w.bias == "uniform":
        return rng(seed, STREAM_BIAS).uniform(-w.bias_range, w.bias_range, w.E).astype(np.float32)
    raise ValueError(w.bias)


def make_inputs(w: Workload, seed: int = 0, with_activations: bool = True) -> dict:
    """All host inputs of one batch as numpy arrays (bf16 tensors as uint16 bits)."""
    d = {
        "logits": make_logits(w, seed),
        "bias": make_bias(w, seed),
        "capacity": w.capacity,
    }
    if with_activations:
        d["x"] = normal_bf16(seed, STREAM_X, (w.T, w.H))
        d["residual"] = normal_bf16(seed, STREAM_RESIDUAL, (w.T, w.H)) if w.residual else None
        d["shared"] = normal_bf16(seed, STREAM_SHARED, (w.T, w.H)) if w.shared else None
    return d


def make_expert_weights(E_l: int, H_out: int, H: int, seed: int = 0) -> np.ndarray:
    """Stand-in expert weights [E_l][H_out][H] (one linear map per local
    expert, output-major like a linear layer's weight), float32 normals
    scaled by 1/sqrt(H) so outputs keep unit scale, as bf16 bits."""
    w = rng(seed, STREAM_EXPERT_W).standard_normal((E_l, H_out, H), dtype=np.float32)
    return bf16_bits_from_f32(w * np.float32(1.0 / math.sqrt(H)))


def round_robin_idx(T: int, E: int, k: int) -> np.ndarray:
    """Uniform round-robin assignment: token t's slot j goes to (t*k + j) mod E."""
    if k > E:
        raise ValueError("round-robin needs k <= E")
    a = np.arange(T * k, dtype=np.int64)
    return (a % E).astype(np.int32).reshape(T, k)
