"""The five MoE-layer workloads, as shape and routing parameters.

A workload fixes the layer's shape (T tokens, model dim d, expert hidden
dim h, N experts, top-k), the gate variant, whether the k selected weights
are renormalised, the capacity factor and the arithmetic type of the
activations and weights. Nothing here computes anything of the method.
"""
from __future__ import annotations

from dataclasses import dataclass, replace
from typing import Optional


@dataclass(frozen=True)
class MoESpec:
    name: str
    T: int                  # tokens
    d: int                  # model dim
    h: int                  # expert hidden dim
    N: int                  # experts
    k: int                  # experts chosen per token
    capacity_factor: float  # capacity C = min(T, ceil(cf * T * k / N))
    gate: str               # "softmax" | "noisy" | "cosine"
    renorm: bool            # True: softmax over the k selected logits
                            # False: full softmax probability of each selected expert
    dtype: str              # "f32" | "bf16": x, gate matrices, expert weights, outputs
    proj_dim: int = 0       # cosine gate: projection width p
    temperature: float = 0.0  # cosine gate: tau (logits are cos / tau)
    zipf_s: float = 0.0     # > 0: per-expert logit bias from Zipf(s) rank weights
    expert_bias: bool = False  # b1/b2 present (all five workloads: absent, i.e. 0)

    def with_(self, **kw) -> "MoESpec":
        return replace(self, **kw)

    @property
    def inv_temperature(self) -> float:
        return 1.0 / self.temperature if self.temperature else 0.0


WORKLOADS = {
    # Tiny top-1 layer in fp32: the case the oracle finishes in well under a second.
    "tiny_top1_f32": MoESpec("tiny_top1_f32", T=256, d=64, h=256, N=4, k=1,
                             capacity_factor=1.2, gate="softmax", renorm=False, dtype="f32"),
    # Noisy top-2 gate, bf16 activations and weights, fp32 accumulation.
    "noisy_top2_bf16": MoESpec("noisy_top2_bf16", T=4096, d=1024, h=2048, N=8, k=2,
                               capacity_factor=1.2, gate="noisy", renorm=True, dtype="bf16"),
    # Large experts: the grouped GEMMs are compute bound.
    "large_expert_top2_bf16": MoESpec("large_expert_top2_bf16", T=8192, d=4096, h=14336, N=8, k=2,
                                      capacity_factor=1.25, gate="softmax", renorm=False, dtype="bf16"),
    # Fine-grained, Zipf-skewed cosine gate: most assignments are dropped.
    "cosine_zipf_top4_bf16": MoESpec("cosine_zipf_top4_bf16", T=16384, d=2048, h=1024, N=64, k=4,
                                     capacity_factor=1.5, gate="cosine", renorm=False, dtype="bf16",
                                     proj_dim=256, temperature=0.07, zipf_s=1.1),
    # Decode shape: 64 tokens over 128 experts, expert weights streamed from HBM.
    "decode_top8_bf16": MoESpec("decode_top8_bf16", T=64, d=4096, h=2048, N=128, k=8,
                                capacity_factor=128 / 8, gate="softmax", renorm=True, dtype="bf16"),
}

# Order in which the workloads are listed everywhere (smallest first).
WORKLOAD_ORDER = ["tiny_top1_f32", "noisy_top2_bf16", "large_expert_top2_bf16",
                  "cosine_zipf_top4_bf16", "decode_top8_bf16"]

# Seed of each workload's synthetic inputs.
WORKLOAD_SEED = {name: i + 1 for i, name in enumerate(WORKLOAD_ORDER)}


def get(name: str) -> MoESpec:
    return WORKLOADS[name]


def scaled(spec: MoESpec, T: Optional[int] = None, d: Optional[int] = None,
           h: Optional[int] = None, name: Optional[str] = None) -> MoESpec:
    """Same routing parameters at a smaller shape (for parity tests the oracle can finish)."""
    kw = {}
    if T is not None:
        kw["T"] = T
    if d is not None:
        kw["d"] = d
    if h is not None:
        kw["h"] = h
    kw["name"] = name or f"{spec.name}_T{T or spec.T}_d{d or spec.d}_h{h or spec.h}"
    return replace(spec, **kw)
