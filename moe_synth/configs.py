"""Workload shapes of the LatentMoE layer.

Shapes follow the pages:
* MAI-Base-1: hidden 6,656, latent ("shared down-projection") 3,072, 8 of 512
  experts with softmax gating, expert FFN 10,240 ("The Training and RL
  Infrastructure Behind MAI-Thinking-1", section "The model the systems run",
  model table, MoE row).
* MAI-Base-2: hidden 8,704, MoE down-projection dimension 4,096, 7 of 512 routed
  experts plus one shared expert that is not down/up projected ("MAI-Base-2:
  Microsoft's 2.8T base model...", section "The model").
The routed width 8,192 and shared width 12,288 of the Base-2 shape are
synthetic choices (the pages give neither).  The tiny shape is a parity case.

Notation: T tokens, d hidden, L latent, E experts, k top-k, F routed SwiGLU
width (per branch), Fs shared SwiGLU width (0 = no shared expert).
"""
from __future__ import annotations

import dataclasses


@dataclasses.dataclass(frozen=True)
class MoEConfig:
    name: str
    T: int
    d: int
    L: int
    E: int
    k: int
    F: int
    Fs: int = 0
    zipf_bias: bool = False   # per-expert router bias b_e = -2.4 ln(rank_e)
    seed: int = 0
    description: str = ""

    @property
    def slots(self) -> int:
        return self.T * self.k

    def replace(self, **kw) -> "MoEConfig":
        return dataclasses.replace(self, **kw)

    def flops(self) -> float:
        """Algorithmic FLOPs of one forward pass: router 2TdE, latent down and
        up projections 4TdL, routed SwiGLU experts 6TkLF, shared expert 6TdFs."""
        T, d, L, E, k, F, Fs = self.T, self.d, self.L, self.E, self.k, self.F, self.Fs
        return 2.0 * T * d * E + 4.0 * T * d * L + 6.0 * T * k * L * F + 6.0 * T * d * Fs


CONFIGS = {
    "tiny": MoEConfig("tiny", T=256, d=512, L=256, E=16, k=2, F=512,
                      description="tiny LatentMoE, T=256 d=512 L=256 E=16 top-2 F=512"),
    "base1_small_batch": MoEConfig(
        "base1_small_batch", T=4096, d=6656, L=3072, E=512, k=8, F=10240,
        description="MAI-Base-1-shaped layer, T=4096 (memory-bound, weight streaming)"),
    "base1_compute": MoEConfig(
        "base1_compute", T=32768, d=6656, L=3072, E=512, k=8, F=10240,
        description="MAI-Base-1-shaped layer, T=32768 (compute-bound)"),
    "base1_imbalanced": MoEConfig(
        "base1_imbalanced", T=32768, d=6656, L=3072, E=512, k=8, F=10240, zipf_bias=True,
        description="MAI-Base-1-shaped layer, T=32768, Zipf-like router bias"),
    # Base-1 with the expert width the pages' parameter counts imply: 34.7B
    # active / 962B total parameters over 39 MoE layers give ~5,120 per SwiGLU
    # branch, so the table's "expert FFN 10,240" may be the fused gate+up width
    "base1_f5120": MoEConfig(
        "base1_f5120", T=4096, d=6656, L=3072, E=512, k=8, F=5120,
        description="MAI-Base-1-shaped layer, T=4096, SwiGLU width 5,120 per branch"),
    # one expert-parallel rank's share of the Base-1 layer (EP 8: 64 of the 512
    # experts, each receiving ~T*k/64 rows of the rank's T tokens); sized so
    # that the backward pass (fp32 weight gradients, transposed weight copies,
    # recomputed activations) fits one GPU
    "base1_ep8": MoEConfig(
        "base1_ep8", T=32768, d=6656, L=3072, E=64, k=8, F=10240,
        description="MAI-Base-1 layer, one EP-8 rank's share: T=32768, 64 experts"),
    "base2": MoEConfig(
        "base2", T=16384, d=8704, L=4096, E=512, k=7, F=8192, Fs=12288,
        description="MAI-Base-2-shaped layer, T=16384, top-7 + one shared expert"),
    # one expert-parallel rank's share of the Base-2 layer for the backward
    # pass (EP 8: 64 of the 512 routed experts, the shared expert replicated
    # and run on the rank's own T tokens)
    "base2_ep8": MoEConfig(
        "base2_ep8", T=16384, d=8704, L=4096, E=64, k=7, F=8192, Fs=12288,
        description="MAI-Base-2 layer, one EP-8 rank's share: T=16384, 64 experts + shared"),
}


def get_config(name: str) -> MoEConfig:
    return CONFIGS[name]
