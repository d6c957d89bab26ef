"""Seeded synthetic inputs for the LatentMoE layer forward pass.

This package is the one piece of code shared by the CPU oracle side (tests,
bench's CPU baseline) and the GPU side (parity tests, bench). It holds no
arithmetic of the layer itself: only workload shapes, a counter-based hash,
inverse-CDF lookup tables and the bf16 bit packing needed to materialise
identical input bytes on the host (numpy) and on the device (a small HIP
fill kernel of its own, ``moe_synth/csrc/synth_fill.hip``).
"""
from .configs import CONFIGS, MoEConfig, get_config  # noqa: F401
