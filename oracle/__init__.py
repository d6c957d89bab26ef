"""CPU oracle of the LatentMoE layer forward and backward passes.

TEST INFRASTRUCTURE ONLY: imported by ``tests/``, ``__graft_entry__.smoke()``
and the ``cpu_baseline`` leg of ``bench.py``; never by the product path.
"""
from .latent_moe import (BIAS_MODES, E4M3_MAX, MODES, combine, expert_fp8_scales,  # noqa: F401
                         expert_rows, forward, forward_dense_bruteforce, forward_tokens,
                         fp8_matmul, fp8_scale_from_history, latent_down, latent_up,
                         lbl_stats, permute, quantize_e4m3, round_bf16, round_e4m3, round_schedule,
                         route,
                         router_logits, shared_expert, silu, softmax, swiglu_activation,
                         swiglu_expert,
                         topk_stable)
from . import latent_moe_backward  # noqa: F401,E402
from .latent_moe_backward import backward  # noqa: F401,E402
