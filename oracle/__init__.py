"""CPU oracle of the LatentMoE layer forward pass.

TEST INFRASTRUCTURE ONLY: imported by ``tests/``, ``__graft_entry__.smoke()``
and the ``cpu_baseline`` leg of ``bench.py``; never by the product path.
"""
from .latent_moe import (BIAS_MODES, MODES, combine, lbl_stats, expert_rows, forward,  # noqa: F401
                         forward_dense_bruteforce, forward_tokens, latent_down,
                         latent_up, permute, round_bf16, route, router_logits,
                         shared_expert, silu, softmax, swiglu_expert, topk_stable)
