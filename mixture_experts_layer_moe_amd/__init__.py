"""LatentMoE feed-forward layer forward and backward passes on AMD MI355X (gfx950).

The compute lives in libmoe.so (hand-written HIP kernels behind the C ABI of
include/moe.h); this package is its Python binding.  Importing the package
does not load the library; the first call does, and raises if it is missing.
"""
from ._lib import (MOE_BIAS_LOGITS, MOE_BIAS_SELECTION, MOE_OP_BACKWARD,  # noqa: F401
                   MOE_OP_BACKWARD_FP8, MOE_OP_COMBINE, MOE_OP_LATENT_FFN, MOE_OP_LATENT_FFN_FP8,
                   MOE_OP_PERMUTE, MOE_OP_ROUTE, MOE_OP_SHARED_BACKWARD, MOE_ROUND_NEAREST,
                   MOE_ROUND_STOCHASTIC, MoEError, load, moe_backward, moe_backward_fp8,
                   moe_backward_prepare, moe_backward_prepare_shared, moe_backward_rounds,
                   moe_combine, moe_fp8_amax, moe_fp8_quantize, moe_fp8_scale_update,
                   moe_grad_cast_bf16, moe_grad_cast_e5m2, moe_latent_ffn_forward,
                   moe_latent_ffn_forward_fp8, moe_latent_ffn_forward_rounds, moe_permute,
                   moe_permute_noalloc, moe_route, moe_route_ex, moe_set_kernel_events,
                   moe_shared_backward, moe_status_string, moe_workspace_bytes,
                   moe_workspace_bytes_backward_rounds, moe_workspace_bytes_rounds)
from .layer import (Fp8GradScaling, Fp8Scaling, LatentMoEBuffers,  # noqa: F401
                    LatentMoEFp8Experts, LatentMoEFp8Transposed, LatentMoEGrads,
                    LatentMoETransposed, LatentMoEWeights, backward, backward_fp8,
                    backward_prepare, backward_rounds, forward, forward_fp8, forward_rounds, quantize_experts,
                    quantize_transposed)
