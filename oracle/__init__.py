"""fp64 CPU oracle of the GPT-2 Pre-LN forward (test infrastructure only).

This package is the checker, not the product.  Only the test suite, the
smoke check and the CPU-baseline leg of the benchmark may import it; the HIP
library never calls into it, and nothing here calls the HIP library.

See ``oracle.gpt2`` for the functions and the passages each one follows.
"""
from .gpt2 import (  # noqa: F401
    bf16_round, layer_norm, gelu_new, gelu_erf, causal_attention, block_forward,
    embed, forward_hidden, forward, decode_logits, shifted_cross_entropy, lm_loss, generate_greedy,
    splitmix64, sample_uniforms, sample_token, generate_sample,
    gelu_new_grad, gelu_erf_grad, layer_norm_backward, block_backward, block_backward_batch, prepare_params,
    TRACE_POINTS,
)
