"""CPU oracle for the block-canvas denoising step -- TEST INFRASTRUCTURE ONLY.

This package is the plain, slow, obviously-correct reference that the HIP
path is checked against. Only the test-suite, the smoke check and the
benchmark's CPU-baseline leg may import it; the library never does, and
nothing here shares code with the HIP sources.

It follows the DiffusionGemma Technical Report as summarised on hyper.ai
(cited below as "TR summary"), section "Method":
  * forward path equation: per coordinate, kappa_t * delta(x_t, x_0) +
    (1 - kappa_t) / V, with kappa_0 = 1, kappa_1 = 0, smooth and decreasing;
  * Step relation: P(X_{t-dt} | x_t) ~ Step(x_t, P(X_0 | x_t));
  * decoder equation: L_t = Decoder(x_t, z_t, H) in R^{C x V};
  * three-line update: p0 = Softmax(L_t / tau_t), z = FFW(p0 E),
    x_{t-dt} ~ Step(x_t, p0);
  * sampler paragraph: tau anneals linearly from 0.8 to 0.4; the
    entropy-bounded acceptance, uniform re-noising and adaptive stopping of
    the recommended sampler (entropy.py);
  * block-autoregressive paragraph and pipeline figure: prompt prefill,
    canvas commit to the KV cache and canvas-by-canvas generation
    (blocks.py);
  * the decoder as a deeper pre-norm stack with a gated MLP per layer, and
    that stack's causal encoder pass for prefill and commit (stack.py).

Readings taken where the pages stop short (each documented where used):
Step is the Euler step of the uniform-path CTMC,
(1 - lambda) delta(y, x_t) + lambda p0(y) with
lambda = clamp(dt * (-dkappa/dt) / (1 - kappa), 0, 1); FFW is the identity
(z = p0 E) unless a gated feed-forward block is given (ffw.py); the decoder
is one residual attention block with a tied head.

Floating point: reductions in float64; tensors are rounded to the
activation dtype (bf16 round-to-nearest-even or fp32) at the same tensor
boundaries as the library; integer decisions (Gumbel argmax, Bernoulli) are
taken in float32.

Parity pins: every function here is pinned by tests under tests/ that use
closed forms, invariants, published Philox known-answer vectors, brute force
and chi-square tests. The only part left "parity unpinned" is the complete
decoder output at configuration scale (no worked example is printed on the
pages); its parts are pinned separately.
"""
from .philox import philox4x32_10, uniform01, philox_scalar
from .schedule import schedule_terms, step_lambda, temperature, inv_temperature
from .rounding import round_act, round_bf16, round_f32
from .decoder import embed, qkv_proj, attention, out_proj, lm_head
from .sampling import bernoulli_uniforms, gumbel_noise, step_select
from .corrupt import corrupt
from .step import denoise_step, generate_canvas, self_condition
from .ffw import gelu_tanh, ffw, ffw_hidden
from .blocks import encode_kv, generate_blocks
from .stack import rmsnorm, layer, stack_step, causal_attention, encode_kv_stack
from .entropy import (row_entropy, accept_mask, renoise_tokens, entropy_step,
                      generate_canvas_entropy)

__all__ = [
    "philox4x32_10", "uniform01", "philox_scalar", "schedule_terms", "step_lambda",
    "temperature", "inv_temperature", "round_act", "round_bf16", "round_f32", "embed",
    "qkv_proj", "attention", "out_proj", "lm_head", "bernoulli_uniforms", "gumbel_noise",
    "step_select", "corrupt", "denoise_step", "generate_canvas", "row_entropy", "accept_mask",
    "renoise_tokens", "entropy_step", "generate_canvas_entropy", "self_condition", "gelu_tanh",
    "ffw", "ffw_hidden", "encode_kv", "generate_blocks", "rmsnorm", "layer", "stack_step",
    "causal_attention", "encode_kv_stack",
]
