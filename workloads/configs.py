"""The five synthetic workload shapes of the denoising step.

Sizes follow the decoder stand-in used throughout: one attention layer
(bidirectional over the canvas plus cross-attention to a prompt KV cache)
and a tied LM head, on a canvas of C tokens, as in the DiffusionGemma
Technical Report summary (hyper.ai), Method section: the decoder takes the
noisy canvas x_t, the self-conditioning signal z_t and the KV cache H, and
the canvas holds 256 tokens.
"""
from dataclasses import dataclass, field, replace
import math


@dataclass(frozen=True)
class Config:
    name: str
    B: int            # canvases in the batch
    C: int            # canvas length
    P: int            # prompt (prefix) length held in the KV cache
    d: int            # model width
    n_q_heads: int
    n_kv_heads: int
    head_dim: int
    V: int            # vocabulary size
    dtype: str        # "f32" or "bf16": weights, activations, KV cache
    schedule: str     # "linear" (kappa = 1 - t) or "cosine" (kappa = cos^2(pi t / 2))
    steps: int        # Euler steps of one canvas generation
    w_std: float      # std of Wq/Wk/Wv/Wo and of E
    kv_std: float = 1.0
    per_canvas_t: bool = False    # draw t_b ~ U(0, 1] per canvas
    zero_z_half: bool = False     # z_t = 0 for a seeded random half of the canvases
    seed: int = 0
    note: str = ""
    ffw_hidden: int = 0           # width F of the gated self-conditioning block (0: identity)
    ffw_gain: float = 1.0         # W_gate, W_up ~ N(0, (gain / sqrt(d))^2); W_down ~ N(0, 1 / F)
    n_layers: int = 0             # layers of the pre-norm decoder stack (0: the single block)
    mlp_hidden: int = 0           # hidden width of each stack layer's gated MLP (per expert)
    n_experts: int = 0            # experts of each stack layer's MLP (0: one dense MLP)
    top_k: int = 0                # experts per token

    @property
    def R(self):
        return self.B * self.C

    @property
    def group(self):
        return self.n_q_heads // self.n_kv_heads

    def with_(self, **kw):
        return replace(self, **kw)

    def flops_per_step(self):
        """Algorithmic FLOPs of one step (QKV, attention, O-projection, LM head + z)."""
        R, d, hd = self.R, self.d, self.head_dim
        Hq, Hkv = self.n_q_heads, self.n_kv_heads
        qkv = 2 * R * d * (Hq + 2 * Hkv) * hd
        attn = 4 * self.B * self.C * (self.P + self.C) * Hq * hd
        oproj = 2 * R * Hq * hd * d
        lm = 4 * R * self.V * d
        ffw = 6 * R * d * self.ffw_hidden
        L = max(1, self.n_layers)
        mlp = 6 * R * d * self.mlp_hidden * self.n_layers * (self.top_k if self.n_experts else 1)
        return dict(qkv=L * qkv, attn=L * attn, oproj=L * oproj, lm=lm, ffw=ffw, mlp=mlp,
                    total=L * (qkv + attn + oproj) + lm + ffw + mlp)


CONFIGS = {
    "c1": Config("tiny-fp32", B=1, C=16, P=8, d=32, n_q_heads=2, n_kv_heads=2, head_dim=16,
                 V=64, dtype="f32", schedule="linear", steps=8, w_std=1.0 / math.sqrt(32)),
    "c2": Config("standard", B=1, C=256, P=512, d=2048, n_q_heads=16, n_kv_heads=8, head_dim=128,
                 V=32768, dtype="bf16", schedule="cosine", steps=12, w_std=0.02),
    "c3": Config("long-prefix", B=1, C=256, P=32768, d=2048, n_q_heads=16, n_kv_heads=8,
                 head_dim=128, V=32768, dtype="bf16", schedule="cosine", steps=12, w_std=0.02),
    "c4": Config("large-vocab", B=1, C=256, P=2048, d=2816, n_q_heads=16, n_kv_heads=8,
                 head_dim=176, V=262144, dtype="bf16", schedule="cosine", steps=12, w_std=0.02),
    "c5": Config("batched", B=32, C=256, P=4096, d=2048, n_q_heads=16, n_kv_heads=8, head_dim=128,
                 V=131072, dtype="bf16", schedule="linear", steps=12, w_std=0.02,
                 per_canvas_t=True, zero_z_half=True),
}


def get_config(name, **overrides):
    cfg = CONFIGS[name]
    return cfg.with_(**overrides) if overrides else cfg
