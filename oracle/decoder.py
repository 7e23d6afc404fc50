"""Decoder stand-in: embedding + self-conditioning, one attention block, tied LM head.

TR summary, Method, decoder equation: the decoder maps (x_t, z_t, H) to
logits L_t in R^{C x V}, with bidirectional attention across the canvas and
cross-attention to the KV cache H (three-stage generation pipeline
paragraph). The inner structure is not given; the reading used here is the
plainest one the configurations support:
  h0 = E[x_t] + z_t                      (z enters as an input embedding)
  q = h0 Wq^T, k = h0 Wk^T, v = h0 Wv^T  (weights stored [out, in])
  o = Attn(q, [K_pre ; k], [V_pre ; v])  one joint softmax over prefix and
                                         canvas keys, no mask, scale 1/sqrt(hd),
                                         query head h reads kv head h // G
  h1 = h0 + o Wo^T
  L = h1 E^T                              (tied embedding / LM head)
Tensors are rounded to the activation dtype at h0, q, k, v, o, h1 and z.
"""
import numpy as np
from .rounding import round_act


def embed(E, x, z, act):
    """h0 [B, C, d] = round(E[x] + z)."""
    return round_act(np.asarray(E, dtype=np.float64)[x] + np.asarray(z, dtype=np.float64), act)


def qkv_proj(h0, Wq, Wk, Wv, n_q_heads, n_kv_heads, head_dim, act):
    """Returns q [B, C, Hq, hd], k and v [B, Hkv, C, hd]."""
    B, C, d = h0.shape
    h = h0.reshape(B * C, d)
    q = round_act(h @ np.asarray(Wq, np.float64).T, act).reshape(B, C, n_q_heads, head_dim)
    k = round_act(h @ np.asarray(Wk, np.float64).T, act).reshape(B, C, n_kv_heads, head_dim)
    v = round_act(h @ np.asarray(Wv, np.float64).T, act).reshape(B, C, n_kv_heads, head_dim)
    return q, k.transpose(0, 2, 1, 3).copy(), v.transpose(0, 2, 1, 3).copy()


def attention(q, k, v, K_pre, V_pre, act):
    """o [B, C, Hq, hd]: per (b, h) a full softmax over the P + C keys of kv head h // G."""
    B, C, Hq, hd = q.shape
    Hkv = k.shape[1]
    G = Hq // Hkv
    o = np.empty((B, C, Hq, hd), dtype=np.float64)
    scale = 1.0 / np.sqrt(hd)
    for b in range(B):
        for h in range(Hq):
            g = h // G
            keys = np.concatenate([np.asarray(K_pre[b, g], np.float64), k[b, g]], axis=0)
            vals = np.concatenate([np.asarray(V_pre[b, g], np.float64), v[b, g]], axis=0)
            s = (q[b, :, h, :] @ keys.T) * scale           # [C, P + C]
            s = s - s.max(axis=1, keepdims=True)
            a = np.exp(s)
            a /= a.sum(axis=1, keepdims=True)
            o[b, :, h, :] = a @ vals
    return round_act(o, act)


def out_proj(o, Wo, h0, act):
    B, C, Hq, hd = o.shape
    y = o.reshape(B * C, Hq * hd) @ np.asarray(Wo, np.float64).T
    return round_act(h0 + y.reshape(h0.shape), act)


def lm_head(h1, E, inv_tau, act, want_p0=False):
    """Scaled logits s = (h1 E^T) * inv_tau_b, their log-sum-exp, p0 and z = p0 E.

    TR summary, Method, three-line update: p0 = Softmax(L_t / tau_t) and the
    self-conditioning signal z = FFW(p0 E) with FFW read as the identity.
    `inv_tau` holds one float32 value per canvas. Returns a dict with
    s [R, V] (float64), lse [R], z [B, C, d] (rounded) and optionally p0.
    """
    B, C, d = h1.shape
    Ef = np.asarray(E, dtype=np.float64)
    L = h1.reshape(B * C, d) @ Ef.T
    s = L * np.repeat(np.asarray(inv_tau, np.float64), C)[:, None]
    m = s.max(axis=1, keepdims=True)
    e = np.exp(s - m)
    l = e.sum(axis=1, keepdims=True)
    p0 = e / l
    lse = (m + np.log(l))[:, 0]
    z = round_act(p0 @ Ef, act).reshape(B, C, d)
    out = {"s": s, "lse": lse, "z": z}
    if want_p0:
        out["p0"] = p0
    return out
