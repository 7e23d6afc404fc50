"""Multi-layer decoder stack for the denoising step -- TEST INFRASTRUCTURE.

TR summary, Method: the decoder is a transformer (weight-shared
encoder-decoder, initialised from a Gemma mixture-of-experts checkpoint)
that maps the noisy canvas, the self-conditioning signal and the KV cache H
to logits; its layers are not described. This stack is the plainest deeper
stand-in built from the same parts as the single block, with the Gemma
family's pre-norm layout. Readings:
  * h0 = E[x] + z (as the single block);
  * layer l (own prefix cache K_l, V_l):
        a = rmsnorm(h) g_attn_l,   q, k, v = a Wq_l^T, a Wk_l^T, a Wv_l^T,
        h = h + attention(q, [K_l ; k], [V_l ; v]) Wo_l^T,
        m = rmsnorm(h) g_mlp_l,    h = h + W_down_l (gelu(W_gate_l m) * (W_up_l m));
    with rmsnorm(x) = x / sqrt(mean(x^2) + 1e-6), no biases;
  * mixture-of-experts variant of the MLP (the pages' model routes each
    token to a few of many experts; they give no routing rule): router
    logits r = m W_router^T in float32, the top_k experts by logit (ties to
    the lower expert index), weights = softmax over the top_k selected
    logits, h = h + sum_j w_j W_down_e (gelu(W_gate_e m) * (W_up_e m)) with
    each expert's hidden activations rounded to act and the weighted sum
    rounded once into h;
  * the LM head reads rmsnorm(h_L) g_final through the tied embedding;
  * everything after the logits (temperature, p0, z = FFW(p0 E), Step) is
    the single block's.
Rounding points (act dtype): h0, each normalised activation, q, k, v, o, each
residual sum, the MLP hidden activations, the final normalised activation;
sums in float64.

Causal encoder pass of the stack (encode_kv_stack): the pipeline figure's
first and third stages run the clean tokens through the causal encoder, which
fills and extends the KV cache; the encoder shares the decoder's weights
(weight-shared encoder-decoder). Readings: the encoder is the same pre-norm
stack run on h = E[x] (no self-conditioning input) with a causal mask: a new
token at cache row p attends to every cache row below p (the history and the
earlier new tokens) and to itself; layer l's cache entries are that layer's
key and value projections k = a Wk_l^T, v = a Wv_l^T of a = rmsnorm(h) g_attn_l.
The last layer's attention output and every MLP after it feed no cache entry
and are not computed.
"""
import numpy as np

from .decoder import attention, embed, lm_head
from .ffw import gelu_tanh
from .rounding import round_act
from .sampling import step_select
from .schedule import inv_temperature, step_lambda
from .step import self_condition

RMS_EPS = 1e-6


def rmsnorm(x, g, act):
    """round(x / sqrt(mean(x^2) + eps) * g) over the last axis."""
    x = np.asarray(x, np.float64)
    r = 1.0 / np.sqrt(np.mean(x * x, axis=-1, keepdims=True) + RMS_EPS)
    return round_act(x * r * np.asarray(g, np.float64), act)


def route(m, W_router, top_k):
    """Experts [R, top_k] (by float32 logit, ties to the lower index) and
    their softmax weights [R, top_k] (float64), plus the float32 logits."""
    r = (np.asarray(m, np.float64) @ np.asarray(W_router, np.float64).T).astype(np.float32)
    X = r.shape[1]
    idx = np.broadcast_to(np.arange(X), r.shape)
    order = np.lexsort((idx, -r.astype(np.float64)), axis=1)
    sel = order[:, :top_k]
    lg = np.take_along_axis(r, sel, axis=1).astype(np.float64)
    e = np.exp(lg - lg.max(axis=1, keepdims=True))
    return sel, e / e.sum(axis=1, keepdims=True), r


def moe_mlp(m, W_router, W_gate, W_up, W_down, top_k, act):
    """sum_j w_j expert_{e_j}(m) per row of m [R, d] (float64, unrounded)."""
    sel, wts, _ = route(m, W_router, top_k)
    out = np.zeros_like(np.asarray(m, np.float64))
    for e in range(np.shape(W_router)[0]):
        rows, slot = np.nonzero(sel == e)
        if rows.size == 0:
            continue
        x = np.asarray(m, np.float64)[rows]
        g = x @ np.asarray(W_gate[e], np.float64).T
        u = x @ np.asarray(W_up[e], np.float64).T
        hid = round_act(gelu_tanh(g) * u, act)
        out[rows] += wts[rows, slot][:, None] * (hid @ np.asarray(W_down[e], np.float64).T)
    return out


def layer(cfg, lw, h, K_pre, V_pre):
    """One pre-norm layer on h [B, C, d]; returns (h_out, parts)."""
    act = cfg.dtype
    B, C, d = h.shape
    Hq, Hkv, hd = cfg.n_q_heads, cfg.n_kv_heads, cfg.head_dim
    a = rmsnorm(h, lw["g_attn"], act)
    x = a.reshape(B * C, d)
    q = round_act(x @ np.asarray(lw["Wq"], np.float64).T, act).reshape(B, C, Hq, hd)
    k = round_act(x @ np.asarray(lw["Wk"], np.float64).T, act).reshape(B, C, Hkv, hd).transpose(0, 2, 1, 3)
    v = round_act(x @ np.asarray(lw["Wv"], np.float64).T, act).reshape(B, C, Hkv, hd).transpose(0, 2, 1, 3)
    o = attention(q, k, v, K_pre, V_pre, act)
    h1 = round_act(h + (o.reshape(B * C, Hq * hd) @ np.asarray(lw["Wo"], np.float64).T).reshape(B, C, d), act)
    m = rmsnorm(h1, lw["g_mlp"], act).reshape(B * C, d)
    if lw.get("W_router") is not None:
        y = moe_mlp(m, lw["W_router"], lw["W_gate"], lw["W_up"], lw["W_down"], lw["top_k"], act)
    else:
        g = m @ np.asarray(lw["W_gate"], np.float64).T
        u = m @ np.asarray(lw["W_up"], np.float64).T
        y = round_act(gelu_tanh(g) * u, act) @ np.asarray(lw["W_down"], np.float64).T
    h2 = round_act(h1 + y.reshape(B, C, d), act)
    return h2, dict(a=a, q=q, k=k, v=v, o=o, h_attn=h1, m=m.reshape(B, C, d), h=h2)


def stack_step(cfg, w, sw, x_t, z_t, K_pre, V_pre, t, dt, seed, canvas_ids=None):
    """One denoising step through the stack. `w` holds E (and optionally the
    FFW block); `sw` holds the per-layer weights as lists (Wq, Wk, Wv, Wo,
    g_attn, g_mlp, W_gate, W_up, W_down; with experts also W_router and the
    expert-major W_gate, W_up [X, F, d], W_down [X, d, F]) and g_final (and
    top_k with experts); K_pre, V_pre are [L, B, Hkv, P, hd]."""
    act = cfg.dtype
    Bp = x_t.shape[0]
    cid = np.arange(Bp) if canvas_ids is None else np.asarray(canvas_ids)
    t = np.asarray(t, dtype=np.float32)
    lam = np.array([step_lambda(float(tb), float(dt), cfg.schedule) for tb in t], dtype=np.float32)
    inv_tau = np.array([inv_temperature(float(tb)) for tb in t], dtype=np.float32)
    h = embed(w["E"], x_t, z_t, act)
    layers = []
    for l in range(len(sw["Wq"])):
        lw = {n: sw[n][l] for n in ["Wq", "Wk", "Wv", "Wo", "g_attn", "g_mlp", "W_gate", "W_up", "W_down"]}
        if sw.get("W_router") is not None:
            lw["W_router"], lw["top_k"] = sw["W_router"][l], sw["top_k"]
        h, parts = layer(cfg, lw, h, K_pre[l], V_pre[l])
        layers.append(parts)
    hf = rmsnorm(h, sw["g_final"], act)
    head = lm_head(hf, w["E"], inv_tau, act)
    smp = step_select(x_t, head["s"], lam, seed, cid)
    out = dict(h0=embed(w["E"], x_t, z_t, act), layers=layers, h_final=hf, lam=lam, inv_tau=inv_tau,
               **head, **smp)
    out["p0E"] = head["z"]
    out["z_out"] = self_condition(w, head["z"], act)
    return out


def causal_attention(q, k, v, K_hist, V_hist, act):
    """o [B, n, Hq, hd]: new token i attends to the history rows and to new
    tokens 0..i (one joint softmax, scale 1/sqrt(hd), head h reads kv head
    h // G). k, v [B, Hkv, n, hd]; K_hist, V_hist [B, Hkv, pos, hd]."""
    B, n, Hq, hd = q.shape
    Hkv = k.shape[1]
    G = Hq // Hkv
    pos = K_hist.shape[2]
    o = np.empty((B, n, Hq, hd), dtype=np.float64)
    scale = 1.0 / np.sqrt(hd)
    for b in range(B):
        for h in range(Hq):
            g = h // G
            keys = np.concatenate([np.asarray(K_hist[b, g], np.float64), k[b, g]], axis=0)
            vals = np.concatenate([np.asarray(V_hist[b, g], np.float64), v[b, g]], axis=0)
            s = (q[b, :, h, :] @ keys.T) * scale                 # [n, pos + n]
            visible = np.arange(pos + n)[None, :] <= pos + np.arange(n)[:, None]
            s = np.where(visible, s, -np.inf)
            s = s - s.max(axis=1, keepdims=True)
            a = np.exp(s)
            a /= a.sum(axis=1, keepdims=True)
            o[b, :, h, :] = a @ vals
    return round_act(o, act)


def encode_kv_stack(cfg, E, sw, tokens, K_cache, V_cache, pos):
    """Causal encoder pass of the stack over `tokens` [B, n] written at cache
    rows [pos, pos + n) of every layer. K_cache, V_cache [L, B, Hkv, P_cap, hd]
    hold the history in rows [0, pos). Returns copies of the caches with the
    new rows filled in, and the per-layer entries k, v [L][B, Hkv, n, hd]."""
    act = cfg.dtype
    tokens = np.asarray(tokens)
    B, n = tokens.shape
    Hq, Hkv, hd = cfg.n_q_heads, cfg.n_kv_heads, cfg.head_dim
    K = np.array(K_cache, dtype=np.float64, copy=True)
    V = np.array(V_cache, dtype=np.float64, copy=True)
    L = len(sw["Wq"])
    h = embed(E, tokens, np.zeros((B, n, cfg.d)), act)
    ks, vs = [], []
    for l in range(L):
        a = rmsnorm(h, sw["g_attn"][l], act)
        x = a.reshape(B * n, cfg.d)
        k = round_act(x @ np.asarray(sw["Wk"][l], np.float64).T, act).reshape(B, n, Hkv, hd).transpose(0, 2, 1, 3)
        v = round_act(x @ np.asarray(sw["Wv"][l], np.float64).T, act).reshape(B, n, Hkv, hd).transpose(0, 2, 1, 3)
        K[l, :, :, pos:pos + n] = k
        V[l, :, :, pos:pos + n] = v
        ks.append(k)
        vs.append(v)
        if l == L - 1:
            break
        q = round_act(x @ np.asarray(sw["Wq"][l], np.float64).T, act).reshape(B, n, Hq, hd)
        o = causal_attention(q, k, v, K[l, :, :, :pos], V[l, :, :, :pos], act)
        h = round_act(h + (o.reshape(B * n, Hq * hd) @ np.asarray(sw["Wo"][l], np.float64).T).reshape(B, n, cfg.d), act)
        m = rmsnorm(h, sw["g_mlp"][l], act).reshape(B * n, cfg.d)
        if sw.get("W_router") is not None:
            y = moe_mlp(m, sw["W_router"][l], sw["W_gate"][l], sw["W_up"][l], sw["W_down"][l], sw["top_k"], act)
        else:
            g = m @ np.asarray(sw["W_gate"][l], np.float64).T
            u = m @ np.asarray(sw["W_up"][l], np.float64).T
            y = round_act(gelu_tanh(g) * u, act) @ np.asarray(sw["W_down"][l], np.float64).T
        h = round_act(h + y.reshape(B, n, cfg.d), act)
    return {"K": K, "V": V, "k": ks, "v": vs}
