"""One denoising step and one canvas generation, composed from the parts.

TR summary, Method: per iteration compute the logits, p0 = Softmax(L/tau),
the next self-conditioning signal z = FFW(p0 E), and resample every position
with Step (three-line update); FFW is the identity unless `w` carries the
gated block's weights (ffw.py); generation starts from noise and iterates over a
fixed time grid (the pages report about 12 steps per 256-token canvas and at
most 48, Experiments). Time grid (reading): t_k = 1 - k dt, dt = 1/steps,
k = 0 .. steps-1; step k uses Philox seed `seed + k` (mod 2^64) and the
initial canvas is the corruption of any canvas at kappa = 0 with `seed`.
"""
import numpy as np
from .schedule import step_lambda, inv_temperature
from .decoder import embed, qkv_proj, attention, out_proj, lm_head
from .sampling import step_select
from .corrupt import corrupt
from .ffw import ffw


def denoise_step(cfg, w, x_t, z_t, K_pre, V_pre, t, dt, seed, canvas_ids=None, want_p0=False):
    """`cfg` supplies shapes, dtype and schedule; `w` holds E, Wq, Wk, Wv, Wo
    and, for a feed-forward self-conditioning block, W_gate, W_up, W_down.

    x_t [B', C], z_t [B', C, d], K_pre/V_pre [B', Hkv, P, hd] and t [B'] may be
    a subset of canvases; `canvas_ids` gives their canvas indices (default
    0..B'-1), which select their Philox counters.
    """
    act = cfg.dtype
    Bp = x_t.shape[0]
    cid = np.arange(Bp) if canvas_ids is None else np.asarray(canvas_ids)
    t = np.asarray(t, dtype=np.float32)
    lam = np.array([step_lambda(float(tb), float(dt), cfg.schedule) for tb in t], dtype=np.float32)
    inv_tau = np.array([inv_temperature(float(tb)) for tb in t], dtype=np.float32)
    h0 = embed(w["E"], x_t, z_t, act)
    q, k, v = qkv_proj(h0, w["Wq"], w["Wk"], w["Wv"], cfg.n_q_heads, cfg.n_kv_heads, cfg.head_dim, act)
    o = attention(q, k, v, K_pre, V_pre, act)
    h1 = out_proj(o, w["Wo"], h0, act)
    head = lm_head(h1, w["E"], inv_tau, act, want_p0=want_p0)
    smp = step_select(x_t, head["s"], lam, seed, cid)
    out = dict(h0=h0, q=q, k=k, v=v, o=o, h1=h1, lam=lam, inv_tau=inv_tau, **head, **smp)
    out["p0E"] = head["z"]
    out["z_out"] = self_condition(w, head["z"], act)
    return out


def self_condition(w, p0E, act):
    """z = FFW(p0 E): the gated block when `w` holds its weights, else p0 E."""
    if w.get("W_gate") is None:
        return p0E
    return ffw(p0E, w["W_gate"], w["W_up"], w["W_down"], act)


def generate_canvas(cfg, w, K_pre, V_pre, steps, seed, keep_trace=False):
    """Generate a batch of canvases from uniform noise; returns x, z and the per-step trace."""
    B, C = K_pre.shape[0], cfg.C
    x = corrupt(np.zeros((B, C), np.int32), np.zeros(B, np.float32), seed, cfg.V)
    z = np.zeros((B, C, cfg.d))
    dt = float(np.float32(1.0 / steps))      # the step size and times travel as float32
    trace = [x.copy()]
    gaps = []
    for k in range(steps):
        t = np.float32(1.0 - k / steps)
        r = denoise_step(cfg, w, x, z, K_pre, V_pre, np.full(B, t, np.float32), dt,
                         (seed + k) % (1 << 64))
        x, z = r["x_out"], r["z_out"]
        trace.append(x.copy())
        gaps.append((r["resample"], r["gap"], r["top1"]))
    return {"x": x, "z": z, "trace": trace, "gaps": gaps}
