"""Entropy-bounded Step with adaptive stopping (the pages' recommended sampler).

TR summary, Method, sampler paragraph: the sampler ranks canvas positions by
the entropy of their predicted distribution, from low to high, and accepts
tokens in that order while a bound on their mutual information stays strictly
below an error tolerance; every other position is re-noised with a uniformly
random token. Probabilities are sharpened by the annealed temperature
(tau 0.8 -> 0.4, the same schedule as the Step path); z is the same
self-conditioning signal as on the Step path (step.self_condition). Adaptive stopping ends
the loop once the mean predicted entropy over the canvas is below a threshold
and the deterministic predictions of two consecutive steps are identical.
Experiments: at most 48 steps, about 12 on average; acceptance and stopping
use different entropy thresholds.

Readings taken here (the pages give no formulas):
  * entropy H = -sum_v p0(v) ln p0(v), in nats, of the tempered distribution;
  * the mutual-information bound of a set of simultaneously accepted tokens
    is the sum of their entropies (the total correlation of a set is at most
    the sum of the marginal entropies); the accepted set is the longest prefix
    of the entropy order whose running sum stays below eps_accept, and always
    holds at least the lowest-entropy position, so every step commits a token;
  * entropy ties are ordered by canvas position;
  * an accepted position takes the Gumbel-max draw of the Step path (Philox
    stream 0, same counters);
  * a rejected position is re-noised with floor(w V / 2^32), w = word 0 of
    Philox block (0, i, b, 3);
  * the deterministic prediction is argmax_v s(v) of the float32 scaled
    logits, lowest id on ties;
  * stop_b = (mean_i H_{b,i} < eps_stop) and (the deterministic predictions
    equal the previous step's at every position); never on a canvas's first
    step; a stopped canvas keeps its tokens and z.
"""
import numpy as np
from .schedule import inv_temperature
from .decoder import embed, qkv_proj, attention, out_proj, lm_head
from .sampling import gumbel_noise
from .philox import philox4x32_10, mulhi_token
from .corrupt import corrupt
from .step import self_condition


def row_entropy(s):
    """H[n] = -sum_v p ln p with p = softmax(s[n]) (float64, nats)."""
    s = np.asarray(s, dtype=np.float64)
    m = s.max(axis=1, keepdims=True)
    e = np.exp(s - m)
    l = e.sum(axis=1)
    return np.log(l) - (e * (s - m)).sum(axis=1) / l


def accept_mask(H, eps_accept):
    """Per canvas (rows of H [B, C]): positions in entropy order (ties by
    position), accepted while the running entropy sum is < eps_accept, and
    at least the first."""
    H = np.asarray(H, dtype=np.float64)
    B, C = H.shape
    mask = np.zeros((B, C), dtype=bool)
    pos = np.arange(C)
    for b in range(B):
        order = np.lexsort((pos, H[b]))          # primary key H, then position
        run = np.cumsum(H[b][order])
        take = run < eps_accept
        take[0] = True
        mask[b, order] = take
    return mask


def renoise_tokens(seed, canvas_ids, C, V):
    """Uniform re-noise token of every (canvas, position): floor(w V / 2^32)."""
    b = np.asarray(canvas_ids, dtype=np.uint64)[:, None]
    i = np.arange(C, dtype=np.uint64)[None, :]
    w0, _, _, _ = philox4x32_10(0, i, b, 3, seed)
    return mulhi_token(w0, V).astype(np.int32)


def entropy_step(cfg, w, x_t, z_t, K_pre, V_pre, t, seed, eps_accept, eps_stop, det_prev=None,
                 canvas_ids=None, want_p0=False):
    """One entropy-bounded step for canvases x_t [B', C] (a subset when
    `canvas_ids` is given); `det_prev` [B', C] are the previous step's
    deterministic predictions, or None on the first step."""
    act = cfg.dtype
    Bp, C = x_t.shape
    V = cfg.V
    cid = np.arange(Bp) if canvas_ids is None else np.asarray(canvas_ids)
    t = np.asarray(t, dtype=np.float32)
    inv_tau = np.array([inv_temperature(float(tb)) for tb in t], dtype=np.float32)
    h0 = embed(w["E"], x_t, z_t, act)
    q, k, v = qkv_proj(h0, w["Wq"], w["Wk"], w["Wv"], cfg.n_q_heads, cfg.n_kv_heads, cfg.head_dim, act)
    o = attention(q, k, v, K_pre, V_pre, act)
    h1 = out_proj(o, w["Wo"], h0, act)
    head = lm_head(h1, w["E"], inv_tau, act, want_p0=want_p0)
    s = head["s"]
    H = row_entropy(s).reshape(Bp, C)
    s32 = s.astype(np.float32)
    det = np.argmax(s32, axis=1).reshape(Bp, C)
    srt = np.sort(s32, axis=1)
    det_gap = (srt[:, -1] - srt[:, -2]).reshape(Bp, C) if V > 1 else np.full((Bp, C), np.inf)
    det_top = srt[:, -1].reshape(Bp, C)
    rows_b = np.repeat(cid, C)
    rows_i = np.tile(np.arange(C), Bp)
    pert = s32 + gumbel_noise(seed, rows_b, rows_i, V)
    y = np.argmax(pert, axis=1).reshape(Bp, C)
    ps = np.sort(pert, axis=1)
    top1 = ps[:, -1].reshape(Bp, C)
    gap = (ps[:, -1] - ps[:, -2]).reshape(Bp, C) if V > 1 else np.full((Bp, C), np.inf)
    acc = accept_mask(H, eps_accept)
    rn = renoise_tokens(seed, cid, C, V)
    x_out = np.where(acc, y, rn).astype(np.int32)
    if det_prev is None:
        stop = np.zeros(Bp, dtype=bool)
    else:
        stop = (H.mean(axis=1) < eps_stop) & np.all(det == np.asarray(det_prev), axis=1)
    out = dict(h0=h0, q=q, k=k, v=v, o=o, h1=h1, inv_tau=inv_tau, **head)
    out.update(H=H, det=det.astype(np.int32), det_gap=det_gap, det_top=det_top, y=y.astype(np.int32),
               top1=top1, gap=gap, accept=acc, renoise=rn, x_out=x_out, stop=stop, p0E=head["z"],
               z_out=self_condition(w, head["z"], act))
    return out


def generate_canvas_entropy(cfg, w, K_pre, V_pre, max_steps, seed, eps_accept, eps_stop):
    """Generate a batch of canvases with the entropy-bounded step and
    adaptive stopping, from uniform noise, on the time grid t_k = 1 - k /
    max_steps with Philox seed `seed + k` at step k (as the Step path).
    Returns x, z, the steps each canvas took and the per-step records."""
    B, C = K_pre.shape[0], cfg.C
    x = corrupt(np.zeros((B, C), np.int32), np.zeros(B, np.float32), seed, cfg.V)
    z = np.zeros((B, C, cfg.d))
    det_prev = None
    stopped = np.zeros(B, dtype=bool)
    steps = np.full(B, max_steps, dtype=np.int32)
    records = []
    for k in range(max_steps):
        act = np.nonzero(~stopped)[0]
        if act.size == 0:
            break
        t = np.full(act.size, np.float32(1.0 - k / max_steps), np.float32)
        dp = None if det_prev is None else det_prev[act]
        r = entropy_step(cfg, w, x[act], z[act], K_pre[act], V_pre[act], t, (seed + k) % (1 << 64),
                         eps_accept, eps_stop, det_prev=dp, canvas_ids=act)
        x[act] = r["x_out"]
        z[act] = r["z_out"]
        if det_prev is None:
            det_prev = np.zeros((B, C), dtype=np.int32)
        det_prev[act] = r["det"]
        newly = act[r["stop"]]
        stopped[newly] = True
        steps[newly] = k + 1
        records.append(dict(k=k, active=act, **{n: r[n] for n in
                                                ["H", "det", "det_gap", "det_top", "y", "gap", "top1",
                                                 "accept", "stop", "x_out"]}))
    return {"x": x, "z": z, "steps": steps, "records": records}
