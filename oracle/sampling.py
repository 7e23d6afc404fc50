"""Step sampling: Bernoulli(lambda) then Gumbel-max over p0.

TR summary, Method, three-line update: x_{t-dt} ~ Step(x_t, p0), all
positions in parallel. With Step = (1 - lambda) delta(., x_t) + lambda p0
(our derivation), a draw is: keep x_t with probability 1 - lambda, else a
draw from p0 = softmax(s). The p0 draw uses the Gumbel-max identity
(argmax_v s_v + G_v with G_v = -log(-log U_v) is distributed as softmax(s));
exact ties go to the lowest vocab id. The Bernoulli uses u < lambda with u
from stream 1; the Gumbel noise uses stream 0 (counter map in philox.py).
Both decisions are taken in float32.
"""
import numpy as np
from .philox import philox4x32_10, uniform01


def bernoulli_uniforms(seed, canvas_ids, C, positions=None):
    """u[b, i] in (0, 1), float32, for canvases `canvas_ids` and positions 0..C-1
    (or the canvas positions listed in `positions`)."""
    b = np.asarray(canvas_ids, dtype=np.uint64)[:, None]
    pos = np.arange(C) if positions is None else np.asarray(positions)
    i = pos.astype(np.uint64)[None, :]
    w0, _, _, _ = philox4x32_10(0, i, b, 1, seed)
    return uniform01(w0)


def gumbel_block(v):
    """(counter word 0, word index) of vocab id v in the Gumbel stream."""
    v = np.asarray(v, dtype=np.uint64)
    return ((v >> np.uint64(6)) << np.uint64(4)) | (v & np.uint64(15)), (v >> np.uint64(4)) & np.uint64(3)


def gumbel_noise(seed, b, i, V):
    """G[n, v] = -log(-log U) in float32 for rows (b[n], i[n]) and all v < V."""
    b = np.asarray(b, dtype=np.uint64)[:, None]
    i = np.asarray(i, dtype=np.uint64)[:, None]
    c0, word = gumbel_block(np.arange(V))
    words = philox4x32_10(c0[None, :], i, b, 0, seed)       # 4 x [N, V]
    w = np.choose(word.astype(np.int64)[None, :], words)    # word (v >> 4) & 3 of v's block
    u = uniform01(w)
    e1 = np.log(u)                      # float32, < 0
    e2 = np.log(-e1)                    # float32
    return (-e2).astype(np.float32)


def step_select(x_t, s, lam, seed, canvas_ids, positions=None):
    """One Step draw for every row.

    x_t [B, C] int, s [B*C, V] scaled logits (float64), lam [B] float32;
    `positions` gives the canvas positions of the C columns when they are a
    subset of a canvas (default 0..C-1).
    Returns x_out, the per-row resample mask, the Gumbel argmax (or -1) and,
    for resampled rows, the top-1 perturbed value and the gap to the top-2
    value (for near-tie accounting).
    """
    B, C = x_t.shape
    V = s.shape[1]
    pos = np.arange(C) if positions is None else np.asarray(positions)
    u = bernoulli_uniforms(seed, canvas_ids, C, pos)                   # [B, C]
    resample = u < np.asarray(lam, dtype=np.float32)[:, None]
    x_out = np.array(x_t, dtype=np.int64, copy=True)
    best = np.full((B, C), -1, dtype=np.int64)
    top1 = np.full((B, C), np.nan, dtype=np.float32)
    gap = np.full((B, C), np.inf, dtype=np.float32)
    rb, ri = np.nonzero(resample)
    if rb.size:
        cid = np.asarray(canvas_ids)[rb]
        g = gumbel_noise(seed, cid, pos[ri], V)
        pert = s.reshape(B, C, V)[rb, ri].astype(np.float32) + g        # float32 add
        y = np.argmax(pert, axis=1)                                       # first max = lowest id
        best[rb, ri] = y
        x_out[rb, ri] = y
        srt = np.sort(pert, axis=1)
        top1[rb, ri] = srt[:, -1]
        gap[rb, ri] = srt[:, -1] - (srt[:, -2] if V > 1 else -np.inf)
    return {"x_out": x_out.astype(np.int32), "u": u, "resample": resample, "best": best,
            "top1": top1, "gap": gap}
