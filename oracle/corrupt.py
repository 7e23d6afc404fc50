"""Forward corruption along the uniform-noise mixture path.

TR summary, Method, forward path equation: each coordinate independently
keeps x0 with probability kappa_t and is otherwise replaced by a token drawn
uniformly from the vocabulary (so the replacement may equal x0 itself, as
the (1 - kappa_t)/V term on every token implies). Per token (b, i), the
Philox block (i >> 1, 0, b, 2) gives the keep draw in word 2*(i&1) and the
replacement in word 2*(i&1)+1; keep iff U(word) < kappa_b (float32), and
the replacement is floor(word * V / 2^32).
"""
import numpy as np
from .philox import philox4x32_10, uniform01, mulhi_token


def corrupt(x0, kappa, seed, V, canvas_ids=None):
    x0 = np.asarray(x0)
    B, C = x0.shape
    cid = np.arange(B) if canvas_ids is None else np.asarray(canvas_ids)
    b = cid.astype(np.uint64)[:, None]
    i = np.arange(C, dtype=np.uint64)[None, :]
    w = philox4x32_10(i >> np.uint64(1), 0, b, 2, seed)
    w = np.stack(w, axis=-1)                                   # [B, C, 4]
    odd = (np.arange(C) & 1)[None, :]
    w_keep = np.where(odd == 1, w[..., 2], w[..., 0])
    w_tok = np.where(odd == 1, w[..., 3], w[..., 1])
    keep = uniform01(w_keep) < np.asarray(kappa, dtype=np.float32)[:, None]
    return np.where(keep, x0.astype(np.int64), mulhi_token(w_tok, V)).astype(np.int32)
