"""Prompt prefill, canvas commit and block-autoregressive generation --
TEST INFRASTRUCTURE.

TR summary, Method: generation runs block by block; one canvas of C = 256
tokens is denoised at a time while the decoder cross-attends to the KV cache
H, and once it is clean it is committed to the sequence history and the next
canvas starts (block-autoregressive paragraph). The pipeline figure's three
stages: a causal encoder turns the prompt into the initial cache, the decoder
refines the noisy canvas against it, and the clean canvas goes back through
the causal encoder and is appended to the cache.

Readings taken here (the pages stop short):
  * the encoder shares the decoder stand-in's weights (the pages describe a
    weight-shared encoder-decoder); in a single attention block the cache
    entries of a token are its key and value projections,
        k = round(round(E[x]) Wk^T),  v = round(round(E[x]) Wv^T),
    with no self-conditioning input (z = 0); the causal mask of the encoder
    only shapes the block's output, which the cache does not keep. Prefill
    and commit are therefore the same operation applied to different tokens;
  * a committed canvas takes cache rows P0 + j C .. P0 + (j + 1) C - 1 in
    canvas order, right after the prompt's P0 rows and the earlier canvases;
  * canvas j is generated exactly like a single canvas with the seed
    seed + j * steps (its initial noise uses that seed and its step k the seed
    plus k), so the Philox keys of different canvases never coincide.
"""
import numpy as np

from .decoder import embed
from .rounding import round_act
from .step import generate_canvas


def encode_kv(cfg, w, tokens):
    """Cache entries of `tokens` [B, n]: k, v [B, Hkv, n, hd] (act-rounded)."""
    tokens = np.asarray(tokens)
    B, n = tokens.shape
    act = cfg.dtype
    h = embed(w["E"], tokens, np.zeros((B, n, cfg.d)), act).reshape(B * n, cfg.d)
    Hkv, hd = cfg.n_kv_heads, cfg.head_dim
    k = round_act(h @ np.asarray(w["Wk"], np.float64).T, act).reshape(B, n, Hkv, hd)
    v = round_act(h @ np.asarray(w["Wv"], np.float64).T, act).reshape(B, n, Hkv, hd)
    return k.transpose(0, 2, 1, 3).copy(), v.transpose(0, 2, 1, 3).copy()


def generate_blocks(cfg, w, K_cache, V_cache, P0, n_canvases, steps, seed):
    """Generate `n_canvases` canvases one after the other, each against the
    cache rows written so far, committing each clean canvas to the cache.

    K_cache, V_cache [B, Hkv, P_cap, hd] hold the prompt in rows [0, P0);
    P0 + n_canvases * C <= P_cap. Returns x [B, n_canvases, C] and the caches
    with the committed rows filled in (copies; the inputs are not modified).
    """
    C = cfg.C
    K = np.array(K_cache, dtype=np.float64, copy=True)
    V = np.array(V_cache, dtype=np.float64, copy=True)
    assert P0 + n_canvases * C <= K.shape[2]
    xs = []
    for j in range(n_canvases):
        Pj = P0 + j * C
        r = generate_canvas(cfg, w, K[:, :, :Pj], V[:, :, :Pj], steps, (seed + j * steps) % (1 << 64))
        x = r["x"]
        xs.append(x)
        k, v = encode_kv(cfg, w, x)
        K[:, :, Pj:Pj + C] = k
        V[:, :, Pj:Pj + C] = v
    return {"x": np.stack(xs, axis=1), "K": K, "V": V}
