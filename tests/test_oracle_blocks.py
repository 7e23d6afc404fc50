"""Pins for the oracle's prefill / commit / block-autoregressive loop (CPU
only): the cache entries against explicit sums, a one-canvas loop against
single-canvas generation, the placement and use of committed rows, and that a
canvas sees no cache row beyond its own prefix."""
import numpy as np

from oracle import encode_kv, generate_blocks, generate_canvas, qkv_proj, embed
from workloads import get_config, make_inputs


def _tiny(**kw):
    return get_config("c1", **kw)


def _w(inp):
    return {k: inp[k] for k in ["E", "Wq", "Wk", "Wv", "Wo"]}


def test_encode_kv_matches_explicit_sums():
    cfg = _tiny(dtype="f64", B=2, C=3)
    inp = make_inputs(cfg)
    w = _w(inp)
    tok = np.array([[5, 0, 63], [7, 7, 1]], np.int32)
    k, v = encode_kv(cfg, w, tok)
    assert k.shape == (2, cfg.n_kv_heads, 3, cfg.head_dim)
    for b in range(2):
        for g in range(cfg.n_kv_heads):
            for i in range(3):
                for e in range(cfg.head_dim):
                    row = g * cfg.head_dim + e
                    want_k = sum(float(w["E"][tok[b, i], c]) * float(w["Wk"][row, c]) for c in range(cfg.d))
                    want_v = sum(float(w["E"][tok[b, i], c]) * float(w["Wv"][row, c]) for c in range(cfg.d))
                    assert abs(k[b, g, i, e] - want_k) < 1e-12 and abs(v[b, g, i, e] - want_v) < 1e-12


def test_encode_kv_is_the_decoders_projection_without_self_conditioning():
    cfg = _tiny(B=2)
    inp = make_inputs(cfg)
    w = _w(inp)
    h0 = embed(w["E"], inp["x"], np.zeros((cfg.B, cfg.C, cfg.d)), cfg.dtype)
    _, k, v = qkv_proj(h0, w["Wq"], w["Wk"], w["Wv"], cfg.n_q_heads, cfg.n_kv_heads, cfg.head_dim, cfg.dtype)
    k2, v2 = encode_kv(cfg, w, inp["x"])
    assert np.array_equal(k, k2) and np.array_equal(v, v2)


def _cache(cfg, inp, P0, n):
    K = np.full((cfg.B, cfg.n_kv_heads, P0 + n * cfg.C, cfg.head_dim), np.nan)
    V = K.copy()
    K[:, :, :P0] = inp["K_pre"][:, :, :P0]
    V[:, :, :P0] = inp["V_pre"][:, :, :P0]
    return K, V


def test_one_canvas_loop_is_single_canvas_generation_plus_commit():
    cfg = _tiny(B=2)
    inp = make_inputs(cfg)
    w = _w(inp)
    K, V = _cache(cfg, inp, cfg.P, 1)
    r = generate_blocks(cfg, w, K, V, cfg.P, 1, 4, 9)
    g = generate_canvas(cfg, w, inp["K_pre"], inp["V_pre"], 4, 9)
    assert np.array_equal(r["x"][:, 0], g["x"])
    k, v = encode_kv(cfg, w, g["x"])
    assert np.array_equal(r["K"][:, :, cfg.P:], k) and np.array_equal(r["V"][:, :, cfg.P:], v)
    assert np.array_equal(r["K"][:, :, :cfg.P], inp["K_pre"])


def test_second_canvas_attends_to_prompt_then_first_canvas():
    cfg = _tiny(B=2)
    inp = make_inputs(cfg)
    w = _w(inp)
    steps, seed = 3, 4
    K, V = _cache(cfg, inp, cfg.P, 2)
    r = generate_blocks(cfg, w, K, V, cfg.P, 2, steps, seed)
    k1, v1 = encode_kv(cfg, w, r["x"][:, 0])
    Kp = np.concatenate([inp["K_pre"], k1], axis=2)
    Vp = np.concatenate([inp["V_pre"], v1], axis=2)
    g = generate_canvas(cfg, w, Kp, Vp, steps, seed + steps)
    assert np.array_equal(r["x"][:, 1], g["x"])
    # the first canvas's rows did change what the second canvas sees
    g0 = generate_canvas(cfg, w, inp["K_pre"], inp["V_pre"], steps, seed + steps)
    assert not np.array_equal(g0["x"], g["x"])


def test_canvas_sees_no_row_beyond_its_prefix():
    # two caches that differ only in rows not yet committed give the same
    # canvases and the same committed rows
    cfg = _tiny(B=1)
    inp = make_inputs(cfg)
    w = _w(inp)
    K, V = _cache(cfg, inp, 5, 3)
    rng = np.random.default_rng(0)
    Ka, Va, Kb, Vb = K.copy(), V.copy(), K.copy(), V.copy()
    for A in (Ka, Va):
        A[:, :, 5:] = 50.0 * rng.standard_normal(A[:, :, 5:].shape)
    for A in (Kb, Vb):
        A[:, :, 5:] = -50.0 * rng.standard_normal(A[:, :, 5:].shape)
    ra = generate_blocks(cfg, w, Ka, Va, 5, 3, 2, 11)
    rb = generate_blocks(cfg, w, Kb, Vb, 5, 3, 2, 11)
    assert np.array_equal(ra["x"], rb["x"])
    assert np.array_equal(ra["K"], rb["K"]) and np.array_equal(ra["V"], rb["V"])
