"""Pins for the oracle's decoder stack (CPU only): RMSNorm against its
definition and invariances, one layer against explicit sums, the residual
structure (zero output projections leave the stream untouched), and a stack
of zero-output layers reducing to the embedding."""
import math

import numpy as np

from oracle import (attention, embed, lm_head, layer, out_proj, qkv_proj, rmsnorm, stack_step,
                    step_select)
from oracle.stack import RMS_EPS
from workloads import get_config, make_inputs


def test_rmsnorm_definition_and_invariances():
    rng = np.random.default_rng(1)
    x = rng.standard_normal((3, 5, 7))
    g = rng.standard_normal(7)
    y = rmsnorm(x, g, "f64")
    for i in range(3):
        for j in range(5):
            r = math.sqrt(sum(float(v) ** 2 for v in x[i, j]) / 7 + RMS_EPS)
            assert np.allclose(y[i, j], x[i, j] / r * g, rtol=1e-13, atol=0)
    # scale invariance (up to eps) and unit rms with unit gains
    assert np.allclose(rmsnorm(1e3 * x, g, "f64"), y, rtol=1e-5)
    u = rmsnorm(x, np.ones(7), "f64")
    assert np.allclose(np.sqrt((u * u).mean(axis=-1)), 1.0, rtol=1e-5)


def _stack_weights(inp, L):
    return {n: [inp["S_" + n][l] for l in range(L)]
            for n in ["Wq", "Wk", "Wv", "Wo", "g_attn", "g_mlp", "W_gate", "W_up", "W_down"]}


def test_layer_matches_explicit_composition_of_pinned_parts():
    cfg = get_config("c1", dtype="f64", n_layers=1, mlp_hidden=24, B=2)
    inp = make_inputs(cfg)
    lw = {n: v[0] for n, v in _stack_weights(inp, 1).items()}
    h = embed(inp["E"], inp["x"], inp["z"], "f64")
    out, parts = layer(cfg, lw, h, inp["S_K_pre"][0], inp["S_V_pre"][0])
    a = rmsnorm(h, lw["g_attn"], "f64")
    q, k, v = qkv_proj(a, lw["Wq"], lw["Wk"], lw["Wv"], cfg.n_q_heads, cfg.n_kv_heads, cfg.head_dim, "f64")
    o = attention(q, k, v, inp["S_K_pre"][0], inp["S_V_pre"][0], "f64")
    h1 = out_proj(o, lw["Wo"], h, "f64")
    assert np.allclose(parts["h_attn"], h1, rtol=1e-12, atol=1e-12)
    # the MLP by explicit sums on one row
    m = rmsnorm(h1, lw["g_mlp"], "f64")
    b, i = 1, 3
    c = math.sqrt(2 / math.pi)
    hid = []
    for f in range(cfg.mlp_hidden):
        gg = sum(float(lw["W_gate"][f, j]) * float(m[b, i, j]) for j in range(cfg.d))
        uu = sum(float(lw["W_up"][f, j]) * float(m[b, i, j]) for j in range(cfg.d))
        hid.append(0.5 * gg * (1 + math.tanh(c * (gg + 0.044715 * gg ** 3))) * uu)
    for e in range(cfg.d):
        want = float(h1[b, i, e]) + sum(float(lw["W_down"][e, f]) * hid[f] for f in range(cfg.mlp_hidden))
        assert abs(out[b, i, e] - want) < 1e-10


def test_zero_output_projections_keep_the_residual_stream():
    cfg = get_config("c1", n_layers=3, mlp_hidden=16)
    inp = make_inputs(cfg)
    sw = _stack_weights(inp, 3)
    sw["Wo"] = [np.zeros_like(W) for W in sw["Wo"]]
    sw["W_down"] = [np.zeros_like(W) for W in sw["W_down"]]
    sw["g_final"] = inp["S_g_final"]
    w = {"E": inp["E"]}
    t = np.full(cfg.B, 0.5, np.float32)
    r = stack_step(cfg, w, sw, inp["x"], inp["z"], inp["S_K_pre"], inp["S_V_pre"], t, 0.125, 3)
    h0 = embed(inp["E"], inp["x"], inp["z"], cfg.dtype)
    for parts in r["layers"]:
        assert np.array_equal(parts["h"], h0)
    hf = rmsnorm(h0, inp["S_g_final"], cfg.dtype)
    head = lm_head(hf, inp["E"], r["inv_tau"], cfg.dtype)
    assert np.array_equal(r["lse"], head["lse"]) and np.array_equal(r["z_out"], head["z"])
    smp = step_select(inp["x"], head["s"], r["lam"], 3, np.arange(cfg.B))
    assert np.array_equal(r["x_out"], smp["x_out"])


def test_layers_apply_in_order_with_their_own_caches():
    cfg = get_config("c1", n_layers=2, mlp_hidden=16)
    inp = make_inputs(cfg)
    sw = _stack_weights(inp, 2)
    sw["g_final"] = inp["S_g_final"]
    t = np.full(cfg.B, 0.5, np.float32)
    r = stack_step(cfg, {"E": inp["E"]}, sw, inp["x"], inp["z"], inp["S_K_pre"], inp["S_V_pre"], t, 0.125, 3)
    h = embed(inp["E"], inp["x"], inp["z"], cfg.dtype)
    for l in range(2):
        h, _ = layer(cfg, {n: v[l] for n, v in sw.items() if n != "g_final"}, h, inp["S_K_pre"][l], inp["S_V_pre"][l])
    assert np.array_equal(r["layers"][1]["h"], h)
    # swapping the layers' caches changes the result
    r2 = stack_step(cfg, {"E": inp["E"]}, sw, inp["x"], inp["z"], inp["S_K_pre"][::-1], inp["S_V_pre"][::-1],
                    t, 0.125, 3)
    assert not np.array_equal(r2["layers"][1]["h"], r["layers"][1]["h"])


def test_route_picks_top_k_with_ties_to_the_lower_expert():
    from oracle.stack import route
    W = np.eye(4)
    m = np.array([[0.5, 2.0, 2.0, -1.0],      # tie between experts 1 and 2
                  [3.0, 1.0, 2.0, 0.0]])
    sel, w, r = route(m, W, 2)
    assert sel.tolist() == [[1, 2], [0, 2]]
    assert np.allclose(w.sum(axis=1), 1.0)
    assert np.allclose(w[1], np.exp([3.0, 2.0]) / np.exp([3.0, 2.0]).sum())
    # brute force on random logits
    rng = np.random.default_rng(3)
    m = rng.standard_normal((50, 6))
    W = rng.standard_normal((8, 6))
    sel, w, r = route(m, W, 3)
    for i in range(50):
        want = sorted(range(8), key=lambda e: (-float(r[i, e]), e))[:3]
        assert sel[i].tolist() == want


def _expert_brute(x, Wg, Wu, Wd):
    c = math.sqrt(2 / math.pi)
    hid = []
    for f in range(Wg.shape[0]):
        g = float(np.dot(Wg[f], x))
        u = float(np.dot(Wu[f], x))
        hid.append(0.5 * g * (1 + math.tanh(c * (g + 0.044715 * g ** 3))) * u)
    return np.array([sum(float(Wd[e, f]) * hid[f] for f in range(len(hid))) for e in range(Wd.shape[0])])


def test_moe_mlp_against_brute_force_and_special_cases():
    from oracle.stack import moe_mlp, route
    rng = np.random.default_rng(4)
    R, d, F, X = 5, 6, 7, 4
    m = rng.standard_normal((R, d))
    Wr = rng.standard_normal((X, d))
    Wg, Wu = rng.standard_normal((X, F, d)), rng.standard_normal((X, F, d))
    Wd = rng.standard_normal((X, d, F))
    for k in (1, 2, X):
        got = moe_mlp(m, Wr, Wg, Wu, Wd, k, "f64")
        sel, w, r = route(m, Wr, k)
        for i in range(R):
            want = sum(w[i, j] * _expert_brute(m[i], Wg[sel[i, j]], Wu[sel[i, j]], Wd[sel[i, j]])
                       for j in range(k))
            assert np.allclose(got[i], want, rtol=1e-12, atol=1e-12)
    # one expert, top-1: the dense gated MLP
    one = moe_mlp(m, Wr[:1], Wg[:1], Wu[:1], Wd[:1], 1, "f64")
    from oracle import ffw
    assert np.allclose(one, ffw(m, Wg[0], Wu[0], Wd[0], "f64"), rtol=1e-12, atol=1e-12)
