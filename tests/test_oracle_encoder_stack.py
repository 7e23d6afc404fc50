"""Pins for the oracle's causal encoder pass of the decoder stack (CPU only):
explicit sums on a two-layer pass, causality, chunking invariance, the role
of the history rows, and the one-layer closed form."""
import math

import numpy as np

from oracle import causal_attention, embed, encode_kv_stack, rmsnorm
from oracle.stack import RMS_EPS
from workloads import get_config, make_inputs


def _setup(L=2, F=6, B=2, P=12, seed=0):
    cfg = get_config("c1", dtype="f64", n_layers=L, mlp_hidden=F, B=B, P=P, seed=seed)
    inp = make_inputs(cfg)
    sw = {n: [inp["S_" + n][l] for l in range(L)]
          for n in ["Wq", "Wk", "Wv", "Wo", "g_attn", "g_mlp", "W_gate", "W_up", "W_down"]}
    sw["g_final"] = inp["S_g_final"]
    return cfg, inp, sw


def _gelu(x):
    return 0.5 * x * (1 + math.tanh(math.sqrt(2 / math.pi) * (x + 0.044715 * x ** 3)))


def _norm(x, g):
    r = math.sqrt(sum(v * v for v in x) / len(x) + RMS_EPS)
    return [x[i] / r * float(g[i]) for i in range(len(x))]


def _mat(W, x):   # W [out, in] times vector x
    return [sum(float(W[o, i]) * x[i] for i in range(len(x))) for o in range(W.shape[0])]


def test_two_layer_pass_matches_explicit_sums():
    cfg, inp, sw = _setup()
    pos, n = 3, 4
    rng = np.random.default_rng(3)
    tokens = rng.integers(0, cfg.V, size=(cfg.B, n))
    K0 = inp["S_K_pre"].copy()
    V0 = inp["S_V_pre"].copy()
    r = encode_kv_stack(cfg, inp["E"], sw, tokens, K0, V0, pos)
    Hq, Hkv, hd, d = cfg.n_q_heads, cfg.n_kv_heads, cfg.head_dim, cfg.d
    G = Hq // Hkv
    for b in range(cfg.B):
        h = [[float(v) for v in inp["E"][tokens[b, i]]] for i in range(n)]
        for l in range(2):
            a = [_norm(h[i], sw["g_attn"][l]) for i in range(n)]
            k = [_mat(sw["Wk"][l], a[i]) for i in range(n)]
            v = [_mat(sw["Wv"][l], a[i]) for i in range(n)]
            for i in range(n):
                for g in range(Hkv):
                    for e in range(hd):
                        assert abs(r["K"][l, b, g, pos + i, e] - k[i][g * hd + e]) < 1e-10
                        assert abs(r["V"][l, b, g, pos + i, e] - v[i][g * hd + e]) < 1e-10
            if l == 1:
                break
            q = [_mat(sw["Wq"][l], a[i]) for i in range(n)]
            newh = []
            for i in range(n):
                o = [0.0] * (Hq * hd)
                for hh in range(Hq):
                    g = hh // G
                    # visible keys: history rows 0..pos-1, then new tokens 0..i
                    keys = [[float(x) for x in K0[l, b, g, j]] for j in range(pos)] + \
                           [k[j][g * hd:(g + 1) * hd] for j in range(i + 1)]
                    vals = [[float(x) for x in V0[l, b, g, j]] for j in range(pos)] + \
                           [v[j][g * hd:(g + 1) * hd] for j in range(i + 1)]
                    sc = [sum(q[i][hh * hd + e] * kk[e] for e in range(hd)) / math.sqrt(hd) for kk in keys]
                    mx = max(sc)
                    w = [math.exp(s - mx) for s in sc]
                    tot = sum(w)
                    for e in range(hd):
                        o[hh * hd + e] = sum(w[j] / tot * vals[j][e] for j in range(len(keys)))
                h1 = [h[i][c] + sum(float(sw["Wo"][l][c, j]) * o[j] for j in range(Hq * hd)) for c in range(d)]
                mm = _norm(h1, sw["g_mlp"][l])
                gg = _mat(sw["W_gate"][l], mm)
                uu = _mat(sw["W_up"][l], mm)
                hid = [_gelu(gg[f]) * uu[f] for f in range(len(gg))]
                newh.append([h1[c] + sum(float(sw["W_down"][l][c, f]) * hid[f] for f in range(len(hid)))
                             for c in range(d)])
            h = newh


def test_causality_and_untouched_rows():
    cfg, inp, sw = _setup()
    pos, n = 2, 5
    tokens = np.random.default_rng(4).integers(0, cfg.V, size=(cfg.B, n))
    r = encode_kv_stack(cfg, inp["E"], sw, tokens, inp["S_K_pre"], inp["S_V_pre"], pos)
    # rows outside [pos, pos + n) keep their values
    for X, X0 in ((r["K"], inp["S_K_pre"]), (r["V"], inp["S_V_pre"])):
        assert np.array_equal(X[:, :, :, :pos], X0[:, :, :, :pos])
        assert np.array_equal(X[:, :, :, pos + n:], X0[:, :, :, pos + n:])
    j = 3
    t2 = tokens.copy()
    t2[:, j] = (t2[:, j] + 1) % cfg.V
    r2 = encode_kv_stack(cfg, inp["E"], sw, t2, inp["S_K_pre"], inp["S_V_pre"], pos)
    for l in range(2):
        # tokens before j do not see token j
        assert np.array_equal(r["k"][l][:, :, :j], r2["k"][l][:, :, :j])
        assert np.array_equal(r["v"][l][:, :, :j], r2["v"][l][:, :, :j])
        assert not np.allclose(r["k"][l][:, :, j], r2["k"][l][:, :, j])
    # layer 0 entries are per token; layer 1 entries of later tokens see token j
    assert np.array_equal(r["k"][0][:, :, j + 1:], r2["k"][0][:, :, j + 1:])
    assert not np.allclose(r["k"][1][:, :, j + 1:], r2["k"][1][:, :, j + 1:])


def test_chunked_encoding_equals_one_pass():
    """Encoding n tokens at once equals encoding a first chunk and then the rest
    at the next rows: the second chunk sees the first as history."""
    cfg, inp, sw = _setup(L=3, P=16)
    pos, n, n1 = 4, 7, 3
    tokens = np.random.default_rng(5).integers(0, cfg.V, size=(cfg.B, n))
    one = encode_kv_stack(cfg, inp["E"], sw, tokens, inp["S_K_pre"], inp["S_V_pre"], pos)
    a = encode_kv_stack(cfg, inp["E"], sw, tokens[:, :n1], inp["S_K_pre"], inp["S_V_pre"], pos)
    b = encode_kv_stack(cfg, inp["E"], sw, tokens[:, n1:], a["K"], a["V"], pos + n1)
    assert np.allclose(b["K"], one["K"], rtol=1e-12, atol=1e-12)
    assert np.allclose(b["V"], one["V"], rtol=1e-12, atol=1e-12)


def test_history_rows_shape_the_deeper_entries():
    cfg, inp, sw = _setup()
    pos, n = 6, 3
    tokens = np.random.default_rng(6).integers(0, cfg.V, size=(cfg.B, n))
    r = encode_kv_stack(cfg, inp["E"], sw, tokens, inp["S_K_pre"], inp["S_V_pre"], pos)
    K2 = inp["S_K_pre"].copy()
    K2[:, :, :, :pos] *= -1.0
    r2 = encode_kv_stack(cfg, inp["E"], sw, tokens, K2, inp["S_V_pre"], pos)
    assert np.array_equal(r["k"][0], r2["k"][0])          # layer 0: no attention before it
    assert not np.allclose(r["k"][1], r2["k"][1])         # layer 1: after attending to the history


def test_one_layer_entries_closed_form():
    cfg, inp, sw = _setup(L=1)
    pos, n = 5, 4
    tokens = np.random.default_rng(7).integers(0, cfg.V, size=(cfg.B, n))
    r = encode_kv_stack(cfg, inp["E"], sw, tokens, inp["S_K_pre"], inp["S_V_pre"], pos)
    a = rmsnorm(embed(inp["E"], tokens, np.zeros((cfg.B, n, cfg.d)), "f64"), sw["g_attn"][0], "f64")
    k = (a.reshape(-1, cfg.d) @ sw["Wk"][0].T).reshape(cfg.B, n, cfg.n_kv_heads, cfg.head_dim)
    assert np.allclose(r["k"][0], k.transpose(0, 2, 1, 3), rtol=1e-12, atol=1e-13)


def test_causal_attention_special_cases():
    rng = np.random.default_rng(8)
    B, n, Hq, Hkv, hd = 1, 3, 2, 1, 4
    q = rng.standard_normal((B, n, Hq, hd))
    k = rng.standard_normal((B, Hkv, n, hd))
    v = rng.standard_normal((B, Hkv, n, hd))
    empty = np.zeros((B, Hkv, 0, hd))
    o = causal_attention(q, k, v, empty, empty, "f64")
    # the first new token with no history sees only itself
    assert np.allclose(o[0, 0, 0], v[0, 0, 0]) and np.allclose(o[0, 0, 1], v[0, 0, 0])
    # with equal scores (q = 0) token i averages history and tokens 0..i
    Kh = rng.standard_normal((B, Hkv, 2, hd))
    Vh = rng.standard_normal((B, Hkv, 2, hd))
    o = causal_attention(np.zeros_like(q), k, v, Kh, Vh, "f64")
    for i in range(n):
        want = np.concatenate([Vh[0, 0], v[0, 0, :i + 1]]).mean(axis=0)
        assert np.allclose(o[0, i, 0], want, atol=1e-14)
