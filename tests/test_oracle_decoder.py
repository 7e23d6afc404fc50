"""Pins for the oracle's decoder stand-in (CPU only): brute force, special
cases and library routines."""
import math

import numpy as np
import pytest
import scipy.special
import torch

from oracle import attention, embed, lm_head, out_proj, qkv_proj, round_bf16


def _brute_attention(q, k, v, K_pre, V_pre):
    """Triple loop over (b, h, i) with explicit sums; head h reads kv head h // G."""
    B, C, Hq, hd = q.shape
    Hkv = k.shape[1]
    G = Hq // Hkv
    P = K_pre.shape[2]
    o = np.zeros((B, C, Hq, hd))
    for b in range(B):
        for h in range(Hq):
            g = h // G
            for i in range(C):
                scores = []
                for j in range(P + C):
                    key = K_pre[b, g, j] if j < P else k[b, g, j - P]
                    scores.append(sum(float(q[b, i, h, e]) * float(key[e]) for e in range(hd)) / math.sqrt(hd))
                mx = max(scores)
                ws = [math.exp(s - mx) for s in scores]
                tot = sum(ws)
                for e in range(hd):
                    acc = 0.0
                    for j in range(P + C):
                        val = V_pre[b, g, j] if j < P else v[b, g, j - P]
                        acc += ws[j] / tot * float(val[e])
                    o[b, i, h, e] = acc
    return o


def test_attention_matches_brute_force():
    rng = np.random.default_rng(1)
    B, C, P, Hq, Hkv, hd = 2, 3, 4, 4, 2, 5
    q = rng.standard_normal((B, C, Hq, hd))
    k = rng.standard_normal((B, Hkv, C, hd))
    v = rng.standard_normal((B, Hkv, C, hd))
    Kp = rng.standard_normal((B, Hkv, P, hd))
    Vp = rng.standard_normal((B, Hkv, P, hd))
    got = attention(q, k, v, Kp, Vp, "f64")
    want = _brute_attention(q, k, v, Kp, Vp)
    assert np.abs(got - want).max() < 1e-12


def test_attention_single_key_returns_its_value():
    rng = np.random.default_rng(2)
    q = rng.standard_normal((1, 1, 2, 4))
    k = rng.standard_normal((1, 2, 1, 4))
    v = rng.standard_normal((1, 2, 1, 4))
    Kp = np.zeros((1, 2, 0, 4))
    got = attention(q, k, v, Kp, Kp, "f64")
    assert np.allclose(got[0, 0, 0], v[0, 0, 0], atol=1e-15)
    assert np.allclose(got[0, 0, 1], v[0, 1, 0], atol=1e-15)


def test_attention_equal_scores_average_values():
    rng = np.random.default_rng(3)
    q = np.zeros((1, 3, 2, 4))                 # all scores zero
    k = rng.standard_normal((1, 1, 3, 4))
    v = rng.standard_normal((1, 1, 3, 4))
    Kp = rng.standard_normal((1, 1, 5, 4))
    Vp = rng.standard_normal((1, 1, 5, 4))
    got = attention(q, k, v, Kp, Vp, "f64")
    mean = np.concatenate([Vp[0, 0], v[0, 0]]).mean(axis=0)
    assert np.allclose(got, mean, atol=1e-14)


def test_gqa_head_to_kv_head_map():
    """Query heads 0..G-1 read kv head 0, heads G..2G-1 read kv head 1 (h // G, not h % Hkv)."""
    B, C, P, Hq, Hkv, hd = 1, 2, 3, 4, 2, 2
    q = np.random.default_rng(4).standard_normal((B, C, Hq, hd))
    k = np.zeros((B, Hkv, C, hd)); Kp = np.zeros((B, Hkv, P, hd))
    v = np.zeros((B, Hkv, C, hd)); Vp = np.zeros((B, Hkv, P, hd))
    v[:, 0] = 1.0; Vp[:, 0] = 1.0
    v[:, 1] = -1.0; Vp[:, 1] = -1.0
    o = attention(q, k, v, Kp, Vp, "f64")
    assert np.allclose(o[:, :, :2], 1.0) and np.allclose(o[:, :, 2:], -1.0)


def test_lm_head_softmax_against_library_routines():
    rng = np.random.default_rng(5)
    B, C, d, V = 2, 3, 6, 11
    h1 = rng.standard_normal((B, C, d))
    E = rng.standard_normal((V, d))
    inv_tau = np.array([1.25, 2.0], dtype=np.float32)
    r = lm_head(h1, E, inv_tau, "f64", want_p0=True)
    s = (h1.reshape(-1, d) @ E.T) * np.repeat(inv_tau.astype(np.float64), C)[:, None]
    assert np.allclose(r["s"], s, atol=1e-13)
    assert np.allclose(r["p0"], scipy.special.softmax(s, axis=1), atol=1e-15)
    assert np.allclose(r["lse"], scipy.special.logsumexp(s, axis=1), atol=1e-13)
    assert np.all(r["p0"] >= 0) and np.allclose(r["p0"].sum(axis=1), 1.0, atol=1e-12)


def test_lm_head_row_shift_moves_lse_not_p0():
    """Adding a row constant c to the scaled logits leaves p0 unchanged and moves
    lse by exactly c. The shift is made through the inputs: an extra column of
    h1 that meets a column of ones appended to E adds h_extra * inv_tau to every
    logit of that row."""
    rng = np.random.default_rng(15)
    B, C, d, V = 2, 3, 6, 11
    h1 = rng.standard_normal((B, C, d))
    E = rng.standard_normal((V, d))
    inv_tau = np.array([1.25, 2.0], dtype=np.float32)
    base = lm_head(h1, E, inv_tau, "f64", want_p0=True)
    shift = rng.uniform(-3.0, 3.0, size=(B, C))
    h1s = np.concatenate([h1, shift[:, :, None]], axis=2)
    Es = np.concatenate([E, np.ones((V, 1))], axis=1)
    r = lm_head(h1s, Es, inv_tau, "f64", want_p0=True)
    c = (shift * inv_tau.astype(np.float64)[:, None]).reshape(-1)
    assert np.allclose(r["s"], base["s"] + c[:, None], atol=1e-12)
    assert np.allclose(r["p0"], base["p0"], atol=1e-14)
    assert np.allclose(r["lse"], base["lse"] + c, atol=1e-12)
    # a slip that dropped the max subtraction or the log would move p0 or
    # break lse - c; a slip that applied tau per row instead of per canvas
    # would break the per-canvas shift above
    assert not np.allclose(r["lse"], base["lse"])


def test_z_special_cases():
    V, d = 5, 4
    E = np.random.default_rng(6).standard_normal((V, d))
    # near one-hot p0 (huge logit on token 2) -> z = E[2]
    h1 = (1e4 * E[2] / np.dot(E[2], E[2]))[None, None, :]
    r = lm_head(h1, E, np.array([1.0], np.float32), "f64", want_p0=True)
    assert np.argmax(r["p0"][0]) == 2
    assert np.allclose(r["z"][0, 0], E[2], atol=1e-10)
    # uniform p0 (zero logits) -> z = mean of the rows of E
    r = lm_head(np.zeros((1, 1, d)), E, np.array([1.0], np.float32), "f64", want_p0=True)
    assert np.allclose(r["p0"], 1.0 / V)
    assert np.allclose(r["z"][0, 0], E.mean(axis=0), atol=1e-15)


def test_decoder_composition_closed_form():
    """With Wv = 0 the block is the identity (residual), so the tied head scores
    x_t against the embedding table: p0 and z have closed forms."""
    V = d = 6
    alpha = 1.5
    E = alpha * np.eye(V)
    x = np.array([[3, 0]])
    z = np.zeros((1, 2, d))
    h0 = embed(E, x, z, "f64")
    Wq = np.ones((4, d)); Wk = np.ones((4, d)); Wv = np.zeros((4, d))
    q, k, v = qkv_proj(h0, Wq, Wk, Wv, 2, 2, 2, "f64")
    Kp = np.ones((1, 2, 3, 2)); Vp = np.zeros((1, 2, 3, 2))
    o = attention(q, k, v, Kp, Vp, "f64")
    assert np.all(o == 0)
    h1 = out_proj(o, np.ones((d, 4)), h0, "f64")
    assert np.array_equal(h1, h0)
    inv_tau = np.float32(1 / 0.6)
    r = lm_head(h1, E, np.array([inv_tau]), "f64", want_p0=True)
    a = alpha * alpha * float(inv_tau)
    p_hit = math.exp(a) / (math.exp(a) + V - 1)
    for row, tok in enumerate(x[0]):
        want_p = np.full(V, (1 - p_hit) / (V - 1)); want_p[tok] = p_hit
        assert np.allclose(r["p0"][row], want_p, atol=1e-14)
        assert np.allclose(r["z"][0, row], alpha * want_p, atol=1e-14)
        assert r["lse"][row] == pytest.approx(math.log(math.exp(a) + V - 1), rel=1e-14)


def test_bf16_rounding_matches_torch_and_ties_to_even():
    rng = np.random.default_rng(8)
    a = (rng.standard_normal(100000) * np.exp(rng.uniform(-20, 20, 100000))).astype(np.float32)
    want = torch.from_numpy(a).to(torch.bfloat16).to(torch.float64).numpy()
    assert np.array_equal(round_bf16(a.astype(np.float64)), want)
    one = 1.0
    assert round_bf16(one + 2 ** -8) == 1.0                  # tie -> even
    assert round_bf16(one + 3 * 2 ** -8) == one + 2 ** -6    # tie -> even (upwards)
    assert round_bf16(-(one + 2 ** -8 + 2 ** -20)) == -(one + 2 ** -7)
    assert round_bf16(0.0) == 0.0


def test_embed_adds_self_conditioning_explicit_sum():
    """h0[b, i, :] = E[x[b, i], :] + z[b, i, :], element by element, with z != 0
    (TR summary, Method, decoder equation: z_t is a decoder input)."""
    rng = np.random.default_rng(16)
    B, C, d, V = 2, 5, 7, 9
    E = rng.standard_normal((V, d))
    x = rng.integers(0, V, size=(B, C))
    z = rng.standard_normal((B, C, d))
    h0 = embed(E, x, z, "f64")
    for b in range(B):
        for i in range(C):
            for e in range(d):
                assert h0[b, i, e] == E[x[b, i], e] + z[b, i, e]
    # the z term matters: zeroing it changes every entry
    assert np.all(embed(E, x, np.zeros_like(z), "f64") != h0)


def test_embed_rounds_the_sum_once_in_bf16():
    """bf16 workloads round E[x] + z once (not E[x] and z separately)."""
    E = np.array([[1.0, 0.0], [0.0, 1.0]])
    z = np.array([[[2 ** -9, 0.0], [0.0, 2 ** -9 + 2 ** -20]]])
    h0 = embed(E, np.array([[0, 1]]), z, "bf16")
    # 1 + 2^-9 is below the bf16 half-ulp (2^-8): rounds to 1; a value just
    # above the tie rounds up to 1 + 2^-7 only when the sum is rounded once
    assert h0[0, 0, 0] == 1.0
    assert h0[0, 1, 1] == 1.0
    z2 = np.array([[[2 ** -8 + 2 ** -20, 0.0], [0.0, 0.0]]])
    h0b = embed(E, np.array([[0, 1]]), z2, "bf16")
    assert h0b[0, 0, 0] == 1.0 + 2 ** -7


def test_qkv_projection_explicit_sums_rectangular():
    """q = h0 Wq^T with Wq [Hq*hd, d] and k, v = h0 W^T written head-major,
    on a rectangular case (Hq*hd != d, Hkv*hd != d), so a product with W
    instead of W^T cannot even be formed the same way."""
    rng = np.random.default_rng(17)
    B, C, d, Hq, Hkv, hd = 2, 3, 5, 4, 2, 3
    h0 = rng.standard_normal((B, C, d))
    Wq = rng.standard_normal((Hq * hd, d))
    Wk = rng.standard_normal((Hkv * hd, d))
    Wv = rng.standard_normal((Hkv * hd, d))
    q, k, v = qkv_proj(h0, Wq, Wk, Wv, Hq, Hkv, hd, "f64")
    assert q.shape == (B, C, Hq, hd) and k.shape == (B, Hkv, C, hd) and v.shape == (B, Hkv, C, hd)
    for b in range(B):
        for i in range(C):
            for h in range(Hq):
                for e in range(hd):
                    want = sum(h0[b, i, c] * Wq[h * hd + e, c] for c in range(d))
                    assert abs(q[b, i, h, e] - want) < 1e-12
            for g in range(Hkv):
                for e in range(hd):
                    wk = sum(h0[b, i, c] * Wk[g * hd + e, c] for c in range(d))
                    wv = sum(h0[b, i, c] * Wv[g * hd + e, c] for c in range(d))
                    assert abs(k[b, g, i, e] - wk) < 1e-12
                    assert abs(v[b, g, i, e] - wv) < 1e-12


def test_out_projection_explicit_sums_rectangular():
    """h1[b, i, c] = h0[b, i, c] + sum_j o[b, i, j] Wo[c, j], with Wo [d, Hq*hd]
    rectangular (Hq*hd != d) and a non-zero o, so an o Wo (untransposed)
    slip or a dropped residual fails."""
    rng = np.random.default_rng(18)
    B, C, d, Hq, hd = 2, 3, 5, 2, 4          # Hq*hd = 8 != d = 5
    o = rng.standard_normal((B, C, Hq, hd))
    Wo = rng.standard_normal((d, Hq * hd))
    h0 = rng.standard_normal((B, C, d))
    h1 = out_proj(o, Wo, h0, "f64")
    assert h1.shape == (B, C, d)
    for b in range(B):
        for i in range(C):
            flat = o[b, i].reshape(-1)
            for c in range(d):
                want = h0[b, i, c] + sum(flat[j] * Wo[c, j] for j in range(Hq * hd))
                assert abs(h1[b, i, c] - want) < 1e-12


def test_out_projection_square_transpose_slip_detected():
    """The square case (d = Hq*hd, as in every configured workload): o Wo^T
    differs from o Wo for a non-symmetric Wo, and the oracle takes the former."""
    rng = np.random.default_rng(19)
    B, C, Hq, hd = 1, 2, 2, 3
    d = Hq * hd
    o = rng.standard_normal((B, C, Hq, hd))
    Wo = rng.standard_normal((d, d))
    h0 = np.zeros((B, C, d))
    h1 = out_proj(o, Wo, h0, "f64")
    flat = o.reshape(B * C, d)
    assert np.allclose(h1.reshape(B * C, d), np.einsum("rj,cj->rc", flat, Wo), atol=1e-13)
    assert not np.allclose(h1.reshape(B * C, d), flat @ Wo, atol=1e-3)
