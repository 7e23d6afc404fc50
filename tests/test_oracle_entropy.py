"""Pins for the entropy-bounded step (CPU only): closed forms of the entropy,
the acceptance rule against direct enumeration, the re-noise distribution and
the stopping logic."""
import itertools

import numpy as np
import scipy.special
import scipy.stats

from oracle import accept_mask, entropy_step, generate_canvas_entropy, renoise_tokens, row_entropy
from oracle.philox import philox_scalar
from workloads import get_config, make_inputs


def test_entropy_closed_forms():
    V = 37
    assert abs(row_entropy(np.zeros((1, V)))[0] - np.log(V)) < 1e-12
    assert abs(row_entropy(np.full((1, V), 5.0))[0] - np.log(V)) < 1e-12       # shift invariant
    s = np.full((1, V), -1e4)
    s[0, 3] = 0.0
    assert row_entropy(s)[0] < 1e-12                                            # one-hot
    # two equally likely ids and the rest negligible: ln 2
    s = np.full((1, V), -1e4)
    s[0, [1, 9]] = 2.0
    assert abs(row_entropy(s)[0] - np.log(2.0)) < 1e-12
    # binary entropy of (q, 1 - q)
    q = 0.2
    s = np.array([[np.log(q), np.log(1 - q)]])
    assert abs(row_entropy(s)[0] - (-q * np.log(q) - (1 - q) * np.log(1 - q))) < 1e-12


def test_entropy_matches_library_on_random_logits():
    rng = np.random.default_rng(3)
    s = rng.normal(0, 3, size=(20, 50))
    ref = scipy.stats.entropy(scipy.special.softmax(s, axis=1), axis=1)
    assert np.abs(row_entropy(s) - ref).max() < 1e-12


def _accept_bruteforce(h, eps):
    """Largest k such that the k lowest-entropy positions (ties by position)
    sum below eps; at least 1. Enumerates candidate sets directly."""
    C = len(h)
    ranked = sorted(range(C), key=lambda i: (h[i], i))
    best = {ranked[0]}
    for k in range(1, C + 1):
        subset = set(ranked[:k])
        if sum(h[i] for i in subset) < eps:
            best = subset
    return best


def test_accept_rule_against_enumeration():
    rng = np.random.default_rng(5)
    for trial in range(200):
        C = int(rng.integers(1, 9))
        h = np.round(rng.uniform(0, 2, size=C), 1)            # rounding makes ties common
        eps = float(rng.uniform(0, 6))
        m = accept_mask(h[None, :], eps)[0]
        assert set(np.nonzero(m)[0]) == _accept_bruteforce(list(h), eps), (h, eps)


def test_accept_rule_special_cases():
    h = np.array([[0.5, 0.5, 0.5, 0.5]])
    assert accept_mask(h, 1.0).sum() == 1          # 0.5 < 1 but 1.0 is not < 1
    assert accept_mask(h, 1.01).sum() == 2
    assert accept_mask(h, 100.0).sum() == 4
    m = accept_mask(h, 0.0)                        # nothing fits: the first position only
    assert m.sum() == 1 and m[0, 0]
    h = np.array([[2.0, 0.1, 3.0, 0.1]])
    assert list(np.nonzero(accept_mask(h, 0.25)[0])[0]) == [1, 3]
    assert list(np.nonzero(accept_mask(h, 0.15)[0])[0]) == [1]   # tie: lower position first


def test_renoise_tokens_uniform_and_defined_by_philox():
    V, C = 16, 20000
    tok = renoise_tokens(seed=9, canvas_ids=[0, 1], C=C, V=V)
    counts = np.bincount(tok.ravel(), minlength=V)
    assert scipy.stats.chisquare(counts).pvalue > 1e-3
    for b, i in [(0, 0), (1, 7), (1, 19999)]:
        w = philox_scalar((0, i, b, 3), (9, 0))[0]
        assert tok[b, i] == (w * V) >> 32


def _tiny():
    cfg = get_config("c1")
    inp = make_inputs(cfg)
    w = {k: inp[k] for k in ["E", "Wq", "Wk", "Wv", "Wo"]}
    return cfg, inp, w


def test_entropy_step_composition():
    cfg, inp, w = _tiny()
    t = np.full(cfg.B, 0.5, np.float32)
    r = entropy_step(cfg, w, inp["x"], inp["z"], inp["K_pre"], inp["V_pre"], t, seed=4,
                     eps_accept=3.0, eps_stop=10.0)
    assert np.array_equal(r["accept"], accept_mask(r["H"], 3.0))
    assert np.array_equal(r["x_out"], np.where(r["accept"], r["y"], r["renoise"]))
    assert np.array_equal(r["renoise"], renoise_tokens(4, [0], cfg.C, cfg.V))
    assert not r["stop"].any()                                  # first step never stops
    assert np.abs(r["H"].ravel() - row_entropy(r["s"])).max() == 0
    # stop needs both conditions
    r2 = entropy_step(cfg, w, inp["x"], inp["z"], inp["K_pre"], inp["V_pre"], t, seed=4,
                      eps_accept=3.0, eps_stop=10.0, det_prev=r["det"])
    assert r2["stop"].all()
    r3 = entropy_step(cfg, w, inp["x"], inp["z"], inp["K_pre"], inp["V_pre"], t, seed=4,
                      eps_accept=3.0, eps_stop=1e-6, det_prev=r["det"])
    assert not r3["stop"].any()
    other = (r["det"] + 1) % cfg.V
    r4 = entropy_step(cfg, w, inp["x"], inp["z"], inp["K_pre"], inp["V_pre"], t, seed=4,
                      eps_accept=3.0, eps_stop=10.0, det_prev=other)
    assert not r4["stop"].any()


def test_generation_freezes_stopped_canvases():
    cfg, inp, w = _tiny()
    K = np.repeat(inp["K_pre"], 3, axis=0)
    V_ = np.repeat(inp["V_pre"], 3, axis=0)
    cfg3 = get_config("c1", B=3)
    # loose stop threshold: a canvas stops as soon as its argmax predictions repeat
    g = generate_canvas_entropy(cfg3, w, K, V_, max_steps=8, seed=2, eps_accept=5.0, eps_stop=100.0)
    for b in range(3):
        k_stop = g["steps"][b]
        recs = [r for r in g["records"] if b in r["active"]]
        assert len(recs) == k_stop                       # active exactly until it stopped
        if k_stop < 8:
            last = recs[-1]
            j = list(last["active"]).index(b)
            assert last["stop"][j]
            prev = recs[-2]
            jp = list(prev["active"]).index(b)
            assert np.array_equal(last["det"][j], prev["det"][jp])
