"""Pins for the oracle's gated self-conditioning block (CPU only): the tanh
GELU against a library routine, an exact identity and the exact GELU; the
block against brute force and special cases that expose the roles and
orientation of its three matrices."""
import numpy as np
import scipy.special
import torch

from oracle import denoise_step, entropy_step, ffw, ffw_hidden, gelu_tanh, round_bf16
from workloads import get_config, make_inputs


def test_gelu_tanh_matches_torch_tanh_form():
    a = np.linspace(-12.0, 12.0, 4001)
    want = torch.nn.functional.gelu(torch.from_numpy(a), approximate="tanh").numpy()
    assert np.abs(gelu_tanh(a) - want).max() <= 1e-14 * max(1.0, np.abs(want).max())


def test_gelu_tanh_odd_part_is_identity():
    # a/2 (1 + tanh(c(a))) - (-a)/2 (1 + tanh(c(-a))) = a exactly, tanh being odd
    a = np.random.default_rng(3).standard_normal(1000) * 4
    assert np.abs(gelu_tanh(a) - gelu_tanh(-a) - a).max() < 1e-14 * 16


def test_gelu_tanh_is_close_to_exact_gelu():
    a = np.linspace(-10.0, 10.0, 20001)
    exact = a * scipy.special.ndtr(a)
    dev = np.abs(gelu_tanh(a) - exact)
    assert dev.max() < 5e-4          # the tanh form's known worst case is about 4.7e-4
    assert gelu_tanh(0.0) == 0.0
    big = np.array([8.0, 10.0, 20.0])
    assert np.abs(gelu_tanh(big) - big).max() < 1e-12
    assert np.abs(gelu_tanh(-big)).max() < 1e-12


def _brute_ffw(u, Wg, Wu, Wd):
    """Explicit sums from the definition: z_r = sum_f Wd[e, f] gelu(sum_c Wg[f, c] u_rc) (sum_c Wu[f, c] u_rc)."""
    R, d = u.shape
    F = Wg.shape[0]
    c = np.sqrt(2.0 / np.pi)
    z = np.zeros((R, Wd.shape[0]))
    for r in range(R):
        hid = []
        for f in range(F):
            g = sum(float(Wg[f, k]) * float(u[r, k]) for k in range(d))
            v = sum(float(Wu[f, k]) * float(u[r, k]) for k in range(d))
            hid.append(0.5 * g * (1.0 + np.tanh(c * (g + 0.044715 * g * g * g))) * v)
        for e in range(Wd.shape[0]):
            z[r, e] = sum(float(Wd[e, f]) * hid[f] for f in range(F))
    return z


def test_ffw_matches_brute_force():
    rng = np.random.default_rng(7)
    R, d, F = 3, 4, 5
    u = rng.standard_normal((R, d))
    Wg, Wu = rng.standard_normal((F, d)), rng.standard_normal((F, d))
    Wd = rng.standard_normal((d, F))
    got = ffw(u, Wg, Wu, Wd, "f64")
    assert got.shape == (R, d)
    assert np.abs(got - _brute_ffw(u, Wg, Wu, Wd)).max() < 1e-12


def test_ffw_special_cases():
    rng = np.random.default_rng(8)
    R, d = 4, 6
    u = rng.standard_normal((R, d))
    I = np.eye(d)
    # zero up-projection or zero input -> zero output
    assert not ffw(u, I, np.zeros((d, d)), I, "f64").any()
    assert not ffw(np.zeros((R, d)), I, I, I, "f64").any()
    # a steep gate acts as a switch: gelu(c u) ~ c u for u > 0 and ~ 0 below;
    # with up = I the output is c u^2 on positive entries only (a swapped
    # gate/up pair would give gelu(u) c u instead)
    c = 200.0
    got = ffw(u, c * I, I, I, "f64")
    want = np.where(u > 0, c * u * u, 0.0)
    assert np.abs(got - want).max() < 1e-6 * c
    # a permutation as W_down moves hidden unit f to output row perm[f]
    perm = rng.permutation(d)
    Wd = np.zeros((d, d))
    Wd[perm, np.arange(d)] = 1.0
    hid = ffw_hidden(u, I, I, "f64")
    got = ffw(u, I, I, Wd, "f64")
    assert np.array_equal(got[:, perm], hid)


def test_ffw_rounds_hidden_and_output_to_bf16():
    rng = np.random.default_rng(9)
    u = round_bf16(rng.standard_normal((5, 8)))
    Wg, Wu = round_bf16(rng.standard_normal((16, 8))), round_bf16(rng.standard_normal((16, 8)))
    Wd = round_bf16(rng.standard_normal((8, 16)))
    hid = ffw_hidden(u, Wg, Wu, "bf16")
    z = ffw(u, Wg, Wu, Wd, "bf16")
    assert np.array_equal(round_bf16(hid), hid) and np.array_equal(round_bf16(z), z)
    assert np.array_equal(z, round_bf16(hid @ Wd.T))


def test_step_applies_the_block_to_p0E_only():
    cfg = get_config("c1", ffw_hidden=48)
    inp = make_inputs(cfg)
    w = {k: inp[k] for k in ["E", "Wq", "Wk", "Wv", "Wo"]}
    wf = dict(w, W_gate=inp["W_gate"], W_up=inp["W_up"], W_down=inp["W_down"])
    t = np.full(cfg.B, 0.6, np.float32)
    a = denoise_step(cfg, w, inp["x"], inp["z"], inp["K_pre"], inp["V_pre"], t, 0.125, 5)
    b = denoise_step(cfg, wf, inp["x"], inp["z"], inp["K_pre"], inp["V_pre"], t, 0.125, 5)
    assert np.array_equal(a["x_out"], b["x_out"]) and np.array_equal(a["p0E"], b["p0E"])
    assert np.array_equal(a["z_out"], a["p0E"])
    assert np.array_equal(b["z_out"], ffw(b["p0E"], inp["W_gate"], inp["W_up"], inp["W_down"], "f32"))
    e = entropy_step(cfg, wf, inp["x"], inp["z"], inp["K_pre"], inp["V_pre"], t, 5, 1.0, 0.5)
    assert np.array_equal(e["z_out"], b["z_out"])
