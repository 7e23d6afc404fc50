"""GPU parity of one denoising step at the full workload sizes, in the launch
configuration the benchmark times. The standard and long-prefix canvases are
checked on every row (p0 included); the large-vocabulary and batched workloads compute
every decoder stage on the oracle for all rows of the sampled canvases and
the LM head, z and the Step draw on sampled rows (rows are independent)."""
import numpy as np
import pytest

from oracle import attention, embed, inv_temperature, lm_head, out_proj, qkv_proj, step_lambda
from oracle.sampling import step_select
from tests.dg_harness import (LSE_RTOL, P0_ATOL, RTOL_BF16, GpuModel, assert_close, to_dev,
                              token_gate)
from workloads import get_config, make_inputs

pytestmark = pytest.mark.gpu


def _gpu_step(cfg, inp, t, seed, p0):
    import torch
    m = GpuModel(cfg, inp)
    x = torch.from_numpy(inp["x"]).cuda()
    dev = {n: to_dev(inp, n, cfg) for n in ["z", "K_pre", "V_pre"]}
    print(f"[gpu] full step {cfg.name} t={t[:2]} seed={seed}", flush=True)
    g = m.step(x, dev["z"], dev["K_pre"], dev["V_pre"], t, float(np.float32(1.0 / cfg.steps)),
               seed, taps=True, p0=p0)
    m.close()
    del dev, x
    torch.cuda.empty_cache()
    return g


def _oracle(cfg, inp, t, seed, canvases, rows, want_p0):
    """Oracle stages for canvases `canvases` (all rows) and the LM head / Step on `rows`."""
    act = cfg.dtype
    w = inp
    x = inp["x"][canvases]
    h0 = embed(w["E"], x, inp["z"][canvases], act)
    q, k, v = qkv_proj(h0, w["Wq"], w["Wk"], w["Wv"], cfg.n_q_heads, cfg.n_kv_heads, cfg.head_dim, act)
    o = attention(q, k, v, inp["K_pre"][canvases], inp["V_pre"][canvases], act)
    h1 = out_proj(o, w["Wo"], h0, act)
    tb = np.asarray(t, np.float32)[canvases]
    dt = float(np.float32(1.0 / cfg.steps))
    lam = np.array([step_lambda(float(a), dt, cfg.schedule) for a in tb], np.float32)
    inv_tau = np.array([inv_temperature(float(a)) for a in tb], np.float32)
    head = lm_head(h1[:, rows], w["E"], inv_tau, act, want_p0=want_p0)
    smp = step_select(x[:, rows], head["s"], lam, seed, canvases, positions=rows)
    return dict(h0=h0, q=q, k=k, v=v, o=o, h1=h1, **head, **smp)


def _compare(cfg, g, o, canvases, rows):
    sel = np.ix_(canvases, rows)
    for name in ["h0", "q", "o", "h1"]:
        assert_close(name, g[name][canvases], o[name], RTOL_BF16)
    for name in ["k", "v"]:
        assert_close(name, g[name][canvases], o[name], RTOL_BF16)
    assert_close("z", g["z_out"][sel], o["z"], RTOL_BF16)
    assert_close("lse", g["lse"][sel].ravel(), o["lse"], LSE_RTOL)
    if "p0" in o and "p0" in g:
        p0g = g["p0"][sel].reshape(o["p0"].shape)
        assert np.abs(p0g - o["p0"]).max() <= P0_ATOL
        assert np.abs(p0g - o["p0"]).max() / o["p0"].max() <= 2e-2
    assert np.array_equal(g["best"][sel] >= 0, o["resample"])
    stats = token_gate(g["x_out"][sel], o)
    print(f"[gpu] tokens: {stats}", flush=True)


@pytest.mark.parametrize("tval", [1.0, 0.5, 1.0 / 12])
def test_standard_canvas_all_rows(tval):
    cfg = get_config("c2")
    inp = make_inputs(cfg)
    t = np.full(cfg.B, tval, np.float32)
    g = _gpu_step(cfg, inp, t, seed=21, p0=True)
    rows = np.arange(cfg.C)
    o = _oracle(cfg, inp, t, 21, np.arange(cfg.B), rows, want_p0=True)
    _compare(cfg, g, o, np.arange(cfg.B), rows)


def test_long_prefix_all_rows():
    cfg = get_config("c3")
    inp = make_inputs(cfg)
    t = np.full(cfg.B, 0.25, np.float32)
    g = _gpu_step(cfg, inp, t, seed=22, p0=True)
    rows = np.arange(cfg.C)
    o = _oracle(cfg, inp, t, 22, np.arange(cfg.B), rows, want_p0=True)
    _compare(cfg, g, o, np.arange(cfg.B), rows)


def test_large_vocabulary_sampled_rows():
    cfg = get_config("c4")
    inp = make_inputs(cfg)
    t = np.full(cfg.B, 1.0 / 12, np.float32)      # lambda = 1: every row draws from p0
    g = _gpu_step(cfg, inp, t, seed=23, p0=True)
    # 58 rows: every fifth row, plus both sides of the 16-, 32- and 128-row
    # block edges and the last two rows
    rows = np.unique(np.concatenate([np.arange(0, cfg.C, 5), [15, 16, 31, 32, 127, 128, 254, 255]]))
    o = _oracle(cfg, inp, t, 23, np.arange(cfg.B), rows, want_p0=True)
    _compare(cfg, g, o, np.arange(cfg.B), rows)


def test_batched_sampled_canvases_and_rows():
    cfg = get_config("c5")
    inp = make_inputs(cfg)
    t = inp["t"]
    g = _gpu_step(cfg, inp, t, seed=24, p0=False)
    nz = inp["z_nonzero"]
    # three canvases with z = 0 and three with z != 0 (the last one included)
    zc = np.flatnonzero(~nz)[:3]
    nzc = np.flatnonzero(nz)[:3]
    canvases = np.unique(np.concatenate([zc, nzc, [cfg.B - 1]]))
    rows = np.array([0, 5, 17, 31, 32, 63, 64, 77, 100, 127, 128, 150, 191, 200, 223, 255])
    o = _oracle(cfg, inp, t, 24, canvases, rows, want_p0=False)
    _compare(cfg, g, o, canvases, rows)
    # every canvas's kept rows carry their input tokens
    keep = g["best"] < 0
    assert np.array_equal(g["x_out"][keep], inp["x"][keep])
