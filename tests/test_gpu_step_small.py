"""GPU parity of one denoising step at sizes the oracle finishes in seconds,
stage by stage through the taps (fp32 and bf16 kernels, several tiles and
ragged tails in rows, keys and heads)."""
import numpy as np
import pytest

from oracle import denoise_step
from tests.dg_harness import (LSE_RTOL, P0_ATOL, RTOL_BF16, RTOL_F32, GpuModel, assert_close,
                              to_dev, token_gate)
from workloads import get_config, make_inputs

pytestmark = pytest.mark.gpu

SMALL = {
    # fp32 workload exactly as configured (C=16, P=8, d=32, MHA 2x16, V=64)
    "c1": dict(base="c1"),
    # bf16, ragged rows (C=40 vs 32-row LM-head blocks), ragged keys (P+C=140);
    # 64 vocabulary splits, more than the wide LM-head merge takes (32)
    "bf16-hd64": dict(base="c2", B=2, C=40, P=100, d=256, n_q_heads=4, n_kv_heads=2, head_dim=64,
                      V=4096),
    "bf16-hd128": dict(base="c2", B=1, C=72, P=130, d=512, n_q_heads=4, n_kv_heads=2,
                       head_dim=128, V=2048),
    # head_dim 176 and d = 2816 (the large-vocabulary model's widths), few rows
    "bf16-hd176": dict(base="c4", B=1, C=24, P=40, d=2816, n_q_heads=16, n_kv_heads=8,
                       head_dim=176, V=1024),
    "bf16-linear-b3": dict(base="c5", B=3, C=33, P=64, d=1024, n_q_heads=8, n_kv_heads=4,
                           head_dim=128, V=1024),
    # V = 1040 = 65 tiles of 16 ids: the last split holds one tile, a partial
    # group of four Gumbel tiles; zero prefix (P = 0: canvas keys only)
    "bf16-vocab-1040-p0": dict(base="c2", B=2, C=40, P=0, d=256, n_q_heads=4, n_kv_heads=2,
                               head_dim=64, V=1040),
    # few query rows against a long prefix: 63 key tiles in 32 splits of two,
    # more splits than the wide attention merge takes (16): the general merge
    "bf16-long-prefix-32-splits": dict(base="c3", B=1, C=8, P=4000, d=256, n_q_heads=4, n_kv_heads=2,
                                       head_dim=64, V=512),
    # four query heads per kv head (400 stacked query rows per head), three
    # ragged canvases: 17 vocabulary splits (the wide merge reading 15 surplus
    # loads) and 13 attention splits
    "bf16-gqa4-splits-17-13": dict(base="c2", B=3, C=100, P=1500, d=256, n_q_heads=4, n_kv_heads=1,
                                   head_dim=64, V=2064),
    # 25 vocabulary splits and 7 attention splits, two canvases
    "bf16-gqa4-splits-25-7": dict(base="c2", B=2, C=100, P=700, d=256, n_q_heads=4, n_kv_heads=1,
                                  head_dim=64, V=3136),
    # 33 vocabulary splits, one more than the wide LM-head merge takes (the
    # general merge), and 13 attention splits
    "bf16-gqa4-splits-33-13": dict(base="c2", B=1, C=40, P=1500, d=256, n_q_heads=4, n_kv_heads=1,
                                   head_dim=64, V=2064),
    # enough rows (2250 = 8 x 256 + 202) for the 256 x 256-tile projections,
    # with a ragged last row tile
    "bf16-many-rows": dict(base="c5", B=9, C=250, P=70, d=256, n_q_heads=4, n_kv_heads=4,
                           head_dim=64, V=4096),
    # enough query blocks for 8-wave attention blocks at head_dim 64 (144
    # blocks): the skewed schedule, in splits of two key tiles (the younger
    # waves' loop runs once) with a ragged last tile (500 keys)
    "bf16-hd64-8-wave-skew": dict(base="c2", B=9, C=200, P=300, d=256, n_q_heads=4, n_kv_heads=2,
                                  head_dim=64, V=1024),
}


def _cfg(name):
    spec = dict(SMALL[name])
    base = spec.pop("base")
    return get_config(base, **spec)


def _run(cfg, t, dt, seed, p0=True):
    import torch
    inp = make_inputs(cfg)
    m = GpuModel(cfg, inp)
    x = torch.from_numpy(inp["x"]).cuda()
    dev = {n: to_dev(inp, n, cfg) for n in ["z", "K_pre", "V_pre"]}
    print(f"[gpu] step {cfg.name} B={cfg.B} C={cfg.C} P={cfg.P} d={cfg.d} V={cfg.V} seed={seed}", flush=True)
    g = m.step(x, dev["z"], dev["K_pre"], dev["V_pre"], t, dt, seed, p0=p0)
    m.close()
    w = {k: inp[k] for k in ["E", "Wq", "Wk", "Wv", "Wo"]}
    o = denoise_step(cfg, w, inp["x"], inp["z"], inp["K_pre"], inp["V_pre"], t, float(dt), seed,
                     want_p0=p0)
    return g, o, inp


@pytest.mark.parametrize("name", list(SMALL))
@pytest.mark.parametrize("tval", [1.0, 0.5, 1.0 / 12])
def test_step_matches_oracle(name, tval):
    cfg = _cfg(name)
    dt = np.float32(1.0 / cfg.steps)
    t = np.full(cfg.B, tval, np.float32)
    if cfg.per_canvas_t:
        t = make_inputs(cfg, ["t"])["t"]
    g, o, _ = _run(cfg, t, dt, seed=11)
    rt = RTOL_F32 if cfg.dtype == "f32" else RTOL_BF16
    for name_ in ["h0", "q", "k", "v", "o", "h1"]:
        assert_close(name_, g[name_], o[name_], rt)
    assert_close("z", g["z_out"], o["z_out"], rt)
    assert_close("lse", g["lse"].ravel(), o["lse"], RTOL_F32 if cfg.dtype == "f32" else LSE_RTOL)
    p0g = g["p0"].reshape(o["p0"].shape)
    assert np.abs(p0g - o["p0"]).max() <= P0_ATOL
    assert np.abs(p0g - o["p0"]).max() / o["p0"].max() <= (1e-4 if cfg.dtype == "f32" else 2e-2)
    # the Bernoulli decisions are exact; the draw of resampled rows is gated
    assert np.array_equal(g["best"] >= 0, o["resample"])
    token_gate(g["x_out"], o)


def test_taps_do_not_change_results():
    import torch
    cfg = _cfg("bf16-hd64")
    inp = make_inputs(cfg)
    m = GpuModel(cfg, inp)
    x = torch.from_numpy(inp["x"]).cuda()
    dev = {n: to_dev(inp, n, cfg) for n in ["z", "K_pre", "V_pre"]}
    t = np.full(cfg.B, 0.3, np.float32)
    a = m.step(x, dev["z"], dev["K_pre"], dev["V_pre"], t, 1 / 12, 5, taps=True, p0=True)
    b = m.step(x, dev["z"], dev["K_pre"], dev["V_pre"], t, 1 / 12, 5, taps=False)
    c = m.step(x, dev["z"], dev["K_pre"], dev["V_pre"], t, 1 / 12, 5, taps=False)
    m.close()
    assert np.array_equal(a["x_out"], b["x_out"]) and np.array_equal(b["x_out"], c["x_out"])
    assert np.array_equal(a["z_out"], b["z_out"]) and np.array_equal(b["z_out"], c["z_out"])


def test_out_of_range_tokens_embed_as_zero_rows():
    # a guard, not part of the method: a token outside [0, V) contributes a
    # zero embedding row, so h0 of that position is z itself (rounded)
    import torch
    from tests.dg_harness import to_host
    cfg = _cfg("bf16-hd64")
    inp = make_inputs(cfg)
    m = GpuModel(cfg, inp)
    xh = inp["x"].copy()
    xh[0, 3], xh[1, 7], xh[1, cfg.C - 1] = -1, cfg.V, 2**31 - 1
    x = torch.from_numpy(xh).cuda()
    dev = {n: to_dev(inp, n, cfg) for n in ["K_pre", "V_pre"]}
    gen = torch.Generator(device="cuda").manual_seed(4)
    dev["z"] = (0.05 * torch.randn((cfg.B, cfg.C, cfg.d), device="cuda", generator=gen)).to(torch.bfloat16)
    t = np.full(cfg.B, 0.5, np.float32)
    g = m.step(x, dev["z"], dev["K_pre"], dev["V_pre"], t, 1 / 12, 9)
    m.close()
    zh = to_host(dev["z"])
    for b, i in [(0, 3), (1, 7), (1, cfg.C - 1)]:
        assert np.array_equal(g["h0"][b, i], zh[b, i])
    ok = (xh >= 0) & (xh < cfg.V)
    assert ((g["x_out"] >= 0) & (g["x_out"] < cfg.V) | ~ok).all()
