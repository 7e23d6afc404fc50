"""GPU parity of the gated self-conditioning block z = FFW(p0 E): the block
alone through dg_ffw on inputs that reach GELU's curved range (both GEMM
kernels, ragged rows, several widths), the step with the block attached
(p0 E tap, z, tokens), adaptive generation with frozen canvases, detaching,
and the argument checks."""
import numpy as np
import pytest

from oracle import denoise_step, ffw, generate_canvas_entropy
from tests.dg_harness import (RTOL_BF16, RTOL_F32, GpuModel, act_tensor, assert_close, to_dev,
                              to_host, token_gate)
from workloads import get_config, make_inputs
from workloads.inputs import bf16_bits_from_f32, f32_from_bf16_bits

pytestmark = pytest.mark.gpu

CASES = {
    # fp32 VALU kernels, a width that is not a multiple of anything
    "c1-F48": dict(base="c1", ffw_hidden=48),
    # 64 x 64 tiles with ragged rows (R = 80)
    "bf16-d256-F512": dict(base="c2", B=2, C=40, P=100, d=256, n_q_heads=4, n_kv_heads=2,
                           head_dim=64, V=4096, ffw_hidden=512),
    # the large-vocabulary model's width d = 2816, few rows
    "bf16-d2816-F128": dict(base="c4", B=1, C=24, P=40, d=2816, n_q_heads=16, n_kv_heads=8,
                            head_dim=176, V=1024, ffw_hidden=128),
    # 2250 rows: 256 x 256 tiles for both GEMMs, ragged last row tile
    "bf16-rows2250-F256": dict(base="c5", B=9, C=250, P=70, d=256, n_q_heads=4, n_kv_heads=4,
                               head_dim=64, V=4096, ffw_hidden=256),
    # 200 rows, 2F = 8192: the gate/up GEMM takes 128-row tiles (ragged
    # second tile); the down GEMM 64-row ones
    "bf16-rows200-F4096": dict(base="c2", B=1, C=200, P=100, d=256, n_q_heads=4, n_kv_heads=2,
                               head_dim=64, V=4096, ffw_hidden=4096),
    # 2250 rows with 2F = 384 (not a multiple of 256): gate/up on 64 x 64 tiles
    "bf16-rows2250-F192": dict(base="c5", B=9, C=250, P=70, d=256, n_q_heads=4, n_kv_heads=4,
                               head_dim=64, V=4096, ffw_hidden=192),
}


def _cfg(name):
    spec = dict(CASES[name])
    return get_config(spec.pop("base"), **spec)


def _model_with_ffw(cfg, inp):
    import discrete_diffusion_decoding_dg_amd as dg
    m = GpuModel(cfg, inp)
    fw = {n: to_dev(inp, n, cfg) for n in ["W_gate", "W_up", "W_down"]}
    dg.dg_set_ffw(m.model, fw["W_gate"], fw["W_up"], fw["W_down"])
    return m, fw


def _act_input(cfg, a):
    """float array -> (act-rounded float64 copy, device tensor)."""
    import torch
    a = np.asarray(a, np.float32)
    if cfg.dtype == "bf16":
        bits = bf16_bits_from_f32(a)
        dev = torch.from_numpy(bits.view(np.int16).reshape(a.shape)).view(torch.bfloat16).cuda()
        return f32_from_bf16_bits(bits).reshape(a.shape).astype(np.float64), dev
    return a.astype(np.float64), torch.from_numpy(a).cuda()


@pytest.mark.parametrize("name", list(CASES))
def test_ffw_block_matches_oracle(name):
    import torch
    import discrete_diffusion_decoding_dg_amd as dg
    cfg = _cfg(name)
    inp = make_inputs(cfg)
    m, _ = _model_with_ffw(cfg, inp)
    # u ~ N(0, 1): the gate pre-activations are ~N(0, 1), GELU's curved range
    u_h, u = _act_input(cfg, np.random.default_rng(4).standard_normal((cfg.B, cfg.C, cfg.d)))
    z = act_tensor((cfg.B, cfg.C, cfg.d), cfg)
    print(f"[gpu] ffw block {name} R={cfg.R} d={cfg.d} F={cfg.ffw_hidden}", flush=True)
    dg.dg_ffw(m.model, u, z)
    torch.cuda.synchronize()
    want = ffw(u_h, inp["W_gate"], inp["W_up"], inp["W_down"], cfg.dtype)
    assert_close("z", to_host(z), want, RTOL_F32 if cfg.dtype == "f32" else RTOL_BF16)
    # a second call on the same buffers gives the same bits
    z2 = act_tensor((cfg.B, cfg.C, cfg.d), cfg)
    dg.dg_ffw(m.model, u, z2)
    torch.cuda.synchronize()
    assert np.array_equal(to_host(z), to_host(z2))
    m.close()


@pytest.mark.parametrize("name", ["c1-F48", "bf16-d256-F512"])
def test_step_with_ffw_matches_oracle(name):
    import torch
    cfg = _cfg(name)
    inp = make_inputs(cfg)
    m, _ = _model_with_ffw(cfg, inp)
    dev = {n: to_dev(inp, n, cfg) for n in ["z", "K_pre", "V_pre"]}
    x = torch.from_numpy(inp["x"]).cuda()
    t = np.full(cfg.B, 0.5, np.float32)
    dt = np.float32(1.0 / cfg.steps)
    print(f"[gpu] step with ffw {name}", flush=True)
    import discrete_diffusion_decoding_dg_amd as dg
    x_out = torch.empty((cfg.B, cfg.C), dtype=torch.int32, device="cuda")
    z_out = act_tensor((cfg.B, cfg.C, cfg.d), cfg)
    p0E = act_tensor((cfg.B, cfg.C, cfg.d), cfg)
    dg.dg_denoise_step_taps(m.model, x, dev["z"], dev["K_pre"], dev["V_pre"], t, dt, 9, x_out, z_out,
                            {"p0E": p0E})
    torch.cuda.synchronize()
    w = {k: inp[k] for k in ["E", "Wq", "Wk", "Wv", "Wo", "W_gate", "W_up", "W_down"]}
    o = denoise_step(cfg, w, inp["x"], inp["z"], inp["K_pre"], inp["V_pre"], t, float(dt), 9)
    rt = RTOL_F32 if cfg.dtype == "f32" else RTOL_BF16
    assert_close("p0E", to_host(p0E), o["p0E"], rt)
    assert_close("z", to_host(z_out), o["z_out"], rt)
    token_gate(x_out.cpu().numpy(), o)
    # the block applied to the GPU's own p0 E gives the step's z exactly
    z_blk = act_tensor((cfg.B, cfg.C, cfg.d), cfg)
    dg.dg_ffw(m.model, p0E, z_blk)
    torch.cuda.synchronize()
    assert np.array_equal(to_host(z_blk), to_host(z_out))
    m.close()


def test_detach_restores_identity_block():
    import torch
    import discrete_diffusion_decoding_dg_amd as dg
    cfg = _cfg("bf16-d256-F512")
    inp = make_inputs(cfg)
    m = GpuModel(cfg, inp)
    dev = {n: to_dev(inp, n, cfg) for n in ["z", "K_pre", "V_pre"]}
    x = torch.from_numpy(inp["x"]).cuda()
    t = np.full(cfg.B, 0.4, np.float32)
    a = m.step(x, dev["z"], dev["K_pre"], dev["V_pre"], t, 1 / 12, 3, taps=False)
    fw = {n: to_dev(inp, n, cfg) for n in ["W_gate", "W_up", "W_down"]}
    dg.dg_set_ffw(m.model, fw["W_gate"], fw["W_up"], fw["W_down"])
    b = m.step(x, dev["z"], dev["K_pre"], dev["V_pre"], t, 1 / 12, 3, taps=False)
    dg.dg_set_ffw(m.model)
    c = m.step(x, dev["z"], dev["K_pre"], dev["V_pre"], t, 1 / 12, 3, taps=False)
    m.close()
    assert np.array_equal(a["x_out"], b["x_out"]) and np.array_equal(a["x_out"], c["x_out"])
    assert np.array_equal(a["z_out"], c["z_out"])
    assert not np.array_equal(a["z_out"], b["z_out"])


def test_argument_checks():
    import discrete_diffusion_decoding_dg_amd as dg
    cfg = _cfg("bf16-d256-F512")
    inp = make_inputs(cfg)
    m = GpuModel(cfg, inp)
    u = act_tensor((cfg.B, cfg.C, cfg.d), cfg).zero_()
    z = act_tensor((cfg.B, cfg.C, cfg.d), cfg)
    with pytest.raises(dg.DgError, match="INVALID_ARG"):
        dg.dg_ffw(m.model, u, z)                      # no block attached
    fw = {n: to_dev(inp, n, cfg) for n in ["W_gate", "W_up", "W_down"]}
    with pytest.raises(dg.DgError, match="UNSUPPORTED"):
        dg.dg_set_ffw(m.model, fw["W_gate"][:96], fw["W_up"][:96], fw["W_down"])   # 96 % 64 != 0
    with pytest.raises(dg.DgError, match="INVALID_ARG"):
        dg.dg_ffw(m.model, u, z)                      # the failed attach left none
    dg.dg_set_ffw(m.model, fw["W_gate"], fw["W_up"], fw["W_down"])
    with pytest.raises(dg.DgError, match="INVALID_ARG"):
        dg.dg_ffw(m.model, u, u)                      # output overlaps input
    m.close()


@pytest.mark.parametrize("name,gain", [("c1-F48", 8.0), ("bf16-d256-F512", 64.0)])
def test_adaptive_generation_with_ffw_freezes_stopped_canvases(name, gain):
    """Sharpened embeddings stop canvases early; generation (frozen canvases
    inside the library) equals the single-step calls with freezing on the
    host, and the oracle."""
    import torch
    import discrete_diffusion_decoding_dg_amd as dg
    cfg = _cfg(name).with_(B=3) if name.startswith("c1") else _cfg(name)
    inp = make_inputs(cfg)
    E = inp["E"].astype(np.float32) * np.float32(gain)
    if cfg.dtype == "bf16":
        inp["E_bits"] = bf16_bits_from_f32(E)
        E = f32_from_bf16_bits(inp["E_bits"]).reshape(E.shape)
    inp["E"] = E
    m, _ = _model_with_ffw(cfg, inp)
    dev = {n: to_dev(inp, n, cfg) for n in ["K_pre", "V_pre"]}
    max_steps, seed, eps_a, eps_s = 10, 3, 1e9, 1e9
    x = torch.empty((cfg.B, cfg.C), dtype=torch.int32, device="cuda")
    z = act_tensor((cfg.B, cfg.C, cfg.d), cfg)
    steps = torch.empty((cfg.B,), dtype=torch.int32, device="cuda")
    print(f"[gpu] adaptive generation with ffw {name}", flush=True)
    dg.dg_generate_canvas_entropy(m.model, dev["K_pre"], dev["V_pre"], max_steps, seed, eps_a, eps_s,
                                  x, steps, z)
    torch.cuda.synchronize()
    from tests.test_gpu_entropy import _stepwise_generation
    xs, zs, ss, _ = _stepwise_generation(m, cfg, dev, max_steps, seed, eps_a, eps_s)
    print(f"[gpu] steps taken per canvas: {ss.tolist()}", flush=True)
    assert np.array_equal(steps.cpu().numpy(), ss) and np.array_equal(x.cpu().numpy(), xs)
    assert np.array_equal(to_host(z), zs)
    assert (ss < max_steps).all(), "sharp predictions should stop every canvas early"
    w = {k: inp[k] for k in ["E", "Wq", "Wk", "Wv", "Wo", "W_gate", "W_up", "W_down"]}
    og = generate_canvas_entropy(cfg, w, inp["K_pre"], inp["V_pre"], max_steps, seed, eps_a, eps_s)
    assert np.array_equal(og["steps"], ss)
    assert np.array_equal(og["x"], xs)
    assert_close("z", zs, og["z"], RTOL_F32 if cfg.dtype == "f32" else RTOL_BF16)
    m.close()
