"""GPU parity of the multi-layer decoder stack against the oracle: the step
with a stack attached (embedding, last layer's q/k/v/o, the final normalised
activation, lse, z, tokens), generation equal to step-by-step calls and
detaching (the stack's encoder pass: test_gpu_stack_encoder.py)."""
import numpy as np
import pytest

from oracle import lm_head, stack_step, step_select
from tests.dg_harness import (LSE_RTOL, RTOL_BF16, RTOL_F32, GpuModel, act_tensor, assert_close,
                              to_dev, to_host, token_gate)
from workloads import get_config, make_inputs

pytestmark = pytest.mark.gpu

CASES = {
    "c1-L2": dict(base="c1", n_layers=2, mlp_hidden=48),
    # ragged rows (80 = 64 + 16) and keys, one layer and three layers
    "bf16-L1": dict(base="c2", B=2, C=40, P=100, d=256, n_q_heads=4, n_kv_heads=2, head_dim=64,
                    V=4096, n_layers=1, mlp_hidden=512),
    "bf16-L3": dict(base="c2", B=2, C=40, P=100, d=256, n_q_heads=4, n_kv_heads=2, head_dim=64,
                    V=4096, n_layers=3, mlp_hidden=512),
    # width 2816 and head_dim 176
    "bf16-hd176-L2": dict(base="c4", B=1, C=24, P=40, d=2816, n_q_heads=16, n_kv_heads=8,
                          head_dim=176, V=1024, n_layers=2, mlp_hidden=128),
    # 2250 rows: the 256 x 256-tile GEMMs in every layer
    "bf16-rows2250-L2": dict(base="c5", B=9, C=250, P=70, d=256, n_q_heads=4, n_kv_heads=4,
                             head_dim=64, V=4096, n_layers=2, mlp_hidden=256),
}
LAYER_NAMES = ["Wq", "Wk", "Wv", "Wo", "g_attn", "g_mlp", "W_gate", "W_up", "W_down"]


def _cfg(name):
    spec = dict(CASES[name])
    return get_config(spec.pop("base"), **spec)


def _layers_dev(cfg, inp):
    """Per-layer device tensors (slices of the stacked inputs, made contiguous)."""
    layers = []
    for l in range(cfg.n_layers):
        lw = {}
        for n in LAYER_NAMES:
            full = to_dev(inp, "S_" + n, cfg)
            lw[n] = full[l].contiguous()
        layers.append(lw)
    return layers


def _attach(m, cfg, inp):
    import discrete_diffusion_decoding_dg_amd as dg
    layers = _layers_dev(cfg, inp)
    gf = to_dev(inp, "S_g_final", cfg)
    dg.dg_set_stack(m.model, layers, gf)
    return layers, gf


def _oracle(cfg, inp, x, z, t, dt, seed):
    sw = {n: [inp["S_" + n][l] for l in range(cfg.n_layers)] for n in LAYER_NAMES}
    sw["g_final"] = inp["S_g_final"]
    return stack_step(cfg, {"E": inp["E"]}, sw, x, z, inp["S_K_pre"], inp["S_V_pre"], t, dt, seed)


@pytest.mark.parametrize("name", list(CASES))
def test_stack_step_matches_oracle(name):
    import torch
    import discrete_diffusion_decoding_dg_amd as dg
    cfg = _cfg(name)
    inp = make_inputs(cfg)
    m = GpuModel(cfg, inp)
    keep = _attach(m, cfg, inp)
    Kp, Vp = to_dev(inp, "S_K_pre", cfg), to_dev(inp, "S_V_pre", cfg)
    z = to_dev(inp, "z", cfg)
    x = torch.from_numpy(inp["x"]).cuda()
    t = np.full(cfg.B, 0.5, np.float32)
    dt = np.float32(1.0 / cfg.steps)
    B, C = cfg.B, cfg.C
    taps = dict(h0=act_tensor((B, C, cfg.d), cfg), q=act_tensor((B, C, cfg.n_q_heads, cfg.head_dim), cfg),
                k=act_tensor((B, cfg.n_kv_heads, C, cfg.head_dim), cfg),
                v=act_tensor((B, cfg.n_kv_heads, C, cfg.head_dim), cfg),
                o=act_tensor((B, C, cfg.n_q_heads, cfg.head_dim), cfg), h1=act_tensor((B, C, cfg.d), cfg),
                lse=torch.empty((B, C), dtype=torch.float32, device="cuda"),
                best=torch.empty((B, C), dtype=torch.int32, device="cuda"))
    x_out = torch.empty((B, C), dtype=torch.int32, device="cuda")
    z_out = act_tensor((B, C, cfg.d), cfg)
    print(f"[gpu] stack step {name} L={cfg.n_layers} F={cfg.mlp_hidden} R={cfg.R}", flush=True)
    dg.dg_denoise_step_taps(m.model, x, z, Kp, Vp, t, dt, 13, x_out, z_out, taps)
    torch.cuda.synchronize()
    m.close()
    del keep
    o = _oracle(cfg, inp, inp["x"], inp["z"], t, float(dt), 13)
    # each layer re-rounds the residual stream and its intermediates to act:
    # the single block's tolerance per layer, added over the layers (the
    # norms keep the stream's scale, so the per-layer errors do not grow)
    rt = (RTOL_F32 if cfg.dtype == "f32" else RTOL_BF16) * cfg.n_layers
    last = o["layers"][-1]
    assert_close("h0", to_host(taps["h0"]), o["h0"], rt)
    for n in ["q", "k", "v", "o"]:
        assert_close(f"last layer {n}", to_host(taps[n]), last[n], rt)
    hf = to_host(taps["h1"])
    # entries above rms: the plain relative bound per residual sub-block, two
    # per layer (attention and MLP, each re-rounding the stream like the
    # single block), applied to the final norm that sees both
    assert_close("final norm", hf, o["h_final"], rt, plain_rtol=2 * rt)
    # the head after the stack, from the GPU's own final activation (the
    # softmax amplifies the stack's drift in z; the head itself is checked at
    # the single block's tolerances)
    head = lm_head(hf.astype(np.float64), inp["E"], o["inv_tau"], cfg.dtype)
    smp = step_select(inp["x"], head["s"], o["lam"], 13, np.arange(cfg.B))
    r1 = RTOL_F32 if cfg.dtype == "f32" else RTOL_BF16
    assert_close("lse", taps["lse"].cpu().numpy().ravel(), head["lse"], RTOL_F32 if cfg.dtype == "f32" else LSE_RTOL)
    assert_close("z", to_host(z_out), head["z"], r1)
    assert np.array_equal(taps["best"].cpu().numpy() >= 0, smp["resample"])
    token_gate(x_out.cpu().numpy(), smp)
    # and against the oracle's own stack end to end
    assert_close("lse (end to end)", taps["lse"].cpu().numpy().ravel(), o["lse"],
                 RTOL_F32 if cfg.dtype == "f32" else LSE_RTOL * cfg.n_layers)


def test_stack_generation_equals_step_by_step_calls():
    import torch
    import discrete_diffusion_decoding_dg_amd as dg
    cfg = _cfg("bf16-L3")
    inp = make_inputs(cfg)
    m = GpuModel(cfg, inp)
    keep = _attach(m, cfg, inp)
    Kp, Vp = to_dev(inp, "S_K_pre", cfg), to_dev(inp, "S_V_pre", cfg)
    steps, seed = 4, 8
    xg = torch.empty((cfg.B, cfg.C), dtype=torch.int32, device="cuda")
    zg = act_tensor((cfg.B, cfg.C, cfg.d), cfg)
    dg.dg_generate_canvas(m.model, Kp, Vp, steps, seed, xg, zg)
    x = torch.zeros((cfg.B, cfg.C), dtype=torch.int32, device="cuda")
    kap = torch.zeros((cfg.B,), dtype=torch.float32, device="cuda")
    dg.dg_corrupt_batch(x, kap, cfg.B, cfg.C, cfg.V, seed, x)
    z = act_tensor((cfg.B, cfg.C, cfg.d), cfg).zero_()
    dt = float(np.float32(1.0 / steps))
    for k in range(steps):
        t = np.full(cfg.B, np.float32(1.0 - k / steps), np.float32)
        xn, zn = torch.empty_like(x), torch.empty_like(z)
        dg.dg_denoise_step(m.model, x, z, Kp, Vp, t, dt, seed + k, xn, zn)
        x, z = xn, zn
    torch.cuda.synchronize()
    m.close()
    del keep
    assert np.array_equal(xg.cpu().numpy(), x.cpu().numpy())
    assert np.array_equal(to_host(zg), to_host(z))


def test_detach_restores_the_single_block():
    import torch
    import discrete_diffusion_decoding_dg_amd as dg
    cfg = _cfg("c1-L2")
    inp = make_inputs(cfg)
    m = GpuModel(cfg, inp)
    dev = {n: to_dev(inp, n, cfg) for n in ["z", "K_pre", "V_pre"]}
    x = torch.from_numpy(inp["x"]).cuda()
    t = np.full(cfg.B, 0.4, np.float32)
    a = m.step(x, dev["z"], dev["K_pre"], dev["V_pre"], t, 1 / 8, 3, taps=False)
    keep = _attach(m, cfg, inp)
    dg.dg_set_stack(m.model)
    b = m.step(x, dev["z"], dev["K_pre"], dev["V_pre"], t, 1 / 8, 3, taps=False)
    m.close()
    del keep
    assert np.array_equal(a["x_out"], b["x_out"]) and np.array_equal(a["z_out"], b["z_out"])


MOE = {
    # fp32: one and two layers, 4 experts, top 2
    "c1-moe-L1": dict(base="c1", n_layers=1, mlp_hidden=48, n_experts=4, top_k=2),
    "c1-moe-L2": dict(base="c1", n_layers=2, mlp_hidden=48, n_experts=4, top_k=2),
    # bf16, 8 experts, top 2, ragged rows
    "bf16-moe-L1": dict(base="c2", B=2, C=40, P=100, d=256, n_q_heads=4, n_kv_heads=2, head_dim=64,
                        V=4096, n_layers=1, mlp_hidden=256, n_experts=8, top_k=2),
    # bf16, two layers with every expert selected (no routing decision to drift)
    "bf16-moe-L2-all": dict(base="c2", B=2, C=40, P=100, d=256, n_q_heads=4, n_kv_heads=2,
                            head_dim=64, V=4096, n_layers=2, mlp_hidden=128, n_experts=4, top_k=4),
    # 2250 tokens routed over 4 experts: many expert tiles, partial last tiles;
    # with zero output projections the experts see the embedding itself, so
    # the GPU's routing input equals the oracle's up to one norm's rounding
    "bf16-moe-rows2250-wo0": dict(base="c5", B=9, C=250, P=70, d=256, n_q_heads=4, n_kv_heads=4,
                                  head_dim=64, V=4096, n_layers=1, mlp_hidden=256, n_experts=4, top_k=2,
                                  zero_wo=True),
    "bf16-moe-rows2250": dict(base="c5", B=9, C=250, P=70, d=256, n_q_heads=4, n_kv_heads=4,
                              head_dim=64, V=4096, n_layers=1, mlp_hidden=256, n_experts=4, top_k=2),
    # width 2816, top 1
    "bf16-moe-hd176": dict(base="c4", B=1, C=24, P=40, d=2816, n_q_heads=16, n_kv_heads=8,
                           head_dim=176, V=1024, n_layers=1, mlp_hidden=128, n_experts=4, top_k=1),
    # 66,000 routed entries over 8 experts: more (expert, 64-entry chunk)
    # cells than the one-pass grouping holds, so the per-expert grouping
    # runs; canvases are independent, so the oracle checks the first four
    "bf16-moe-long-list": dict(base="c5", B=132, C=250, P=70, d=256, n_q_heads=4, n_kv_heads=4,
                               head_dim=64, V=1024, n_layers=1, mlp_hidden=128, n_experts=8, top_k=2,
                               zero_wo=True, oracle_canvases=4),
}


@pytest.mark.parametrize("name", list(MOE))
def test_moe_stack_step_matches_oracle(name):
    import torch
    import discrete_diffusion_decoding_dg_amd as dg
    from oracle.stack import route
    spec = dict(MOE[name])
    zero_wo = spec.pop("zero_wo", False)
    nb = spec.pop("oracle_canvases", None)
    cfg = get_config(spec.pop("base"), **spec)
    inp = make_inputs(cfg)
    if zero_wo:
        inp["S_Wo"] = np.zeros_like(inp["S_Wo"])
        if "S_Wo_bits" in inp:
            inp["S_Wo_bits"] = np.zeros_like(inp["S_Wo_bits"])
    m = GpuModel(cfg, inp)
    layers = _layers_dev(cfg, inp)
    wr = to_dev(inp, "S_W_router", cfg)
    for l, lw in enumerate(layers):
        lw["W_router"] = wr[l].contiguous()
    gf = to_dev(inp, "S_g_final", cfg)
    dg.dg_set_stack(m.model, layers, gf, top_k=cfg.top_k)
    Kp, Vp = to_dev(inp, "S_K_pre", cfg), to_dev(inp, "S_V_pre", cfg)
    z = to_dev(inp, "z", cfg)
    x = torch.from_numpy(inp["x"]).cuda()
    t = np.full(cfg.B, 0.5, np.float32)
    dt = np.float32(1.0 / cfg.steps)
    B, C = cfg.B, cfg.C
    h1 = act_tensor((B, C, cfg.d), cfg)
    lse = torch.empty((B, C), dtype=torch.float32, device="cuda")
    x_out = torch.empty((B, C), dtype=torch.int32, device="cuda")
    z_out = act_tensor((B, C, cfg.d), cfg)
    print(f"[gpu] moe stack step {name} L={cfg.n_layers} X={cfg.n_experts} k={cfg.top_k} R={cfg.R}", flush=True)
    dg.dg_denoise_step_taps(m.model, x, z, Kp, Vp, t, dt, 17, x_out, z_out, {"h1": h1, "lse": lse})
    torch.cuda.synchronize()
    m.close()
    del layers, wr, gf
    # the oracle runs the first nb canvases (each canvas is independent of
    # the others: its own cache, its own Philox streams)
    nb = nb or B
    h1, lse, x_out, z_out = h1[:nb], lse[:nb], x_out[:nb], z_out[:nb]
    cfg = cfg.with_(B=nb)
    B = nb
    inp = dict(inp, x=inp["x"][:nb], z=inp["z"][:nb], S_K_pre=inp["S_K_pre"][:, :nb],
               S_V_pre=inp["S_V_pre"][:, :nb])
    t = t[:nb]
    sw = {n: [inp["S_" + n][l] for l in range(cfg.n_layers)] for n in LAYER_NAMES}
    sw["W_router"] = [inp["S_W_router"][l] for l in range(cfg.n_layers)]
    sw["g_final"], sw["top_k"] = inp["S_g_final"], cfg.top_k
    o = stack_step(cfg, {"E": inp["E"]}, sw, inp["x"], inp["z"], inp["S_K_pre"], inp["S_V_pre"], t,
                   float(dt), 17)
    # rows whose routing is within the stream's rounding of a tie may pick
    # another expert on the GPU; they are left out (all of them with one
    # layer; with more layers only when every expert is selected)
    keep = np.ones(cfg.R, bool)
    if cfg.top_k < cfg.n_experts:
        for l in range(cfg.n_layers):
            _, _, r = route(o["layers"][l]["m"].reshape(cfg.R, cfg.d), sw["W_router"][l], cfg.top_k)
            srt = -np.sort(-r.astype(np.float64), axis=1)
            margin = srt[:, cfg.top_k - 1] - srt[:, cfg.top_k]
            # the routing input m drifts by about the stream's tolerance (one
            # norm's rounding only when the attention output is zero)
            drift = 1e-4 if cfg.dtype == "f32" else (5e-3 if zero_wo else 2 * RTOL_BF16)
            tol = drift * np.sqrt((r.astype(np.float64) ** 2).mean())
            keep &= margin > tol
        assert cfg.n_layers == 1 or cfg.dtype == "f32" or keep.all()
    print(f"[gpu] rows compared: {int(keep.sum())} of {cfg.R}", flush=True)
    assert keep.mean() > 0.9
    rt = (RTOL_F32 if cfg.dtype == "f32" else RTOL_BF16) * cfg.n_layers
    hf = to_host(h1).reshape(cfg.R, cfg.d)
    assert_close("final norm", hf[keep], o["h_final"].reshape(cfg.R, cfg.d)[keep], rt,
                 plain_rtol=2 * rt)
    head = lm_head(hf.reshape(B, C, cfg.d).astype(np.float64), inp["E"], o["inv_tau"], cfg.dtype)
    smp = step_select(inp["x"], head["s"], o["lam"], 17, np.arange(cfg.B))
    r1 = RTOL_F32 if cfg.dtype == "f32" else RTOL_BF16
    assert_close("lse", lse.cpu().numpy().ravel()[keep], head["lse"][keep],
                 RTOL_F32 if cfg.dtype == "f32" else LSE_RTOL)
    assert_close("z", to_host(z_out).reshape(cfg.R, cfg.d)[keep], head["z"].reshape(cfg.R, cfg.d)[keep], r1)
    token_gate(x_out.cpu().numpy(), smp)
