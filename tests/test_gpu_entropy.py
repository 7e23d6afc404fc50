"""GPU parity of the entropy-bounded step and of adaptive generation against
the oracle: entropy, argmax, z, the acceptance decided from the entropies,
the re-noised tokens, the stop test, and generation equal to step-by-step
calls of the single-step entry point."""
import numpy as np
import pytest

from oracle import accept_mask, entropy_step, generate_canvas_entropy
from tests.dg_harness import (NEAR_TIE, near_ties, RTOL_BF16, RTOL_F32, GpuModel, act_tensor, assert_close,
                              to_dev, to_host)
from workloads import get_config, make_inputs

pytestmark = pytest.mark.gpu

CASES = {
    "c1": dict(base="c1"),
    "bf16-hd64": dict(base="c2", B=2, C=40, P=100, d=256, n_q_heads=4, n_kv_heads=2, head_dim=64,
                      V=4096),
    # a canvas of 1000 positions: the select kernel's sort at 1024 lanes
    "bf16-c1000": dict(base="c2", B=2, C=1000, P=30, d=256, n_q_heads=4, n_kv_heads=2,
                       head_dim=64, V=2048),
}


def _cfg(name):
    spec = dict(CASES[name])
    return get_config(spec.pop("base"), **spec)


def _htol(cfg, H):
    return (1e-5 if cfg.dtype == "f32" else 2e-3) * np.maximum(1.0, np.abs(H))


def _gpu_entropy_step(m, cfg, dev, x, t, seed, eps_a, eps_s, det_prev=None):
    import torch
    import discrete_diffusion_decoding_dg_amd as dg
    B, C = x.shape
    x_out = torch.empty((B, C), dtype=torch.int32, device="cuda")
    z_out = act_tensor((B, C, cfg.d), cfg)
    det = torch.empty((B, C), dtype=torch.int32, device="cuda")
    H = torch.empty((B, C), dtype=torch.float32, device="cuda")
    stop = torch.empty((B,), dtype=torch.int32, device="cuda")
    print(f"[gpu] entropy step {cfg.name} B={B} C={C} V={cfg.V} seed={seed}", flush=True)
    dg.dg_denoise_step_entropy(m.model, x, dev["z"], dev["K_pre"], dev["V_pre"], t, seed, eps_a,
                               eps_s, det_prev, x_out, z_out, det, stop, H)
    torch.cuda.synchronize()
    return dict(x_out=x_out.cpu().numpy(), z_out=to_host(z_out), det=det, det_h=det.cpu().numpy(),
                H=H.cpu().numpy(), stop=stop.cpu().numpy())


@pytest.mark.parametrize("name", list(CASES))
def test_entropy_step_matches_oracle(name):
    import torch
    cfg = _cfg(name)
    inp = make_inputs(cfg)
    w = {k: inp[k] for k in ["E", "Wq", "Wk", "Wv", "Wo"]}
    m = GpuModel(cfg, inp)
    dev = {n: to_dev(inp, n, cfg) for n in ["z", "K_pre", "V_pre"]}
    x = torch.from_numpy(inp["x"]).cuda()
    t = np.full(cfg.B, 0.5, np.float32)
    seed = 21
    # acceptance threshold half way between the running sums at ranks C/4 and C/4+1 of canvas 0
    o0 = entropy_step(cfg, w, inp["x"], inp["z"], inp["K_pre"], inp["V_pre"], t, seed, 0.0, 0.0)
    cs = np.cumsum(np.sort(o0["H"][0]))
    k = max(1, cfg.C // 4)
    eps_a = float(0.5 * (cs[k - 1] + cs[k])) if cfg.C > 1 else 1.0
    o = entropy_step(cfg, w, inp["x"], inp["z"], inp["K_pre"], inp["V_pre"], t, seed, eps_a, 0.0)
    g = _gpu_entropy_step(m, cfg, dev, x, t, seed, eps_a, 0.0)

    # entropy, z, argmax
    htol = _htol(cfg, o["H"])
    assert np.all(np.abs(g["H"] - o["H"]) <= htol), f"entropy: max err {np.abs(g['H'] - o['H']).max():.3e}"
    assert_close("z", g["z_out"], o["z_out"], RTOL_F32 if cfg.dtype == "f32" else RTOL_BF16)
    # the plain argmax has no Gumbel noise: its top logits are far below 1 at
    # these weight scales, so the near-tie band is floored at NEAR_TIE
    # absolute (the logits' own bf16 rounding is of that order)
    det_near = o["det_gap"] < NEAR_TIE * np.maximum(1.0, np.abs(o["det_top"]))
    assert not ((g["det_h"] != o["det"]) & ~det_near).any(), "argmax differs off near-ties"
    assert not g["stop"].any(), "first step must not stop"

    # which positions the GPU accepted: rejected ones carry the re-noise token
    # (positions whose draw equals their re-noise token are ambiguous)
    amb = o["y"] == o["renoise"]
    g_acc = g["x_out"] != o["renoise"]
    # exactness of the rule on the GPU's own entropies, outside a rounding band at eps
    own = accept_mask(g["H"].astype(np.float64), eps_a)
    band = np.zeros_like(amb)
    for b in range(cfg.B):
        order = np.lexsort((np.arange(cfg.C), g["H"][b]))
        run = np.cumsum(g["H"][b][order].astype(np.float64))
        band[b, order] = np.abs(run - eps_a) <= 1e-4 * max(1.0, eps_a)
    bad = (g_acc != own) & ~amb & ~band
    assert not bad.any(), f"acceptance differs from the rule on the GPU entropies at {np.argwhere(bad)[:5]}"
    # against the oracle's acceptance: differences only between positions whose
    # entropies lie within the entropy tolerance of the canvas's boundary value
    for b in range(cfg.B):
        diff = (g_acc[b] != o["accept"][b]) & ~amb[b]
        if diff.any():
            Hs = np.sort(o["H"][b])
            kk = int(o["accept"][b].sum())
            hb = Hs[kk - 1] if kk < cfg.C else Hs[-1]
            assert np.all(np.abs(o["H"][b][diff] - hb) <= 4 * htol[b][diff]), \
                f"canvas {b}: acceptance differs away from the boundary"
    # accepted tokens are the draws (up to near-ties); rejected ones the re-noise tokens exactly
    both = g_acc & o["accept"] & ~amb
    near = near_ties(o["gap"], o["top1"])
    assert not ((g["x_out"] != o["y"]) & both & ~near).any(), "accepted draws differ off near-ties"
    rej = ~g_acc & ~o["accept"]
    assert np.array_equal(g["x_out"][rej], o["renoise"][rej])

    # stop test: same inputs give the same argmax
    H_mean = g["H"].mean(axis=1)
    g2 = _gpu_entropy_step(m, cfg, dev, x, t, seed, eps_a, float(H_mean.max() + 1.0), det_prev=g["det"])
    assert g2["stop"].all()
    g3 = _gpu_entropy_step(m, cfg, dev, x, t, seed, eps_a, float(H_mean.min() - 1.0), det_prev=g["det"])
    assert not g3["stop"].any()
    dp = g["det"].clone()
    dp[0, cfg.C // 2] = (dp[0, cfg.C // 2] + 1) % cfg.V
    g4 = _gpu_entropy_step(m, cfg, dev, x, t, seed, eps_a, float(H_mean.max() + 1.0), det_prev=dp)
    assert g4["stop"][0] == 0 and (cfg.B == 1 or g4["stop"][1:].all())
    m.close()


def _stepwise_generation(m, cfg, dev, max_steps, seed, eps_a, eps_s):
    """Adaptive generation from the single-step entry point, freezing stopped canvases on the host."""
    import torch
    import discrete_diffusion_decoding_dg_amd as dg
    B, C = cfg.B, cfg.C
    x = torch.empty((B, C), dtype=torch.int32, device="cuda")
    dg.dg_corrupt(m.model, torch.zeros((B, C), dtype=torch.int32, device="cuda"), [0.0] * B, seed, x)
    z = act_tensor((B, C, cfg.d), cfg)
    z.zero_()
    det_prev = None
    stopped = np.zeros(B, bool)
    steps = np.full(B, max_steps, np.int32)
    trace = []
    for k in range(max_steps):
        if stopped.all():
            break
        t = np.full(B, np.float32(1.0 - k / max_steps), np.float32)
        x_out = torch.empty_like(x)
        z_out = torch.empty_like(z)
        det = torch.empty((B, C), dtype=torch.int32, device="cuda")
        stop = torch.empty((B,), dtype=torch.int32, device="cuda")
        dg.dg_denoise_step_entropy(m.model, x, z, dev["K_pre"], dev["V_pre"], t, seed + k, eps_a,
                                   eps_s, det_prev, x_out, z_out, det, stop)
        torch.cuda.synchronize()
        keep = torch.from_numpy(stopped).cuda()
        x_out[keep] = x[keep]
        z_out[keep] = z[keep]
        if det_prev is not None:
            det[keep] = det_prev[keep]
        st = stop.cpu().numpy().astype(bool) & ~stopped
        steps[st] = k + 1
        stopped |= st
        x, z, det_prev = x_out, z_out, det
        trace.append(x.cpu().numpy())
    return x.cpu().numpy(), to_host(z), steps, trace


@pytest.mark.parametrize("name,eps_a,eps_s", [("c1", 9.0, 4.3), ("bf16-hd64", 60.0, 9.0)])
def test_adaptive_generation_equals_stepwise_and_oracle(name, eps_a, eps_s):
    import torch
    import discrete_diffusion_decoding_dg_amd as dg
    cfg = _cfg(name)
    inp = make_inputs(cfg)
    m = GpuModel(cfg, inp)
    dev = {n: to_dev(inp, n, cfg) for n in ["K_pre", "V_pre"]}
    max_steps, seed = 12, 5
    x = torch.empty((cfg.B, cfg.C), dtype=torch.int32, device="cuda")
    z = act_tensor((cfg.B, cfg.C, cfg.d), cfg)
    steps = torch.empty((cfg.B,), dtype=torch.int32, device="cuda")
    print(f"[gpu] adaptive generation {name} max_steps={max_steps}", flush=True)
    dg.dg_generate_canvas_entropy(m.model, dev["K_pre"], dev["V_pre"], max_steps, seed, eps_a, eps_s,
                                  x, steps, z)
    torch.cuda.synchronize()
    xs, zs, ss, trace = _stepwise_generation(m, cfg, dev, max_steps, seed, eps_a, eps_s)
    print(f"[gpu] steps taken per canvas: {ss.tolist()}", flush=True)
    assert np.array_equal(x.cpu().numpy(), xs)
    assert np.array_equal(steps.cpu().numpy(), ss)
    assert np.array_equal(to_host(z), zs)
    # against the oracle trajectory, up to the first step with a near-tie or
    # an acceptance decision within rounding of the threshold
    w = {k: inp[k] for k in ["E", "Wq", "Wk", "Wv", "Wo"]}
    og = generate_canvas_entropy(cfg, w, inp["K_pre"], inp["V_pre"], max_steps, seed, eps_a, eps_s)
    for k, rec in enumerate(og["records"]):
        if k >= len(trace):
            break
        act = rec["active"]
        htol = _htol(cfg, rec["H"])
        near = near_ties(rec["gap"], rec["top1"]) & rec["accept"]
        dnear = rec["det_gap"] < NEAR_TIE * np.maximum(1.0, np.abs(rec["det_top"]))
        border = np.zeros(len(act), dtype=bool)
        for j in range(len(act)):
            run = np.cumsum(np.sort(rec["H"][j]))
            border[j] = np.any(np.abs(run - eps_a) <= 4 * htol[j].max())
        if near.any() or dnear.any() or border.any():
            break                                      # later steps may legitimately diverge
        assert np.array_equal(trace[k][act], rec["x_out"]), f"step {k} differs from the oracle"
    m.close()


def test_adaptive_generation_stops_early_with_sharp_predictions():
    """A sharpened embedding (E x 8, fp32) makes every token predict itself:
    with every position accepted the argmax predictions settle and canvases
    stop early; generation must equal the step-by-step calls and the oracle."""
    import torch
    import discrete_diffusion_decoding_dg_amd as dg
    cfg = get_config("c1", B=3)
    inp = make_inputs(cfg)
    inp["E"] = (inp["E"] * 8.0).astype(np.float32)
    m = GpuModel(cfg, inp)
    dev = {n: to_dev(inp, n, cfg) for n in ["K_pre", "V_pre"]}
    max_steps, seed, eps_a, eps_s = 10, 3, 1e9, 1e9
    x = torch.empty((cfg.B, cfg.C), dtype=torch.int32, device="cuda")
    z = act_tensor((cfg.B, cfg.C, cfg.d), cfg)
    steps = torch.empty((cfg.B,), dtype=torch.int32, device="cuda")
    dg.dg_generate_canvas_entropy(m.model, dev["K_pre"], dev["V_pre"], max_steps, seed, eps_a, eps_s,
                                  x, steps, z)
    torch.cuda.synchronize()
    xs, zs, ss, _ = _stepwise_generation(m, cfg, dev, max_steps, seed, eps_a, eps_s)
    print(f"[gpu] sharp: steps taken per canvas: {ss.tolist()}", flush=True)
    assert np.array_equal(steps.cpu().numpy(), ss) and np.array_equal(x.cpu().numpy(), xs)
    assert np.array_equal(to_host(z), zs)
    assert (ss < max_steps).all(), "sharp predictions should stop every canvas early"
    w = {k: inp[k] for k in ["E", "Wq", "Wk", "Wv", "Wo"]}
    og = generate_canvas_entropy(cfg, w, inp["K_pre"], inp["V_pre"], max_steps, seed, eps_a, eps_s)
    assert np.array_equal(og["steps"], ss)
    assert np.array_equal(og["x"], xs)
    m.close()
