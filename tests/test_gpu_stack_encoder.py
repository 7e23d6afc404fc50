"""GPU parity of the decoder stack's causal encoder pass: prompt prefill and
canvas commit with a stack attached (every layer's cache entries against the
oracle, chunked prompts longer than a canvas, untouched rows), and
block-autoregressive generation through the stack (every canvas equal to a
single-canvas generation over exactly its prefix, every commit equal to the
oracle's entries of that canvas)."""
import numpy as np
import pytest

from oracle import encode_kv_stack
from tests.dg_harness import RTOL_BF16, RTOL_F32, GpuModel, assert_close, to_dev, to_host
from workloads import get_config, make_inputs

pytestmark = pytest.mark.gpu

LAYER_NAMES = ["Wq", "Wk", "Wv", "Wo", "g_attn", "g_mlp", "W_gate", "W_up", "W_down"]

CASES = {
    # fp32, two layers; 30 tokens after 5 history rows: two chunks of C = 16
    "c1-L2": dict(base="c1", P=48, n_layers=2, mlp_hidden=48, pos=5, n=30),
    # bf16, three layers: 100 tokens in chunks of 40 (two whole, one ragged)
    "bf16-L3": dict(base="c2", B=2, C=40, P=160, d=256, n_q_heads=4, n_kv_heads=2, head_dim=64,
                    V=4096, n_layers=3, mlp_hidden=512, pos=37, n=100),
    # no history rows: the first new token sees only itself
    "bf16-L2-from-0": dict(base="c2", B=1, C=64, P=96, d=512, n_q_heads=8, n_kv_heads=2, head_dim=64,
                           V=2048, n_layers=2, mlp_hidden=256, pos=0, n=96),
    # width 2816, head_dim 176
    "bf16-hd176-L2": dict(base="c4", B=1, C=24, P=64, d=2816, n_q_heads=16, n_kv_heads=8,
                          head_dim=176, V=1024, n_layers=2, mlp_hidden=128, pos=10, n=30),
    # a 256-token chunk after 300 history rows with four query heads per kv
    # head: 8-wave causal attention blocks (the skewed schedule, 5 splits of
    # two key tiles), then a 44-token chunk
    "bf16-L2-8-wave-skew": dict(base="c2", B=4, C=256, P=640, d=512, n_q_heads=8, n_kv_heads=2,
                                head_dim=64, V=2048, n_layers=2, mlp_hidden=256, pos=300, n=300),
    # experts in every layer, all selected (no routing decision to drift)
    "bf16-moe-L2-all": dict(base="c2", B=2, C=40, P=100, d=256, n_q_heads=4, n_kv_heads=2,
                            head_dim=64, V=4096, n_layers=2, mlp_hidden=128, n_experts=4, top_k=4,
                            pos=20, n=50),
}


def _split(spec):
    spec = dict(spec)
    base = spec.pop("base")
    ex = {k: spec.pop(k) for k in ["pos", "n", "P0", "n_canvases"] if k in spec}
    return get_config(base, **spec), ex


def _attach(m, cfg, inp):
    import discrete_diffusion_decoding_dg_amd as dg
    layers = []
    for l in range(cfg.n_layers):
        lw = {n: to_dev(inp, "S_" + n, cfg)[l].contiguous() for n in LAYER_NAMES}
        if cfg.n_experts:
            lw["W_router"] = to_dev(inp, "S_W_router", cfg)[l].contiguous()
        layers.append(lw)
    gf = to_dev(inp, "S_g_final", cfg)
    dg.dg_set_stack(m.model, layers, gf, top_k=cfg.top_k)
    return layers, gf


def _sw(cfg, inp):
    sw = {n: [inp["S_" + n][l] for l in range(cfg.n_layers)] for n in LAYER_NAMES}
    sw["g_final"] = inp["S_g_final"]
    if cfg.n_experts:
        sw["W_router"] = [inp["S_W_router"][l] for l in range(cfg.n_layers)]
        sw["top_k"] = cfg.top_k
    return sw


def _tol(cfg):
    # every layer re-rounds the stream (as in the stack's step tests): L times
    # the single block's tolerance, the plain bound at two sub-blocks per layer
    rt = (RTOL_F32 if cfg.dtype == "f32" else RTOL_BF16) * cfg.n_layers
    return rt, 2 * rt


@pytest.mark.parametrize("name", list(CASES))
def test_stack_encoder_matches_oracle(name):
    import torch
    import discrete_diffusion_decoding_dg_amd as dg
    cfg, ex = _split(CASES[name])
    pos, n = ex["pos"], ex["n"]
    inp = make_inputs(cfg)
    m = GpuModel(cfg, inp)
    keep = _attach(m, cfg, inp)
    # history rows [0, pos) from the seeded cache; the rest starts as a marker
    K0 = inp["S_K_pre"].copy()
    V0 = inp["S_V_pre"].copy()
    K0[:, :, :, pos:] = 7.0
    V0[:, :, :, pos:] = -3.0
    K = torch.from_numpy(K0).to(torch.bfloat16 if cfg.dtype == "bf16" else torch.float32).cuda()
    V = torch.from_numpy(V0).to(torch.bfloat16 if cfg.dtype == "bf16" else torch.float32).cuda()
    tokens = np.random.default_rng(11).integers(0, cfg.V, size=(cfg.B, n)).astype(np.int32)
    print(f"[gpu] stack encoder {name} L={cfg.n_layers} pos={pos} n={n} C={cfg.C}", flush=True)
    dg.dg_encode_kv(m.model, torch.from_numpy(tokens).cuda(), pos, K, V)
    torch.cuda.synchronize()
    m.close()
    del keep
    Kh, Vh = to_host(K), to_host(V)
    Kin, Vin = to_host(K.new_tensor(K0)), to_host(V.new_tensor(V0))   # history as stored (act)
    o = encode_kv_stack(cfg, inp["E"], _sw(cfg, inp), tokens, Kin, Vin, pos)
    rt, prt = _tol(cfg)
    for l in range(cfg.n_layers):
        assert_close(f"layer {l} k", Kh[l][:, :, pos:pos + n], o["k"][l], rt, plain_rtol=prt)
        assert_close(f"layer {l} v", Vh[l][:, :, pos:pos + n], o["v"][l], rt, plain_rtol=prt)
    # nothing outside rows [pos, pos + n) of any layer is touched
    rest = np.ones(cfg.P, bool)
    rest[pos:pos + n] = False
    assert np.array_equal(Kh[:, :, :, rest], Kin[:, :, :, rest])
    assert np.array_equal(Vh[:, :, :, rest], Vin[:, :, :, rest])


BLOCKS = {
    "c1-L2": dict(base="c1", P=8 + 2 * 16, n_layers=2, mlp_hidden=48, P0=8, n_canvases=2),
    "bf16-L2": dict(base="c2", B=2, C=40, P=60 + 2 * 40, d=256, n_q_heads=4, n_kv_heads=2,
                    head_dim=64, V=512, n_layers=2, mlp_hidden=256, P0=60, n_canvases=2),
}


@pytest.mark.parametrize("name", list(BLOCKS))
def test_stack_generate_blocks(name):
    import torch
    import discrete_diffusion_decoding_dg_amd as dg
    cfg, ex = _split(BLOCKS[name])
    P0, nb = ex["P0"], ex["n_canvases"]
    steps, seed = 3, 17
    inp = make_inputs(cfg)
    m = GpuModel(cfg, inp)
    keep = _attach(m, cfg, inp)
    dtype = torch.bfloat16 if cfg.dtype == "bf16" else torch.float32
    K = to_dev(inp, "S_K_pre", cfg).clone()
    V = to_dev(inp, "S_V_pre", cfg).clone()
    K[:, :, :, P0:] = 100.0
    V[:, :, :, P0:] = -100.0
    Kstart, Vstart = to_host(K), to_host(V)
    x = torch.empty((cfg.B, nb, cfg.C), dtype=torch.int32, device="cuda")
    print(f"[gpu] stack blocks {name} P0={P0} canvases={nb} steps={steps}", flush=True)
    dg.dg_generate_blocks(m.model, K, V, P0, nb, steps, seed, x)
    torch.cuda.synchronize()
    m.close()
    xh, Kh, Vh = x.cpu().numpy(), to_host(K), to_host(V)
    rt, prt = _tol(cfg)
    sw = _sw(cfg, inp)
    for j in range(nb):
        Pj = P0 + j * cfg.C
        # canvas j: the same kernels on a stack model whose caches hold exactly Pj rows
        mj = GpuModel(cfg.with_(P=Pj), inp)
        kj = _attach(mj, cfg, inp)
        Kj = torch.from_numpy(Kh[:, :, :, :Pj].copy()).to(dtype).cuda()
        Vj = torch.from_numpy(Vh[:, :, :, :Pj].copy()).to(dtype).cuda()
        xj = torch.empty((cfg.B, cfg.C), dtype=torch.int32, device="cuda")
        dg.dg_generate_canvas(mj.model, Kj, Vj, steps, seed + j * steps, xj)
        torch.cuda.synchronize()
        mj.close()
        del kj
        assert np.array_equal(xh[:, j], xj.cpu().numpy()), f"canvas {j} differs from a single-canvas generation"
        # the commit holds the stack encoder's entries of that canvas, over the
        # cache rows written before it
        o = encode_kv_stack(cfg, inp["E"], sw, xh[:, j], Kh, Vh, Pj)
        for l in range(cfg.n_layers):
            assert_close(f"layer {l} k rows of canvas {j}", Kh[l][:, :, Pj:Pj + cfg.C], o["k"][l], rt,
                         plain_rtol=prt)
            assert_close(f"layer {l} v rows of canvas {j}", Vh[l][:, :, Pj:Pj + cfg.C], o["v"][l], rt,
                         plain_rtol=prt)
    # the prompt rows keep their values; rows past the last canvas too
    assert np.array_equal(Kh[:, :, :, :P0], Kstart[:, :, :, :P0])
    end = P0 + nb * cfg.C
    assert np.array_equal(Kh[:, :, :, end:], Kstart[:, :, :, end:])
    del keep


def test_stack_generate_blocks_entropy():
    """The recommended sampler's block generation through a stack: every canvas
    and its step count equal a single-canvas adaptive generation over exactly
    its prefix; every commit holds the stack encoder's entries."""
    import math

    import torch
    import discrete_diffusion_decoding_dg_amd as dg
    cfg, ex = _split(BLOCKS["bf16-L2"])
    P0, nb = ex["P0"], ex["n_canvases"]
    max_steps, seed = 6, 9
    eps_a, eps_s = 2.0 * math.log(cfg.V), 1.0
    inp = make_inputs(cfg)
    m = GpuModel(cfg, inp)
    keep = _attach(m, cfg, inp)
    K = to_dev(inp, "S_K_pre", cfg).clone()
    V = to_dev(inp, "S_V_pre", cfg).clone()
    K[:, :, :, P0:] = 100.0
    V[:, :, :, P0:] = -100.0
    x = torch.empty((cfg.B, nb, cfg.C), dtype=torch.int32, device="cuda")
    steps = torch.empty((cfg.B, nb), dtype=torch.int32, device="cuda")
    print(f"[gpu] stack adaptive blocks P0={P0} canvases={nb} max_steps={max_steps}", flush=True)
    dg.dg_generate_blocks_entropy(m.model, K, V, P0, nb, max_steps, seed, eps_a, eps_s, x, steps)
    torch.cuda.synchronize()
    m.close()
    xh, sh, Kh, Vh = x.cpu().numpy(), steps.cpu().numpy(), to_host(K), to_host(V)
    rt, prt = _tol(cfg)
    sw = _sw(cfg, inp)
    for j in range(nb):
        Pj = P0 + j * cfg.C
        mj = GpuModel(cfg.with_(P=Pj), inp)
        kj = _attach(mj, cfg, inp)
        Kj = torch.from_numpy(Kh[:, :, :, :Pj].copy()).to(torch.bfloat16).cuda()
        Vj = torch.from_numpy(Vh[:, :, :, :Pj].copy()).to(torch.bfloat16).cuda()
        xj = torch.empty((cfg.B, cfg.C), dtype=torch.int32, device="cuda")
        sj = torch.empty((cfg.B,), dtype=torch.int32, device="cuda")
        dg.dg_generate_canvas_entropy(mj.model, Kj, Vj, max_steps, seed + j * max_steps, eps_a, eps_s, xj, sj)
        torch.cuda.synchronize()
        mj.close()
        del kj
        assert np.array_equal(xh[:, j], xj.cpu().numpy()), f"canvas {j} differs from adaptive generation"
        assert np.array_equal(sh[:, j], sj.cpu().numpy())
        o = encode_kv_stack(cfg, inp["E"], sw, xh[:, j], Kh, Vh, Pj)
        for l in range(cfg.n_layers):
            assert_close(f"layer {l} k rows of canvas {j}", Kh[l][:, :, Pj:Pj + cfg.C], o["k"][l], rt,
                         plain_rtol=prt)
    del keep
