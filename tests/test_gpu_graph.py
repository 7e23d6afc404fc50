"""GPU check that dg_denoise_step can be captured into a HIP graph: the
step launches kernels only (no allocation, host synchronisation or memset on
its path), so a captured step replays the same work. Each of three replays,
with unrelated eager work and synchronisations between them, must equal an
eager call with the same arguments bit for bit (tokens, z and lse)."""
import numpy as np
import pytest

from tests.dg_harness import GpuModel, act_tensor, to_dev
from workloads import get_config, make_inputs

pytestmark = pytest.mark.gpu

CASES = {
    # bf16: attention and LM head both split (merge kernels in the graph)
    "bf16": dict(base="c2", B=2, C=64, P=160, d=256, n_q_heads=4, n_kv_heads=2, head_dim=64, V=4096),
    "f32": dict(base="c1"),
}


def _outputs(cfg):
    import torch
    x_out = torch.full((cfg.B, cfg.C), -7, dtype=torch.int32, device="cuda")
    z_out = act_tensor((cfg.B, cfg.C, cfg.d), cfg)
    z_out.fill_(3.0)
    lse = torch.full((cfg.B, cfg.C), -1.0, dtype=torch.float32, device="cuda")
    return x_out, z_out, lse


def _host(outs, cfg):
    import torch
    x_out, z_out, lse = outs
    zb = z_out.view(torch.int16) if cfg.dtype == "bf16" else z_out.view(torch.int32)
    return x_out.cpu().numpy(), zb.cpu().numpy(), lse.view(torch.int32).cpu().numpy()


@pytest.mark.parametrize("name", sorted(CASES))
def test_step_replays_from_a_hip_graph(name):
    import torch
    import discrete_diffusion_decoding_dg_amd as dg
    spec = dict(CASES[name])
    cfg = get_config(spec.pop("base"), **spec)
    inp = make_inputs(cfg)
    m = GpuModel(cfg, inp)
    x = torch.from_numpy(inp["x"]).cuda()
    z, Kp, Vp = (to_dev(inp, n, cfg) for n in ["z", "K_pre", "V_pre"])
    t = np.linspace(1.0, 0.3, cfg.B).astype(np.float32)
    dt = float(np.float32(1.0 / cfg.steps))
    seed = 11
    print(f"[gpu] graph step {name} B={cfg.B} C={cfg.C} d={cfg.d} V={cfg.V}", flush=True)

    eager = _outputs(cfg)
    dg.dg_denoise_step(m.model, x, z, Kp, Vp, t, dt, seed, *eager)
    torch.cuda.synchronize()
    want = _host(eager, cfg)

    graph_out = _outputs(cfg)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):   # one call on a side stream before capture
        dg.dg_denoise_step(m.model, x, z, Kp, Vp, t, dt, seed, *graph_out)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):       # captures on torch's capture stream
        dg.dg_denoise_step(m.model, x, z, Kp, Vp, t, dt, seed, *graph_out)
    for rep in range(3):
        x_g, z_g, lse_g = graph_out
        x_g.fill_(-7)
        z_g.fill_(3.0)
        lse_g.fill_(-1.0)
        noise = torch.randn(4096, device="cuda")
        float(noise.square().sum())   # unrelated eager work, synchronised
        g.replay()
        torch.cuda.synchronize()
        got = _host(graph_out, cfg)
        for what, a, b in zip(("tokens", "z", "lse"), got, want):
            assert np.array_equal(a, b), f"{name}: replay {rep}: {what} differs from the eager step"
    del g
    m.close()
