"""GPU check of dg_denoise_step_static, the step without allocation: its
outputs equal dg_denoise_step's (same kernels, same splits, bit for bit) on
two calls in a row, the second with a smaller input, in bf16 and in fp32."""
import numpy as np
import pytest

from tests.dg_harness import act_tensor, config_args, to_dev
from workloads import get_config, make_inputs

pytestmark = pytest.mark.gpu


def _both(cfg, t, seed):
    import torch
    import discrete_diffusion_decoding_dg_amd as dg
    inp = make_inputs(cfg)
    w = {n: to_dev(inp, n, cfg) for n in ["E", "Wq", "Wk", "Wv", "Wo"]}
    z, Kp, Vp = (to_dev(inp, n, cfg) for n in ["z", "K_pre", "V_pre"])
    x = torch.from_numpy(inp["x"]).cuda()
    B, C = cfg.B, cfg.C
    dt = float(np.float32(1.0 / cfg.steps))
    outs = []
    for static in (True, False):
        x_out = torch.full((B, C), -7, dtype=torch.int32, device="cuda")
        z_out = act_tensor((B, C, cfg.d), cfg)
        z_out.fill_(3.0)
        lse = torch.full((B, C), -1.0, dtype=torch.float32, device="cuda")
        print(f"[gpu] {'static' if static else 'model'} step {cfg.name} B={B} C={C} d={cfg.d} "
              f"V={cfg.V} {cfg.dtype}", flush=True)
        if static:
            dg.dg_denoise_step_static(config_args(cfg), w["E"], w["Wq"], w["Wk"], w["Wv"], w["Wo"], x, z,
                                      Kp, Vp, t, dt, seed, x_out, z_out, lse)
        else:
            m = dg.dg_create(config_args(cfg), w["E"], w["Wq"], w["Wk"], w["Wv"], w["Wo"])
            dg.dg_denoise_step(m, x, z, Kp, Vp, t, dt, seed, x_out, z_out, lse)
            torch.cuda.synchronize()
            m.close()
        torch.cuda.synchronize()
        zb = z_out.view(torch.int16) if cfg.dtype == "bf16" else z_out.view(torch.int32)
        outs.append((x_out.cpu().numpy(), zb.cpu().numpy(), lse.view(torch.int32).cpu().numpy()))
    return outs


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_static_step_equals_model_step_twice(dtype):
    if dtype == "bf16":
        big = get_config("c2", B=2, C=64, P=96, d=256, n_q_heads=4, n_kv_heads=2, head_dim=64, V=4096)
        small = big.with_(B=1, C=40, P=100)
    else:
        big = get_config("c1", B=2, C=24)
        small = get_config("c1")
    for cfg, seed in ((big, 5), (small, 6)):
        t = np.linspace(1.0, 0.25, cfg.B).astype(np.float32)
        (xs, zs, ls), (xm, zm, lm) = _both(cfg, t, seed)
        assert np.array_equal(xs, xm), f"{cfg.dtype} B={cfg.B} C={cfg.C}: tokens differ"
        assert np.array_equal(zs, zm), f"{cfg.dtype} B={cfg.B} C={cfg.C}: z differs"
        assert np.array_equal(ls, lm), f"{cfg.dtype} B={cfg.B} C={cfg.C}: lse differs"
        assert (xs >= 0).all() and (xs < cfg.V).all()


def test_static_step_refuses_a_workspace_beyond_the_scratch():
    import torch
    import discrete_diffusion_decoding_dg_amd as dg
    cfg = get_config("c2")
    e = torch.zeros(16, dtype=torch.bfloat16, device="cuda")
    with pytest.raises(dg.DgError) as err:
        dg.dg_denoise_step_static(config_args(cfg), e, e, e, e, e, e, e, e, e, [0.5], 0.1, 0, e, e)
    assert err.value.status == 2 and "static" in str(err.value)
