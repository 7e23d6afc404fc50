"""Seeded synthetic inputs drawn on the GPU, for timing runs.

Same shapes and distributions as `inputs.make_inputs` (weights and E ~
N(0, w_std^2), KV cache ~ N(0, kv_std^2), tokens uniform over [0, V), z = 0
or a seeded half of the canvases at N(0, w_std^2), per-canvas t ~ U(0, 1]
where the workload asks for it), but drawn by torch's device generator, so a
multi-gigabyte workload is ready in milliseconds. The values differ from the
host generator's (another generator); the timing does not depend on them.
Holds none of the method's arithmetic.
"""
import numpy as np


def make_device_inputs(cfg, seed=0, device="cuda"):
    """Returns a dict of device tensors: E, Wq, Wk, Wv, Wo, K_pre, V_pre, x, z
    (bf16 or fp32 as the workload's dtype) and host arrays t [B] float32 and,
    when a half of the canvases carries z, z_nonzero [B] bool."""
    import torch
    g = torch.Generator(device=device)
    g.manual_seed(int(seed))
    dt = torch.bfloat16 if cfg.dtype == "bf16" else torch.float32
    hq, hkv, hd = cfg.n_q_heads * cfg.head_dim, cfg.n_kv_heads * cfg.head_dim, cfg.head_dim

    def normal(shape, std):
        a = torch.randn(shape, generator=g, device=device, dtype=torch.float32)
        a.mul_(float(std))
        return a.to(dt)

    out = {
        "E": normal((cfg.V, cfg.d), cfg.w_std),
        "Wq": normal((hq, cfg.d), cfg.w_std),
        "Wk": normal((hkv, cfg.d), cfg.w_std),
        "Wv": normal((hkv, cfg.d), cfg.w_std),
        "Wo": normal((cfg.d, hq), cfg.w_std),
        "K_pre": normal((cfg.B, cfg.n_kv_heads, cfg.P, hd), cfg.kv_std),
        "V_pre": normal((cfg.B, cfg.n_kv_heads, cfg.P, hd), cfg.kv_std),
        "x": torch.randint(0, cfg.V, (cfg.B, cfg.C), generator=g, device=device, dtype=torch.int32),
    }
    z = torch.zeros((cfg.B, cfg.C, cfg.d), device=device, dtype=dt)
    rng = np.random.default_rng(int(seed))
    if cfg.zero_z_half:
        keep = np.zeros(cfg.B, dtype=bool)
        keep[rng.permutation(cfg.B)[: cfg.B // 2]] = True
        idx = torch.from_numpy(np.flatnonzero(keep)).to(device)
        z[idx] = normal((int(keep.sum()), cfg.C, cfg.d), cfg.w_std)
        out["z_nonzero"] = keep
    out["z"] = z
    if cfg.per_canvas_t:
        out["t"] = (1.0 - rng.random(cfg.B)).astype(np.float32)
    else:
        out["t"] = np.ones(cfg.B, dtype=np.float32)
    return out


def to_host_f32(t):
    """Device tensor -> host float32 (or int32) numpy array (bf16 values are exact in float32)."""
    import torch
    if t.dtype in (torch.bfloat16, torch.float16):
        t = t.float()
    return t.cpu().numpy()
