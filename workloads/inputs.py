"""Seeded input generation.

One PCG64 stream per tensor, spawned from SeedSequence(cfg.seed) in a fixed
order, so any tensor can be regenerated alone. Values for bf16 workloads are
drawn in float32 and rounded to bfloat16 (round to nearest, ties to even);
both sides then consume the same bits.
"""
import numpy as np

# New streams go at the end: child i of the spawn does not depend on the count.
STREAMS = ["E", "Wq", "Wk", "Wv", "Wo", "K_pre", "V_pre", "x", "t", "z_mask", "z",
           "W_gate", "W_up", "W_down",
           "S_Wq", "S_Wk", "S_Wv", "S_Wo", "S_g_attn", "S_g_mlp", "S_g_final", "S_W_gate", "S_W_up",
           "S_W_down", "S_K_pre", "S_V_pre", "S_W_router"]


def bf16_bits_from_f32(a):
    """float32 array -> uint16 bfloat16 bit patterns, round to nearest even (finite inputs)."""
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32)
    bias = ((u >> 16) & 1) + np.uint32(0x7FFF)
    return ((u + bias) >> 16).astype(np.uint16)


def f32_from_bf16_bits(b):
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def _rng(cfg, name):
    ss = np.random.SeedSequence(cfg.seed).spawn(len(STREAMS))[STREAMS.index(name)]
    return np.random.Generator(np.random.PCG64(ss))


def _normal(cfg, name, shape, std):
    a = _rng(cfg, name).standard_normal(size=shape, dtype=np.float32)
    a *= np.float32(std)
    return a


class Inputs(dict):
    """Dict of named arrays. For bf16 configs each float tensor is stored as
    float32 values that are exactly bf16-representable, plus `<name>_bits`."""


def make_inputs(cfg, which=None):
    """Return the seeded inputs of `cfg`.

    Layouts (row-major): E [V, d]; Wq [Hq*hd, d]; Wk, Wv [Hkv*hd, d];
    Wo [d, Hq*hd]; K_pre, V_pre [B, Hkv, P, hd]; x [B, C] int32;
    z [B, C, d]; t [B] float32 (per-canvas t when the config asks for it);
    with a self-conditioning block of width F: W_gate, W_up [F, d], W_down [d, F];
    with a decoder stack of L layers and MLP width F: S_Wq [L, Hq*hd, d],
    S_Wk, S_Wv [L, Hkv*hd, d], S_Wo [L, d, Hq*hd], S_g_attn, S_g_mlp [L, d],
    S_g_final [d], S_W_gate, S_W_up [L, F, d], S_W_down [L, d, F],
    S_K_pre, S_V_pre [L, B, Hkv, P, hd]; with X experts per layer the MLP
    weights are expert-major (S_W_gate, S_W_up [L, X, F, d], S_W_down
    [L, X, d, F]) and S_W_router is [L, X, d]. Norm gains ~ N(1, 0.1^2); the
    stack's matrices ~ N(0, w_std^2).
    """
    names = which or (["E", "Wq", "Wk", "Wv", "Wo", "K_pre", "V_pre", "x", "t", "z"] +
                      (["W_gate", "W_up", "W_down"] if cfg.ffw_hidden else []) +
                      (STREAMS[14:26] if cfg.n_layers else []) +
                      (["S_W_router"] if cfg.n_layers and cfg.n_experts else []))
    out = Inputs()
    hq, hkv, hd = cfg.n_q_heads * cfg.head_dim, cfg.n_kv_heads * cfg.head_dim, cfg.head_dim
    shapes = {
        "E": ((cfg.V, cfg.d), cfg.w_std),
        "Wq": ((hq, cfg.d), cfg.w_std),
        "Wk": ((hkv, cfg.d), cfg.w_std),
        "Wv": ((hkv, cfg.d), cfg.w_std),
        "Wo": ((cfg.d, hq), cfg.w_std),
        "K_pre": ((cfg.B, cfg.n_kv_heads, cfg.P, hd), cfg.kv_std),
        "V_pre": ((cfg.B, cfg.n_kv_heads, cfg.P, hd), cfg.kv_std),
    }
    if cfg.n_layers:
        L, Fm = cfg.n_layers, cfg.mlp_hidden
        shapes.update({
            "S_Wq": ((L, hq, cfg.d), cfg.w_std), "S_Wk": ((L, hkv, cfg.d), cfg.w_std),
            "S_Wv": ((L, hkv, cfg.d), cfg.w_std), "S_Wo": ((L, cfg.d, hq), cfg.w_std),
            "S_W_gate": ((L, Fm, cfg.d), cfg.w_std), "S_W_up": ((L, Fm, cfg.d), cfg.w_std),
            "S_W_down": ((L, cfg.d, Fm), cfg.w_std),
            "S_W_router": ((L, max(1, cfg.n_experts), cfg.d), cfg.w_std),
            "S_K_pre": ((L, cfg.B, cfg.n_kv_heads, cfg.P, hd), cfg.kv_std),
            "S_V_pre": ((L, cfg.B, cfg.n_kv_heads, cfg.P, hd), cfg.kv_std)})
        if cfg.n_experts:
            X = cfg.n_experts
            shapes.update({"S_W_gate": ((L, X, Fm, cfg.d), cfg.w_std), "S_W_up": ((L, X, Fm, cfg.d), cfg.w_std),
                           "S_W_down": ((L, X, cfg.d, Fm), cfg.w_std)})
    gains = {"S_g_attn": (cfg.n_layers, cfg.d), "S_g_mlp": (cfg.n_layers, cfg.d), "S_g_final": (cfg.d,)}
    if cfg.ffw_hidden:
        F = cfg.ffw_hidden
        shapes["W_gate"] = ((F, cfg.d), cfg.ffw_gain / np.sqrt(cfg.d))
        shapes["W_up"] = ((F, cfg.d), cfg.ffw_gain / np.sqrt(cfg.d))
        shapes["W_down"] = ((cfg.d, F), 1.0 / np.sqrt(F))
    for n in names:
        if n in gains:
            a = np.float32(1.0) + _normal(cfg, n, gains[n], 0.1)
            if cfg.dtype == "bf16":
                bits = bf16_bits_from_f32(a)
                out[n + "_bits"] = bits
                a = f32_from_bf16_bits(bits).reshape(gains[n])
            out[n] = a
        elif n in shapes:
            shape, std = shapes[n]
            a = _normal(cfg, n, shape, std)
            if cfg.dtype == "bf16":
                bits = bf16_bits_from_f32(a)
                out[n + "_bits"] = bits
                a = f32_from_bf16_bits(bits).reshape(shape)
            out[n] = a
        elif n == "x":
            out["x"] = _rng(cfg, "x").integers(0, cfg.V, size=(cfg.B, cfg.C), dtype=np.int64).astype(np.int32)
        elif n == "t":
            if cfg.per_canvas_t:
                # uniform on (0, 1]: 1 - U[0, 1)
                u = _rng(cfg, "t").random(cfg.B)
                out["t"] = (1.0 - u).astype(np.float32)
            else:
                out["t"] = np.ones(cfg.B, dtype=np.float32)
        elif n == "z":
            # Self-conditioning input. Zero everywhere unless the config zeroes a
            # seeded half: then the other half carries a synthetic previous-pass
            # signal drawn at the scale of an embedding row.
            z = np.zeros((cfg.B, cfg.C, cfg.d), dtype=np.float32)
            if cfg.zero_z_half:
                keep = np.zeros(cfg.B, dtype=bool)
                keep[_rng(cfg, "z_mask").permutation(cfg.B)[: cfg.B // 2]] = True
                zz = _normal(cfg, "z", (int(keep.sum()), cfg.C, cfg.d), cfg.w_std)
                z[keep] = zz
                out["z_nonzero"] = keep
            if cfg.dtype == "bf16":
                bits = bf16_bits_from_f32(z)
                out["z_bits"] = bits
                z = f32_from_bf16_bits(bits).reshape(z.shape)
            out["z"] = z
        else:
            raise KeyError(n)
    return out
