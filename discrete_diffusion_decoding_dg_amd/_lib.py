"""ctypes binding of libdg (include/dg.h). Argument marshalling only.

Tensors are torch tensors on the GPU; their data pointers cross the ABI. A
missing library raises at import time: there is no fallback path.
"""
import ctypes
import os

DG_OK, DG_ERR_INVALID_ARG, DG_ERR_UNSUPPORTED, DG_ERR_HIP, DG_ERR_OOM = 0, 1, 2, 3, 4
DG_DTYPE_F32, DG_DTYPE_BF16 = 0, 1
DG_SCHEDULE_LINEAR, DG_SCHEDULE_COSINE = 0, 1

_HERE = os.path.dirname(os.path.abspath(__file__))


def library_path():
    return os.environ.get("DG_LIBRARY", os.path.join(_HERE, "libdg.so"))


class dg_config(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in
                ["B", "C", "P", "d", "n_q_heads", "n_kv_heads", "head_dim", "V", "dtype", "schedule"]]


class dg_weights(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in ["E", "Wq", "Wk", "Wv", "Wo"]]


class dg_taps(ctypes.Structure):
    _fields_ = [("h0", ctypes.c_void_p), ("q", ctypes.c_void_p), ("k", ctypes.c_void_p),
                ("v", ctypes.c_void_p), ("o", ctypes.c_void_p), ("h1", ctypes.c_void_p),
                ("lse", ctypes.c_void_p), ("p0", ctypes.c_void_p), ("best", ctypes.c_void_p),
                ("p0E", ctypes.c_void_p)]


NUM_STAGES = 10
STAGES = ["embed", "qkv", "attention", "oproj", "lmhead", "combine", "corrupt", "ffw", "encode",
          "stack_mlp"]


class dg_layer_weights(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in
                ["Wq", "Wk", "Wv", "Wo", "g_attn", "g_mlp", "W_gate", "W_up", "W_down"]]


class dg_profile(ctypes.Structure):
    _fields_ = [("ms", ctypes.c_double * NUM_STAGES), ("count", ctypes.c_int64 * NUM_STAGES)]


EXPORTS = ["dg_create", "dg_destroy", "dg_workspace_bytes", "dg_corrupt", "dg_corrupt_batch",
           "dg_denoise_step", "dg_denoise_step_taps", "dg_denoise_step_static", "dg_generate_canvas",
           "dg_denoise_step_entropy", "dg_generate_canvas_entropy", "dg_set_ffw", "dg_ffw",
           "dg_encode_kv", "dg_generate_blocks", "dg_generate_blocks_entropy", "dg_set_stack",
           "dg_set_stack_moe",
           "dg_profile_enable",
           "dg_profile_read", "dg_status_string", "dg_last_error"]

_lib = None


def load_library():
    global _lib
    if _lib is not None:
        return _lib
    # One HIP runtime per process: torch bundles its own libamdhip64 (same
    # SONAME as the system one). Importing torch first makes libdg bind to the
    # runtime torch already loaded, so device pointers and stream handles
    # coming from torch are valid in libdg. Loading libdg first would pull in
    # the system runtime and torch would then load a second, separate one.
    import torch  # noqa: F401
    path = library_path()
    if not os.path.exists(path):
        raise ImportError(f"libdg.so not found at {path}: build it with "
                          "`python -m discrete_diffusion_decoding_dg_amd.build`")
    lib = ctypes.CDLL(path)
    vp, u64, i32, f32 = ctypes.c_void_p, ctypes.c_uint64, ctypes.c_int32, ctypes.c_float
    lib.dg_create.argtypes = [ctypes.POINTER(dg_config), ctypes.POINTER(dg_weights), ctypes.POINTER(vp)]
    lib.dg_destroy.argtypes = [vp]
    lib.dg_workspace_bytes.argtypes = [ctypes.POINTER(dg_config), ctypes.POINTER(ctypes.c_size_t)]
    lib.dg_corrupt.argtypes = [vp, vp, ctypes.POINTER(f32), u64, vp, vp]
    lib.dg_corrupt_batch.argtypes = [vp, vp, i32, i32, i32, u64, vp, vp]
    lib.dg_denoise_step.argtypes = [vp, vp, vp, vp, vp, ctypes.POINTER(f32), f32, u64, vp, vp, vp, vp, vp]
    lib.dg_denoise_step_taps.argtypes = [vp, vp, vp, vp, vp, ctypes.POINTER(f32), f32, u64, vp, vp,
                                         ctypes.POINTER(dg_taps), vp]
    lib.dg_denoise_step_static.argtypes = [ctypes.POINTER(dg_config), ctypes.POINTER(dg_weights), vp, vp,
                                           vp, vp, ctypes.POINTER(f32), f32, u64, vp, vp, vp, vp, vp]
    lib.dg_generate_canvas.argtypes = [vp, vp, vp, i32, u64, vp, vp, vp]
    lib.dg_denoise_step_entropy.argtypes = [vp, vp, vp, vp, vp, ctypes.POINTER(f32), u64, f32, f32,
                                            vp, vp, vp, vp, vp, vp, vp]
    lib.dg_generate_canvas_entropy.argtypes = [vp, vp, vp, i32, u64, f32, f32, vp, vp, vp, vp]
    lib.dg_encode_kv.argtypes = [vp, vp, i32, i32, vp, vp, vp]
    lib.dg_generate_blocks.argtypes = [vp, vp, vp, i32, i32, i32, u64, vp, vp]
    lib.dg_generate_blocks_entropy.argtypes = [vp, vp, vp, i32, i32, i32, u64, f32, f32, vp, vp, vp]
    lib.dg_set_ffw.argtypes = [vp, i32, vp, vp, vp]
    lib.dg_set_stack.argtypes = [vp, i32, i32, ctypes.POINTER(dg_layer_weights), vp]
    lib.dg_set_stack_moe.argtypes = [vp, i32, i32, i32, i32, ctypes.POINTER(dg_layer_weights),
                                     ctypes.POINTER(vp), vp]
    lib.dg_ffw.argtypes = [vp, vp, vp, vp]
    lib.dg_profile_enable.argtypes = [vp, ctypes.c_int]
    lib.dg_profile_read.argtypes = [vp, ctypes.POINTER(dg_profile)]
    lib.dg_status_string.argtypes = [ctypes.c_int]
    lib.dg_status_string.restype = ctypes.c_char_p
    lib.dg_last_error.restype = ctypes.c_char_p
    for n in EXPORTS:
        if n not in ("dg_status_string", "dg_last_error"):
            getattr(lib, n).restype = ctypes.c_int
    _lib = lib
    return lib


class DgError(RuntimeError):
    def __init__(self, status, message):
        super().__init__(f"{dg_status_string(status)}: {message}")
        self.status = status


def dg_status_string(status):
    return load_library().dg_status_string(int(status)).decode()


def dg_last_error():
    return load_library().dg_last_error().decode()


def _check(status):
    if status != DG_OK:
        raise DgError(status, dg_last_error())


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    if stream is None:
        import torch
        return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    if isinstance(stream, int):
        return ctypes.c_void_p(stream)
    return ctypes.c_void_p(stream.cuda_stream)


def _floats(values):
    vals = [float(v) for v in values]
    return (ctypes.c_float * max(1, len(vals)))(*vals)


def make_config(B, C, P, d, n_q_heads, n_kv_heads, head_dim, V, dtype, schedule):
    return dg_config(B, C, P, d, n_q_heads, n_kv_heads, head_dim, V, dtype, schedule)


class Model:
    """Owns a dg_model handle and keeps the weight tensors alive."""

    def __init__(self, handle, cfg, weights):
        self.handle = handle
        self.cfg = cfg
        self._weights = weights

    def close(self):
        if self.handle:
            _check(load_library().dg_destroy(self.handle))
            self.handle = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


def dg_workspace_bytes(cfg):
    n = ctypes.c_size_t(0)
    _check(load_library().dg_workspace_bytes(ctypes.byref(cfg), ctypes.byref(n)))
    return n.value


def dg_create(cfg, E, Wq, Wk, Wv, Wo):
    w = dg_weights(*[t.data_ptr() if t is not None else None for t in (E, Wq, Wk, Wv, Wo)])
    h = ctypes.c_void_p()
    _check(load_library().dg_create(ctypes.byref(cfg), ctypes.byref(w), ctypes.byref(h)))
    return Model(h, cfg, (E, Wq, Wk, Wv, Wo))


def dg_destroy(model):
    model.close()


def dg_corrupt(model, x0, kappa, seed, xt_out, stream=None):
    _check(load_library().dg_corrupt(model.handle, _ptr(x0), _floats(kappa), int(seed),
                                     _ptr(xt_out), _stream(stream)))


def dg_corrupt_batch(x0, kappa_dev, B, C, V, seed, xt_out, stream=None):
    _check(load_library().dg_corrupt_batch(_ptr(x0), _ptr(kappa_dev), int(B), int(C), int(V),
                                           int(seed), _ptr(xt_out), _stream(stream)))


def dg_denoise_step(model, x_t, z_t, K_pre, V_pre, t, dt, seed, x_out, z_out, lse_out=None,
                    p0_out=None, stream=None):
    _check(load_library().dg_denoise_step(model.handle, _ptr(x_t), _ptr(z_t), _ptr(K_pre),
                                          _ptr(V_pre), _floats(t), float(dt), int(seed),
                                          _ptr(x_out), _ptr(z_out), _ptr(lse_out), _ptr(p0_out),
                                          _stream(stream)))


def dg_denoise_step_taps(model, x_t, z_t, K_pre, V_pre, t, dt, seed, x_out, z_out, taps=None,
                         stream=None):
    """`taps` maps any of h0, q, k, v, o, h1, lse, p0, best, p0E to output tensors."""
    tp = None
    if taps:
        tp = dg_taps(**{k: (v.data_ptr() if v is not None else None) for k, v in taps.items()})
    _check(load_library().dg_denoise_step_taps(model.handle, _ptr(x_t), _ptr(z_t), _ptr(K_pre),
                                               _ptr(V_pre), _floats(t), float(dt), int(seed),
                                               _ptr(x_out), _ptr(z_out),
                                               ctypes.byref(tp) if tp is not None else None,
                                               _stream(stream)))


def dg_denoise_step_static(cfg, E, Wq, Wk, Wv, Wo, x_t, z_t, K_pre, V_pre, t, dt, seed, x_out, z_out,
                           lse_out=None, p0_out=None, stream=None):
    """dg_denoise_step without a model and without allocation (static scratch)."""
    w = dg_weights(*[t_.data_ptr() if t_ is not None else None for t_ in (E, Wq, Wk, Wv, Wo)])
    _check(load_library().dg_denoise_step_static(ctypes.byref(cfg), ctypes.byref(w), _ptr(x_t), _ptr(z_t),
                                                 _ptr(K_pre), _ptr(V_pre), _floats(t), float(dt),
                                                 int(seed), _ptr(x_out), _ptr(z_out), _ptr(lse_out),
                                                 _ptr(p0_out), _stream(stream)))


def dg_generate_canvas(model, K_pre, V_pre, steps, seed, x_out, z_out=None, stream=None):
    _check(load_library().dg_generate_canvas(model.handle, _ptr(K_pre), _ptr(V_pre), int(steps),
                                             int(seed), _ptr(x_out), _ptr(z_out), _stream(stream)))


def dg_denoise_step_entropy(model, x_t, z_t, K_pre, V_pre, t, seed, eps_accept, eps_stop,
                            det_prev, x_out, z_out, det_out, stop_out, entropy_out=None,
                            stream=None):
    _check(load_library().dg_denoise_step_entropy(model.handle, _ptr(x_t), _ptr(z_t), _ptr(K_pre),
                                                  _ptr(V_pre), _floats(t), int(seed),
                                                  float(eps_accept), float(eps_stop),
                                                  _ptr(det_prev), _ptr(x_out), _ptr(z_out),
                                                  _ptr(det_out), _ptr(entropy_out),
                                                  _ptr(stop_out), _stream(stream)))


def dg_generate_canvas_entropy(model, K_pre, V_pre, max_steps, seed, eps_accept, eps_stop, x_out,
                               steps_out, z_out=None, stream=None):
    _check(load_library().dg_generate_canvas_entropy(model.handle, _ptr(K_pre), _ptr(V_pre),
                                                     int(max_steps), int(seed), float(eps_accept),
                                                     float(eps_stop), _ptr(x_out), _ptr(z_out),
                                                     _ptr(steps_out), _stream(stream)))


def dg_encode_kv(model, tokens, pos, K_cache, V_cache, stream=None):
    """Encoder cache entries of tokens [B, n] into rows [pos, pos + n) of the caches."""
    _check(load_library().dg_encode_kv(model.handle, _ptr(tokens), int(tokens.shape[1]), int(pos),
                                       _ptr(K_cache), _ptr(V_cache), _stream(stream)))


def dg_generate_blocks(model, K_cache, V_cache, P0, n_canvases, steps, seed, x_out, stream=None):
    _check(load_library().dg_generate_blocks(model.handle, _ptr(K_cache), _ptr(V_cache), int(P0),
                                             int(n_canvases), int(steps), int(seed), _ptr(x_out),
                                             _stream(stream)))


def dg_generate_blocks_entropy(model, K_cache, V_cache, P0, n_canvases, max_steps, seed, eps_accept,
                               eps_stop, x_out, steps_out, stream=None):
    _check(load_library().dg_generate_blocks_entropy(model.handle, _ptr(K_cache), _ptr(V_cache), int(P0),
                                                     int(n_canvases), int(max_steps), int(seed),
                                                     float(eps_accept), float(eps_stop), _ptr(x_out),
                                                     _ptr(steps_out), _stream(stream)))


def dg_set_stack(model, layers=None, g_final=None, top_k=0):
    """Attach a decoder stack: `layers` is a list of dicts with tensors Wq, Wk,
    Wv, Wo, g_attn, g_mlp, W_gate, W_up, W_down (and W_router with experts:
    then W_gate/W_up are [X, F, d], W_down [X, d, F], and top_k > 0); no
    layers detach it. The model keeps references to the tensors."""
    if not layers:
        _check(load_library().dg_set_stack(model.handle, 0, 0, None, None))
        model._stack = None
        return
    names = [f[0] for f in dg_layer_weights._fields_]
    arr = (dg_layer_weights * len(layers))(
        *[dg_layer_weights(*[lw[n].data_ptr() for n in names]) for lw in layers])
    if layers[0].get("W_router") is not None:
        X, F = int(layers[0]["W_router"].shape[0]), int(layers[0]["W_gate"].shape[1])
        routers = (ctypes.c_void_p * len(layers))(*[lw["W_router"].data_ptr() for lw in layers])
        _check(load_library().dg_set_stack_moe(model.handle, len(layers), F, X, int(top_k), arr, routers,
                                               _ptr(g_final)))
    else:
        _check(load_library().dg_set_stack(model.handle, len(layers), int(layers[0]["W_gate"].shape[0]),
                                           arr, _ptr(g_final)))
    model._stack = (layers, g_final)


def dg_set_ffw(model, W_gate=None, W_up=None, W_down=None):
    """Attach the gated feed-forward block (W_gate, W_up [F, d], W_down [d, F]);
    no tensors detach it. The model keeps references to the tensors."""
    if W_gate is None:
        _check(load_library().dg_set_ffw(model.handle, 0, None, None, None))
        model._ffw = None
        return
    _check(load_library().dg_set_ffw(model.handle, int(W_gate.shape[0]), _ptr(W_gate), _ptr(W_up),
                                     _ptr(W_down)))
    model._ffw = (W_gate, W_up, W_down)


def dg_ffw(model, u, z_out, stream=None):
    _check(load_library().dg_ffw(model.handle, _ptr(u), _ptr(z_out), _stream(stream)))


def dg_profile_enable(model, stages=None):
    """Time the named stages (all when None; nothing for an empty list)."""
    names = STAGES if stages is None else stages
    mask = 0
    for n in names:
        mask |= 1 << STAGES.index(n)
    _check(load_library().dg_profile_enable(model.handle, mask))


def dg_profile_read(model):
    """Returns {stage: (total_ms, launches)} and clears the recorded events."""
    p = dg_profile()
    _check(load_library().dg_profile_read(model.handle, ctypes.byref(p)))
    return {STAGES[i]: (p.ms[i], int(p.count[i])) for i in range(NUM_STAGES)}


load_library()
