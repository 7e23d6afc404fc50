"""C-ABI contract checks that need no GPU: the library loads, exports every
function include/dg.h declares, and rejects bad arguments on the host before
any launch."""
import ctypes
import os
import re

import pytest

import discrete_diffusion_decoding_dg_amd as dg
from discrete_diffusion_decoding_dg_amd import _lib
from discrete_diffusion_decoding_dg_amd._lib import make_config

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared():
    with open(os.path.join(ROOT, "include", "dg.h")) as f:
        text = f.read()
    return sorted(set(re.findall(r"\b(dg_[a-z0-9_]+)\s*\(", text)))


def test_library_exports_every_declared_function():
    lib = _lib.load_library()
    names = _declared()
    assert "dg_denoise_step" in names and "dg_generate_canvas" in names and "dg_corrupt" in names
    for n in names:
        assert hasattr(lib, n), f"{n} declared in dg.h but not exported"
    assert set(names) == set(_lib.EXPORTS)


def _cfg(**kw):
    base = dict(B=1, C=256, P=512, d=2048, n_q_heads=16, n_kv_heads=8, head_dim=128, V=32768,
                dtype=dg.DG_DTYPE_BF16, schedule=dg.DG_SCHEDULE_COSINE)
    base.update(kw)
    return make_config(**base)


def test_valid_configs_report_workspace():
    for kw in [{}, dict(P=32768), dict(d=2816, head_dim=176, V=262144, P=2048),
               dict(B=32, P=4096, V=131072, schedule=dg.DG_SCHEDULE_LINEAR),
               dict(B=1, C=16, P=8, d=32, n_q_heads=2, n_kv_heads=2, head_dim=16, V=64,
                    dtype=dg.DG_DTYPE_F32, schedule=dg.DG_SCHEDULE_LINEAR)]:
        assert dg.dg_workspace_bytes(_cfg(**kw)) > 0


@pytest.mark.parametrize("kw,status", [
    (dict(B=0), _lib.DG_ERR_INVALID_ARG),
    (dict(C=-1), _lib.DG_ERR_INVALID_ARG),
    (dict(P=-1), _lib.DG_ERR_INVALID_ARG),
    (dict(V=1), _lib.DG_ERR_INVALID_ARG),
    (dict(n_q_heads=12, n_kv_heads=8), _lib.DG_ERR_INVALID_ARG),
    (dict(dtype=7), _lib.DG_ERR_INVALID_ARG),
    (dict(schedule=5), _lib.DG_ERR_INVALID_ARG),
    (dict(B=1 << 20, C=1 << 12), _lib.DG_ERR_INVALID_ARG),        # B*C*d overflows
    (dict(head_dim=96, n_q_heads=16), _lib.DG_ERR_UNSUPPORTED),
    (dict(d=768), _lib.DG_ERR_UNSUPPORTED),
    (dict(V=32760), _lib.DG_ERR_UNSUPPORTED),
    (dict(dtype=dg.DG_DTYPE_F32, d=8192), _lib.DG_ERR_UNSUPPORTED),
    (dict(dtype=dg.DG_DTYPE_F32, P=20000), _lib.DG_ERR_UNSUPPORTED),
])
def test_invalid_configs_are_rejected(kw, status):
    with pytest.raises(dg.DgError) as e:
        dg.dg_workspace_bytes(_cfg(**kw))
    assert e.value.status == status
    assert dg.dg_last_error()


def test_create_rejects_null_and_misaligned_weights():
    lib = _lib.load_library()
    cfg = _cfg()
    h = ctypes.c_void_p()
    w = _lib.dg_weights(None, 16, 16, 16, 16)
    assert lib.dg_create(ctypes.byref(cfg), ctypes.byref(w), ctypes.byref(h)) == _lib.DG_ERR_INVALID_ARG
    w = _lib.dg_weights(18, 16, 16, 16, 16)
    assert lib.dg_create(ctypes.byref(cfg), ctypes.byref(w), ctypes.byref(h)) == _lib.DG_ERR_INVALID_ARG
    assert "aligned" in dg.dg_last_error()
    assert lib.dg_create(None, ctypes.byref(w), ctypes.byref(h)) == _lib.DG_ERR_INVALID_ARG
    assert h.value is None


def test_calls_reject_null_model_and_pointers():
    lib = _lib.load_library()
    t = (ctypes.c_float * 1)(0.5)
    assert lib.dg_denoise_step(None, 16, 16, 16, 16, t, ctypes.c_float(0.1), 0, 32, 32, None, None,
                               None) == _lib.DG_ERR_INVALID_ARG
    assert lib.dg_generate_canvas(None, 16, 16, 12, 0, 32, None, None) == _lib.DG_ERR_INVALID_ARG
    k = (ctypes.c_float * 1)(0.5)
    assert lib.dg_corrupt(None, 16, k, 0, 32, None) == _lib.DG_ERR_INVALID_ARG
    assert lib.dg_corrupt_batch(None, 16, 1, 1, 2, 0, 32, None) == _lib.DG_ERR_INVALID_ARG
    assert lib.dg_corrupt_batch(16, 16, -1, 1, 2, 0, 32, None) == _lib.DG_ERR_INVALID_ARG
    # partially overlapping in/out ranges are rejected (exact in-place is allowed)
    assert lib.dg_corrupt_batch(1024, 16, 1, 64, 2, 0, 1028, None) == _lib.DG_ERR_INVALID_ARG
    assert lib.dg_set_ffw(None, 64, 16, 16, 16) == _lib.DG_ERR_INVALID_ARG
    assert lib.dg_encode_kv(None, 16, 4, 0, 32, 32, None) == _lib.DG_ERR_INVALID_ARG
    assert lib.dg_set_stack(None, 1, 64, None, None) == _lib.DG_ERR_INVALID_ARG
    assert lib.dg_set_stack_moe(None, 1, 128, 4, 2, None, None, None) == _lib.DG_ERR_INVALID_ARG
    assert lib.dg_generate_blocks(None, 32, 32, 0, 1, 4, 0, 16, None) == _lib.DG_ERR_INVALID_ARG
    assert lib.dg_generate_blocks_entropy(None, 32, 32, 0, 1, 4, 0, ctypes.c_float(1.0),
                                          ctypes.c_float(1.0), 16, 16, None) == _lib.DG_ERR_INVALID_ARG
    assert lib.dg_ffw(None, 16, 32, None) == _lib.DG_ERR_INVALID_ARG
    assert lib.dg_profile_enable(None, 1) == _lib.DG_ERR_INVALID_ARG
    assert lib.dg_profile_read(None, None) == _lib.DG_ERR_INVALID_ARG
    assert lib.dg_destroy(None) == _lib.DG_OK


def test_status_strings():
    assert dg.dg_status_string(0) == "DG_OK"
    assert dg.dg_status_string(2) == "DG_ERR_UNSUPPORTED"
    assert dg.dg_status_string(99) == "DG_ERR_UNKNOWN"


def test_single_hip_runtime_in_process():
    """libdg must resolve libamdhip64 to the copy torch loaded (one runtime)."""
    _lib.load_library()
    maps = open("/proc/self/maps").read()
    paths = {line.split()[-1] for line in maps.splitlines() if "libamdhip64" in line}
    assert len(paths) == 1, paths


def test_static_step_rejects_on_the_host():
    """dg_denoise_step_static checks its config, weights and the static scratch
    limit before any HIP call (no device is touched here)."""
    lib = _lib.load_library()
    t = (ctypes.c_float * 256)(*([0.5] * 256))
    w = _lib.dg_weights(16, 16, 16, 16, 16)

    def call(cfg, w=w, lse=None, p0=None):
        return lib.dg_denoise_step_static(ctypes.byref(cfg), ctypes.byref(w), 32, 64, 64, 64, t,
                                          ctypes.c_float(0.1), 0, 96, 128, lse, p0, None)
    # the standard canvas needs more workspace than the static scratch holds
    assert call(_cfg()) == _lib.DG_ERR_UNSUPPORTED
    assert "static" in dg.dg_last_error()
    assert call(_cfg(B=257, C=16, P=8, d=256, n_q_heads=4, n_kv_heads=2, head_dim=64,
                     V=1024)) == _lib.DG_ERR_UNSUPPORTED
    assert "B <= 256" in dg.dg_last_error()
    assert call(_cfg(B=0)) == _lib.DG_ERR_INVALID_ARG
    assert call(_cfg(), w=_lib.dg_weights(None, 16, 16, 16, 16)) == _lib.DG_ERR_INVALID_ARG
    assert call(_cfg(), w=_lib.dg_weights(18, 16, 16, 16, 16)) == _lib.DG_ERR_INVALID_ARG
    assert call(_cfg(), p0=256) == _lib.DG_ERR_INVALID_ARG
    assert lib.dg_denoise_step_static(None, ctypes.byref(w), 32, 64, 64, 64, t, ctypes.c_float(0.1), 0,
                                      96, 128, None, None, None) == _lib.DG_ERR_INVALID_ARG
