"""MI355X-native block-canvas denoising step (DiffusionGemma-style discrete
diffusion decoding), as hand-written gfx950 HIP kernels behind a C ABI.

The binding in `_lib` marshals arguments only; every step of the path runs in
libdg.so. Importing the binding fails loudly when the library is not built.
"""
from ._lib import (DG_DTYPE_BF16, DG_DTYPE_F32, DG_SCHEDULE_COSINE, DG_SCHEDULE_LINEAR,
                   DgError, Model, dg_corrupt, dg_corrupt_batch, dg_create, dg_denoise_step,
                   dg_denoise_step_taps, dg_denoise_step_entropy, dg_denoise_step_static,
                   dg_destroy, dg_generate_canvas,
                   dg_generate_canvas_entropy, dg_last_error, dg_set_ffw, dg_ffw,
                   dg_encode_kv, dg_generate_blocks, dg_generate_blocks_entropy, dg_set_stack,
                   dg_profile_enable, dg_profile_read,
                   dg_status_string, dg_workspace_bytes, library_path, load_library)

__all__ = ["DG_DTYPE_BF16", "DG_DTYPE_F32", "DG_SCHEDULE_COSINE", "DG_SCHEDULE_LINEAR", "DgError",
           "Model", "dg_corrupt", "dg_corrupt_batch", "dg_create", "dg_denoise_step",
           "dg_denoise_step_taps", "dg_denoise_step_entropy", "dg_denoise_step_static", "dg_destroy",
           "dg_generate_canvas",
           "dg_generate_canvas_entropy", "dg_last_error", "dg_set_ffw", "dg_ffw",
           "dg_encode_kv", "dg_generate_blocks", "dg_generate_blocks_entropy", "dg_set_stack",
           "dg_profile_enable", "dg_profile_read",
           "dg_status_string", "dg_workspace_bytes", "library_path", "load_library"]
