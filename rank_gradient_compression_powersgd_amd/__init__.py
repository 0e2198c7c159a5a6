"""MI355X-native PowerSGD gradient compression (the data-parallel hot path of DALL·E training).

The PowerSGD step runs in hand-written gfx950 HIP kernels inside libpsgd.so (C ABI:
include/psgd.h). This package is the thin Python binding over it:
  * binding  - ctypes wrappers with the ABI's names (psgd_create, psgd_compress, ...);
  * group    - a convenience holder of one group of gradient matrices and their state.
"""
from .binding import (  # noqa: F401
    LIB_PATH, PROFILE_SLOTS, PSGD_BF16, PSGD_F16, PSGD_F32, PsgdError, load_library,
    make_adam_matrix, make_adam_tensor, make_matrix, psgd_adam_attach, psgd_adam_prepare,
    psgd_adam_update, psgd_decompress_adam, psgd_block_grad_enter, psgd_block_grad_exit, psgd_block_grad_exit_enter,
    psgd_check_finite, psgd_compress, psgd_compress_p, psgd_compress_q,
    psgd_create, psgd_debug_buffer, psgd_decompress_update, psgd_destroy, psgd_factor_buffer,
    psgd_last_error, psgd_orthogonalize, psgd_plan_counters, psgd_plan_create, psgd_plan_destroy,
    psgd_profile_events, psgd_refresh_q, psgd_reset_errors, psgd_step_noalloc, psgd_version,
)
from .group import PowerSGDGroup  # noqa: F401
