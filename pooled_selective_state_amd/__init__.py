"""MI355X (gfx950) pooled bidirectional selective-scan layer of FastVim.

The layer runs in hand-written HIP kernels behind the C ABI declared in
``include/fastvim.h``; ``binding`` is its ctypes front end.
"""
from .binding import (  # noqa: F401
    BF16, F32, POOL_COLS, POOL_NONE_COLMAJOR, POOL_NONE_ROWMAJOR, POOL_ROWS,
    EXPORT_BAD_TOKENS, EXPORT_ROWS, EXPORT_S_BWD, EXPORT_S_FWD, EXPORT_STATUS, EXPORT_U, EXPORT_XDBL, FLAG_CONV, FLAG_FUSED, FLAG_POST_NORM, FLAG_STAGED,
    CONV_TAPS, FLAG_CHECK_IDX, FLAG_LOCAL_BWD, FLAG_POOL_SCALE, LOCAL_WINDOW, MAX_BWD_GROUPS, NO_WORKSPACE,
    TUNING_POLL1, SCAN_OUT_AUTO, SCAN_OUT_ONE, SCAN_OUT_TWO,
    STAGE_EPILOGUE, STAGE_POOL, STAGE_PROJ, STAGE_ROWS, STAGE_SCAN,
    BwdCall, FastVimError, SSMCall, bwd_workspace_bytes, calib_copy, check_device_error, lib, make_dims, ssm_bwd,
    ssm_fwd, ssm_fwd_stages, tuning_bwd_groups, tuning_lags, tuning_scan_out,
    workspace_bytes,
)
from .autograd import pooled_ssm  # noqa: F401,E402
