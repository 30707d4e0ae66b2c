"""Decoupled sparse attention for video DiTs on MI355X (gfx950).

The computation lives in a HIP library (lib/libdecoupattn.so, C ABI in
include/decoupattn.h); this package holds its sources (csrc/), the in-tree build
(build.py) and a ctypes binding (binding.py) with the same entry-point names.
"""
from .binding import (  # noqa: F401
    DA_OK, DA_ERR_INVALID_ARGUMENT, DA_ERR_UNSUPPORTED, DA_ERR_OUT_OF_MEMORY, DA_ERR_DEVICE,
    DA_DTYPE_F32, DA_DTYPE_BF16, EXPORTED, LIB_PATH, DAError, Plan, da_desc, make_desc,
    da_forward, da_forward_var, da_plan_create, da_plan_destroy, da_reassign, da_reassign_var,
    da_reassign_noalloc,
    da_status_str, da_validate_desc, da_version,
)
