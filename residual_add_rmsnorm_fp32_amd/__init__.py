"""MI355X-native fused "sum of partials + residual add + RMSNorm (+ fp8 quant)" epilogue.

The computation runs in the HIP library ``libfar.so`` (C ABI in ``include/far.h``);
``binding`` is its ctypes binding, ``workloads`` the seeded synthetic inputs, ``build``
the gfx950 build.
"""

from .binding import (  # noqa: F401
    FAR_DTYPE,
    FAR_FP8_GROUP,
    FAR_MAX_PARTIALS,
    FAR_QUANT,
    FarError,
    FarLibraryMissing,
    far_fused_add_rmsnorm,
    far_plan,
    far_status_string,
    far_version,
    far_workspace_bytes,
    fused_add_rmsnorm,
    load_library,
)
