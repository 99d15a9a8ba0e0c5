"""MI355X-native decode-phase GEMV of GRINQH (input-adaptive bit widths).

The product is libgrinqh.so (HIP kernels for gfx950 behind the C ABI in
include/grinqh.h); this package holds its sources (csrc/), the in-tree build
script (build.py) and the ctypes binding (grinqh.py).
"""

from .grinqh import (  # noqa: F401
    GRINQH_BF16, GRINQH_F32, GrinqhError, Layout, EXPORTS, load, status_string,
    grinqh_layout_init, grinqh_packed_bytes, grinqh_gemv_workspace_bytes,
    grinqh_pack, grinqh_assign_bits, grinqh_gemv, grinqh_debug_codes,
    grinqh_debug_force_launch, force_launch_shape, grinqh_gemv_noalloc, NOALLOC_SCRATCH_BYTES,
    grinqh_gemv_group_workspace_bytes, grinqh_gemv_group, Operands, MAX_GROUP,
    new_workspace, new_group_workspace, pack, assign_bits, gemv, debug_codes,
    grinqh_calibrate_workspace_bytes, grinqh_calibrate_thresholds, calibrate_thresholds,
    grinqh_quantize_rtn, quantize_rtn,
    grinqh_prefill_workspace_bytes, grinqh_prefill_gemm, prefill_gemm,
)
