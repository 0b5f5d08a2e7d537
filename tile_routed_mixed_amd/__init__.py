"""Tile-routed mixed-precision causal attention for MI355X (gfx950).

The computation lives in libtm.so (HIP kernels behind the C ABI declared in
include/tm.h); this package is its thin ctypes binding plus device-buffer
helpers.  Importing it does not load the library; the first call does, and it
raises if the library has not been built.
"""
from ._binding import (  # noqa: F401
    TM_OK, TM_E_ARG, TM_E_SHAPE, TM_E_POLICY, TM_E_SPACE, TM_E_UNSUPPORTED, TM_E_HIP,
    TM_F16, TM_BF16, TM_F32, TM_SKIP, TM_INT4, TM_INT8, TM_FP16, TM_ROWS, TM_COLS,
    TM_POLICY_BOUNDARIES, TM_POLICY_BITMASK, TM_POLICY_FOURWAY, TM_POLICY_HYBRID, TMError, lib, Shape, QTensor, Policy, DPolicy,
    tm_quantize_pack, tm_build_traversal, tm_prefill, tm_decode, tm_cache_append, tm_gather_selected, tm_decode_select, tm_select_vertical, traversal_bytes, decode_ws_bytes,
    LIB_PATH,
)
from .pipeline import PrefillPipeline, DecodePipeline, read_traversal  # noqa: F401
from . import calibrate  # noqa: F401
