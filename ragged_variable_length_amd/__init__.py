"""MI355X-native pack -> attend -> unpack for token-pruned Vision Transformers.

The work runs in librattn.so (hand-written HIP kernels for gfx950 behind a C
ABI declared in include/rattn.h).  This package is its Python binding:
`rattn_pack`, `rattn_forward`, `rattn_unpack` and `rattn_fused` have the C
entry points' names and only marshal arguments (through the `_rattn` CPython
extension); `RaggedPipeline` owns the device buffers (allocated once, through
torch) for repeated calls of the three, and `FusedPlan` is a rattn_fused call
whose arguments are checked and marshalled once.
"""
from ._binding import (LIB_PATH, RattnError, load, rattn_forward, rattn_fused,
                       rattn_fused_padded, rattn_get_validate, rattn_init, rattn_pack,
                       rattn_repack, rattn_set_validate, rattn_unpack, status_string)
from .pipeline import FusedPlan, RaggedPipeline

__all__ = ["LIB_PATH", "FusedPlan", "RattnError", "RaggedPipeline", "load", "rattn_forward",
           "rattn_fused", "rattn_fused_padded", "rattn_get_validate", "rattn_init", "rattn_pack",
           "rattn_repack", "rattn_set_validate", "rattn_unpack", "status_string"]
