"""MI355X (gfx950) block-sparse causal prefill attention (FlashPrefill method).

The compute path is the HIP library `lib/libflashprefill.so` (C ABI declared
in include/flashprefill.h); this package is its ctypes binding plus a small
buffer-owning pipeline object.  Importing the package does not require a GPU;
calling into the library does, and fails loudly if the library is missing.
"""

from ._binding import (  # noqa: F401
    EXPORTED,
    FP_BF16,
    FP_E4M3,
    FP_F32,
    FP_WS_ATTN,
    FP_WS_DENSE,
    FP_WS_DISCOVER,
    FP_WS_SELECT,
    LIB_PATH,
    FpError,
    Problem,
    fp_discover,
    fp_select,
    fp_select_noalloc,
    fp_select_topk,
    fp_select_topp,
    fp_sparse_attn_paged,
    fp_dense_attn_paged,
    load_library,
)
from .pipeline import Pipeline, upload  # noqa: F401
