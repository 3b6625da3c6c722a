"""libfa_mi355x: FlashAttention-2 forward (and backward) for AMD Instinct
MI355X (gfx950).

The compute path is the HIP library built from csrc/ (see include/fa_mi355x.h
for its C ABI); this package only binds it.  Importing does not load the
library; the first call does, and fails loudly if it has not been built.
"""
from ._binding import (  # noqa: F401
    EXPORTS, FA_DTYPE_BF16, FA_DTYPE_F32, FA_ERR_HIP, FA_ERR_INVALID_ARGUMENT, FA_ERR_UNSUPPORTED,
    FA_MASK_ADDITIVE, FA_MASK_BOOL, FA_MASK_NONE, FA_OK, LIB_PATH, FaError, FaStrides, bwd, check, fa_abi_version,
    fa_bwd, fa_bwd_supported, fa_fwd, fa_fwd_dropout, fa_fwd_strided, fa_fwd_strided_noalloc, fa_fwd_window,
    fa_last_error, fa_status_string, fa_supported, fa_variant_count, fa_variant_name,
    fwd, load_library,
)
