"""Fused multi-head attention (forward, split-KV decode, backward), attention
KL divergence and the output projection, for AMD MI355X (gfx950).

The computation lives in the HIP library ``libmha.so`` behind the C ABI of
include/mha.h; this package only binds it (see ``_binding``).
"""
from ._binding import (  # noqa: F401
    EXPORTED_SYMBOLS,
    LIB_PATH,
    MHA_DTYPE_BF16,
    MHA_DTYPE_FP16,
    MHA_ERR_DEVICE,
    MHA_ERR_INVALID_ARG,
    MHA_ERR_LAUNCH,
    MHA_ERR_SCRATCH_TOO_SMALL,
    MHA_ERR_UNSUPPORTED,
    MHA_NOALLOC_SCRATCH_BYTES,
    MHA_OK,
    MhaError,
    attention,
    attention_backward,
    attention_kl,
    attention_splitkv,
    attention_splitkv_noalloc,
    load_library,
    out_proj,
    mha_abi_version,
    mha_bwd,
    mha_kl_fwd,
    mha_out_proj,
    mha_fwd_splitkv,
    mha_fwd_splitkv_noalloc,
    mha_fwd_splitkv_splits,
    mha_fwd,
    mha_status_string,
)
