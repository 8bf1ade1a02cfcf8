"""CCA (Core Context Aware) attention forward for AMD MI355X (gfx950).

The computation lives in libcca.so (hand-written HIP kernels behind the C ABI
of include/cca.h); this package only marshals torch tensors into that ABI.
"""
from ._lib import (  # noqa: F401
    CCA_BF16, CCA_ERR_CAPACITY, CCA_ERR_HIP, CCA_ERR_INVALID_ARG, CCA_ERR_UNSUPPORTED, CCA_F16, CCA_F32,
    CCA_OK, CCA_POOL_MAX, CCA_POOL_MEAN, CCA_POOL_SOFTMAX, CCA_POOL_SOFTMAX_HEADS, CCAError,
    EXPORTS, LIB_PATH, cca_attn_backward, cca_attn_backward_workspace_bytes, cca_attn_decode,
    cca_attn_prefill, cca_attn_prefill_chunk, cca_attn_prefill_train,
    cca_cache_fill_ring, cca_pool_core_chunk,
    cca_attn_decode_scratch, cca_decode_scratch_bytes, cca_decode_workspace_bytes, cca_pool_core,
    cca_version, cca_visibility_table, core_dtype, load,
)
