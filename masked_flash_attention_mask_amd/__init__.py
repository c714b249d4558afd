"""masked_flash_attention_mask_amd — masked flash-attention prefill (bf16,
fp32 and fp8 inputs, and its backward), speculative tree verify and masked
decode over ragged, paged K/V on MI355X (gfx950).

The compute path is libmaskattn.so (hand-written HIP kernels behind a C ABI,
declared in include/maskattn.h).  This package is its thin ctypes binding; it
needs the library to be built and raises when it is not.
"""

from ._lib import (  # noqa: F401
    BF16, F32, KIND, LIB, LIB_PATH, MaskAttnError, Plan, RANGE_BI_CAUSAL, RANGE_CAUSAL,
    RANGE_CHUNK_CAUSAL, RANGE_FULL, RANGE_INV_CAUSAL, TILE_FULL, TILE_PARTIAL, TILE_SKIP,
    attn_backward_masked, attn_backward_workspace, attn_prefill_masked_fp8, attn_decode, attn_decode_kv8, attn_decode_workspace, attn_prefill_masked, attn_verify_tree, attn_verify_tree_workspace,
    attn_verify_tree_noalloc,
    mask_compile,
    mask_compile_host,
)
