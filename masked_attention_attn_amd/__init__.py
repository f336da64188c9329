"""MI355X (gfx950) masked / LSE / decode attention.

Python names mirror the C ABI in include/attn.h; all compute runs in the
HIP kernels of libmasked_attn.so.
"""
from ._lib import (  # noqa: F401
    ATTN_BF16, ATTN_F32, AttnError, EXPORTS, LIB_PATH, STATUS,
    attn_decode, attn_decode_workspace_bytes, attn_fwd_lse, attn_fwd_masked, attn_fwd_varlen,
    attn_decode_fp8kv, attn_decode_paged, attn_merge_lse, attn_prefill, attn_prefill_fp8, attn_prefill_varlen, kv_append, kv_append_fp8, kv_append_int8, kv_append_paged, load,
    attn_decode_int8kv, attn_prefill_varlen_fp8, kv_append_fp8_paged, kv_append_int8_paged,
    attn_decode_fp8kv_paged, attn_decode_int8kv_paged, attn_decode_noalloc, DECODE_NOALLOC_SCRATCH_BYTES,
)
