"""CPU oracle (float64, materialising) for the attention library.

Test infrastructure only: imported by the test suite, the smoke check and the
benchmark's CPU-baseline leg, never by the library itself.  It shares no code
with the HIP path.
"""
from .attention import (  # noqa: F401
    scores, masked_softmax, attention, attention_varlen, merge_lse, kv_append, decode,
    gather_pages, kv_append_paged, decode_paged, allowed_keys, prefill, prefill_varlen,
    attention_flops, score_matrix_bytes, kv_bytes_per_token, decode_kv_bytes,
)
from .fp8 import (  # noqa: F401
    E4M3_MAX, e4m3_values, quantize_e4m3, dequantize_e4m3, kv_append_fp8, decode_fp8kv,
    prefill_fp8, prefill_varlen_fp8, kv_append_fp8_paged, decode_fp8kv_paged,
)
from .int8 import (  # noqa: F401
    INT8_MAX, quantize_int8, dequantize_int8, kv_append_int8, decode_int8kv, kv_append_int8_paged,
    decode_int8kv_paged,
)
