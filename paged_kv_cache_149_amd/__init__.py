"""MI355X-native packed, ragged attention step over a paged KV cache.

The product is the C-ABI library libpkv.so (include/pkv.h), built from the
HIP sources in csrc/; this package is its thin Python binding.
"""

from .binding import (  # noqa: F401
    BLOCK_SIZE,
    HEAD_DIM,
    PKVError,
    Plan,
    bf16_bits,
    bf16_tensor,
    header_functions,
    load_library,
    pkv_paged_kv_append,
    pkv_paged_step,
    pkv_paged_varlen_attention,
    pkv_plan,
    pkv_slot_append,
    pkv_slot_mapping,
    pkv_split_kv_reduce,
    pkv_varlen_attention_main,
)
