"""MI355X-native packed, ragged attention step over a paged KV cache.

The product is the C-ABI library libpkv.so (include/pkv.h), built from the
HIP sources in csrc/; this package is its thin Python binding.
"""

from .binding import (  # noqa: F401
    BLOCK_SIZE,
    BlockPool,
    HEAD_DIM,
    PKVError,
    Plan,
    bf16_bits,
    bf16_tensor,
    header_functions,
    load_library,
    pkv_block_hash,
    pkv_copy_blocks,
    pkv_layer_forward,
    pkv_linear,
    pkv_qkv_rope,
    ROPE_THETA,
    pkv_paged_kv_append,
    pkv_paged_step,
    pkv_paged_step_static,
    STATIC_WS_BYTES,
    pkv_paged_varlen_attention,
    pkv_plan,
    pkv_slot_append,
    pkv_slot_append_planned,
    pkv_slot_mapping,
    swap_bytes,
    v_cache_shape,
    pkv_split_kv_reduce,
    pkv_swap_in,
    pkv_swap_out,
    pkv_varlen_attention_main,
)
