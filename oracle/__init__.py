"""fp64 CPU oracle for the packed paged-attention step.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path may import, call or
link anything in this package: only the test suite, the smoke check of the
graft entry point and the CPU-baseline leg of the bench use it.  It shares no
code with the HIP library or its binding and imports neither.

Every function here is pinned by a CPU test against something other than
itself (a printed worked example, a closed form, a textbook routine, brute
force); see ``tests/test_oracle_*.py``.
"""

from .paged_attention import (  # noqa: F401
    BLOCK,
    bf16_bits_to_f64,
    slot_of,
    slot_mapping,
    k_group,
    read_k_token,
    read_v_token,
    gather_kv,
    gather_kv_by_token,
    pools_after_append,
    attention_one_request,
    packed_attention,
    packed_attention_rows,
    dense_mask_attention,
    visibility_grid,
    score_shapes,
    step_from_batch,
)

from . import layer  # noqa: F401,E402
