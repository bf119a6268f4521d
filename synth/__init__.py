"""Seeded synthetic inputs for the packed paged-attention step.

This package draws batches (metadata, query rows, new K/V rows, the paged
pool's contents and its block tables) and drives the iteration-level
scheduler that produces the continuous-batching trace.  It holds no
attention arithmetic: it only draws numbers, lays blocks out, and decides
which rows run in which step.  Both the fp64 oracle's tests and the HIP
path's tests and bench take their inputs from here.
"""

from .workloads import (  # noqa: F401
    Batch,
    BLOCK_SIZE,
    f32_to_bf16_bits,
    make_batch,
    config_worked_step,
    config_decode64,
    config_mixed_chunked,
    config_long_shared,
    permute_placement,
    CONFIG_SEEDS,
)
