"""Put a generated batch on a GPU in the shapes the library takes.

A pool tile of 2048 elements is viewed as [16][128] for keys and [2][128][8]
for values (two halves of 8 tokens; no data moves); lazily defined pools are generated directly on
the device from the counter definition.
"""

from __future__ import annotations

import numpy as np


def bf16_from_bits(bits: np.ndarray, device):
    import torch
    a = np.ascontiguousarray(bits, dtype=np.uint16)
    return torch.from_numpy(a.view(np.int16)).to(device).view(torch.bfloat16)


def pool_to_device(pool, device):
    import torch
    if isinstance(pool, np.ndarray):
        return bf16_from_bits(pool, device)
    return pool.to_device(device).view(torch.bfloat16)


def to_device(batch, device) -> dict:
    import torch
    D = batch.head_dim
    nb, hkv, tile = batch.k_pool.shape
    assert tile == 16 * D
    k = pool_to_device(batch.k_pool, device).view(nb, hkv, 16, D)
    v = pool_to_device(batch.v_pool, device).view(nb, hkv, 2, D, 8)
    i32 = lambda a: torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).to(device)
    return dict(
        q=bf16_from_bits(batch.q, device),
        k_new=bf16_from_bits(batch.k_new, device),
        v_new=bf16_from_bits(batch.v_new, device),
        k_cache=k,
        v_cache=v,
        cu_seqlens_q=i32(batch.cu_seqlens_q),
        seq_lens=i32(batch.seq_lens),
        block_tables=i32(batch.block_tables),
        num_blocks=nb,
        scale=float(batch.scale),
    )
