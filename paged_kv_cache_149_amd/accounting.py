"""Algorithmic work of one step: the bytes the method must move and the
FLOP it must do, independent of how the kernels do it.

* KV bytes per token per layer = 2 (K and V) x Hkv x D x 2 B
  ("continuous batching" (k4i.top), section "为什么 decode 是 bandwidth-bound":
  bytes per token = 2 x L x n_h x d_h x sizeof(dtype), 131,072 B for 32
  layers of 8 KV heads of 128 in bf16, i.e. 4096 B per layer).
* Unique KV bytes count every physical (block, kv head) tile once, with the
  tokens actually used in it (shared prefix blocks are read from one place);
  logical bytes count every sequence's keys.
* Attention FLOP = 4 x D x Hq x (sum over rows of visible keys): two
  multiply-adds per (query, key, dimension, head) pair, causal pairs only
  ("11.2 连续批处理与 PagedAttention", section 11.2.5: 2 T^2 d per layer for a
  T-token prefill, d = Hq x D).
"""

from __future__ import annotations

import numpy as np

BF16 = 2


def kv_bytes_per_token(num_kv_heads: int, head_dim: int, layers: int = 1, elem: int = BF16) -> int:
    return 2 * layers * num_kv_heads * head_dim * elem


def prefill_attention_flop(T: int, hidden: int, layers: int = 1) -> float:
    """The pages' 2 T^2 d per layer approximation for a T-token prefill."""
    return 2.0 * T * T * hidden * layers


def chunk_attention_flop(past: int, C: int, hidden: int, layers: int = 1) -> float:
    """The pages' 2 d L ((past + C)^2 - past^2) for a C-token chunk after
    ``past`` cached tokens."""
    return 2.0 * hidden * layers * ((past + C) ** 2 - past ** 2)


def visible_pairs(cu_seqlens_q, seq_lens) -> int:
    cu = np.asarray(cu_seqlens_q, dtype=np.int64)
    sl = np.asarray(seq_lens, dtype=np.int64)
    ql = np.diff(cu)
    c = sl - ql
    return int((ql * c + ql * (ql + 1) // 2).sum())


def attention_flop(cu_seqlens_q, seq_lens, num_q_heads: int, head_dim: int) -> float:
    return 4.0 * head_dim * num_q_heads * visible_pairs(cu_seqlens_q, seq_lens)


def kv_bytes_logical(cu_seqlens_q, seq_lens, num_kv_heads: int, head_dim: int) -> int:
    ql = np.diff(np.asarray(cu_seqlens_q, dtype=np.int64))
    sl = np.asarray(seq_lens, dtype=np.int64)
    return int(sl[ql > 0].sum()) * kv_bytes_per_token(num_kv_heads, head_dim)


def kv_bytes_unique(cu_seqlens_q, seq_lens, block_tables, num_kv_heads: int, head_dim: int) -> int:
    """Tokens used per distinct physical block (the most any reader uses),
    summed, times the per-token bytes."""
    ql = np.diff(np.asarray(cu_seqlens_q, dtype=np.int64))
    sl = np.asarray(seq_lens, dtype=np.int64)
    bt = np.asarray(block_tables, dtype=np.int64)
    act = np.nonzero(ql > 0)[0]
    if act.size == 0:
        return 0
    nblk = (sl[act] + 15) // 16
    idx = np.arange(bt.shape[1])[None, :]
    mask = idx < nblk[:, None]
    used_tokens = np.clip(sl[act][:, None] - 16 * idx, 0, 16)
    blocks = bt[act][mask]
    tokens = used_tokens[mask]
    order = np.argsort(blocks, kind="stable")
    b_sorted, t_sorted = blocks[order], tokens[order]
    starts = np.concatenate([[0], np.nonzero(np.diff(b_sorted))[0] + 1])
    per_block_max = np.maximum.reduceat(t_sorted, starts) if b_sorted.size else np.zeros(0)
    return int(per_block_max.sum()) * kv_bytes_per_token(num_kv_heads, head_dim)


def step_bytes(cu_seqlens_q, seq_lens, block_tables, num_q_heads: int, num_kv_heads: int,
               head_dim: int) -> dict:
    """Algorithmic HBM bytes of the attention launch: unique KV, Q in, O out,
    the block-table entries read."""
    cu = np.asarray(cu_seqlens_q, dtype=np.int64)
    T = int(cu[-1])
    ql = np.diff(cu)
    sl = np.asarray(seq_lens, dtype=np.int64)
    kv = kv_bytes_unique(cu, sl, block_tables, num_kv_heads, head_dim)
    qo = 2 * T * num_q_heads * head_dim * BF16
    tables = int(((sl[ql > 0] + 15) // 16).sum()) * 4
    return dict(kv_unique=kv, kv_logical=kv_bytes_logical(cu, sl, num_kv_heads, head_dim),
                q_o=qo, tables=tables, total=kv + qo + tables,
                append=2 * T * kv_bytes_per_token(num_kv_heads, head_dim))
