"""Oracle for one packed attention layer around the paged step -- test
infrastructure, slow and plain; only the tests, the smoke check and the
benchmark's CPU baseline use it.  The library's product path never imports
it.

What the pages fix (cited per function):

* [K4I] "continuous batching" (k4i.top), section "把 prefill 和 decode
  打包在一起": the new tokens of every request of the iteration are packed
  into one flat matrix X, row by row in request order, and projected at once
  into Q = X W_Q, K = X W_K, V = X W_V; the packing is a physical layout
  only -- every row keeps its request id, position id and sequence
  boundary, and RoPE sees each request's own position id.
* [YB] "11.2 连续批处理与 PagedAttention", section 11.2.2 (selective
  batching, Figure 11-3): the rows of all requests of a step form one
  matrix without a batch axis, X[7, 4096] in the worked example (R1 prefill
  rows at positions 0..4, R2 decode at position 7, R3 decode at 3); the
  weight layers run over all rows at once (X[7, 4096] x W_Q[4096, 4096] ->
  Q[7, 4096], X x W_K[4096, 1024] -> K[7, 1024]); the new K and V go to
  each request's own cache; attention runs per request and its results are
  put back as [7, 4096].

Readings where the pages leave a choice open (also in the design notes):

* weights are stored as [out features][in features] -- the transpose of
  the pages' W_Q[4096, 4096] -- so each output feature's weights are
  contiguous and a projection is y = x w^T;
* the fused QKV weight stacks the query heads' rows, then the key heads',
  then the value heads' (head h of a kind at rows h*D .. h*D + D - 1);
* RoPE (Su et al., RoFormer): the pages name it without its formula.  The
  plainest reading, and the one Llama-family models use: dimension i of
  the first half of a head pairs with dimension i + D/2; the pair at
  position p turns by the angle p * theta^(-2i/D), i = 0 .. D/2 - 1, with
  theta = 500000 (Llama 3, the model family of the pages' workloads);
  applied to queries and keys, not values;
* the output projection takes the attention output of all query heads,
  row-major [T][Hq * D], and has no bias; no residual, norm or MLP (outside
  the step).

Parity unpinned: none -- every function below has a pin in
``tests/test_layer_oracle.py``.
"""

from __future__ import annotations

from typing import Sequence

import numpy as np

from .paged_attention import attention_one_request, bf16_bits_to_f64, gather_kv

LLAMA3_ROPE_THETA = 500000.0


def row_positions(cu_seqlens_q: Sequence[int], seq_lens: Sequence[int]) -> np.ndarray:
    """[K4I] "把 prefill 和 decode 打包在一起": the position id of every packed
    row -- row j of sequence s sits at seq_lens[s] - q_len_s + j (its cached
    prefix, then its new rows)."""
    cu = np.asarray(cu_seqlens_q, dtype=np.int64)
    sl = np.asarray(seq_lens, dtype=np.int64)
    pos = np.empty(int(cu[-1]), dtype=np.int64)
    for s in range(len(sl)):
        q_len = int(cu[s + 1] - cu[s])
        for j in range(q_len):
            pos[cu[s] + j] = sl[s] - q_len + j
    return pos


def linear(x: np.ndarray, w: np.ndarray) -> np.ndarray:
    """y = x w^T over all packed rows at once ([K4I] Q = X W_Q; [YB] 11.2.2
    the weight layers over all rows), with w stored [out][in]; fp64."""
    return np.asarray(x, dtype=np.float64) @ np.asarray(w, dtype=np.float64).T


def rope_angles(positions: np.ndarray, head_dim: int, theta: float = LLAMA3_ROPE_THETA) -> np.ndarray:
    """Angle of pair i at each position: p * theta^(-2i/D), [n, D/2]."""
    i = np.arange(head_dim // 2, dtype=np.float64)
    inv_freq = theta ** (-2.0 * i / head_dim)
    return np.asarray(positions, dtype=np.float64)[:, None] * inv_freq[None, :]


def rope(x: np.ndarray, positions: np.ndarray, theta: float = LLAMA3_ROPE_THETA) -> np.ndarray:
    """Rotate every head of x [n, H, D] by its row's position: the pair
    (x_i, x_{i+D/2}) becomes (x_i cos a - x_{i+D/2} sin a,
    x_{i+D/2} cos a + x_i sin a), a = the pair's angle."""
    x = np.asarray(x, dtype=np.float64)
    half = x.shape[-1] // 2
    a = rope_angles(positions, x.shape[-1], theta)[:, None, :]
    c, s = np.cos(a), np.sin(a)
    x1, x2 = x[..., :half], x[..., half:]
    return np.concatenate([x1 * c - x2 * s, x2 * c + x1 * s], axis=-1)


def qkv_rope(x: np.ndarray, w_qkv: np.ndarray, positions: np.ndarray, num_q_heads: int, num_kv_heads: int,
             head_dim: int, theta: float = LLAMA3_ROPE_THETA):
    """The fused projection of the packed rows, split into heads, with RoPE
    on queries and keys: (q [T,Hq,D], k [T,Hkv,D], v [T,Hkv,D]), fp64."""
    y = linear(x, w_qkv)
    T = y.shape[0]
    nq, nk = num_q_heads * head_dim, num_kv_heads * head_dim
    q = y[:, :nq].reshape(T, num_q_heads, head_dim)
    k = y[:, nq:nq + nk].reshape(T, num_kv_heads, head_dim)
    v = y[:, nq + nk:nq + 2 * nk].reshape(T, num_kv_heads, head_dim)
    return rope(q, positions, theta), rope(k, positions, theta), v


def layer_forward(x, w_qkv, w_o, cu_seqlens_q, seq_lens, block_tables, k_pool, v_pool, num_q_heads: int,
                  num_kv_heads: int, head_dim: int, scale: float, theta: float = LLAMA3_ROPE_THETA):
    """One layer over the packed rows ([YB] 11.2.2: weight layers over all
    rows, attention per request): project and rotate, then each request's
    rows attend to its cached prefix (read through its block table from the
    pools as they were before the step) followed by its own new rows, then
    the output projection.  Returns (y [T, hidden_out], q, k, v, attn), fp64.
    """
    cu = np.asarray(cu_seqlens_q, dtype=np.int64)
    sl = np.asarray(seq_lens, dtype=np.int64)
    pos = row_positions(cu, sl)
    q, k, v = qkv_rope(x, w_qkv, pos, num_q_heads, num_kv_heads, head_dim, theta)
    T = int(cu[-1])
    attn = np.full((T, num_q_heads, head_dim), np.nan)
    for s in range(len(sl)):
        rows = slice(int(cu[s]), int(cu[s + 1]))
        c = int(sl[s]) - (rows.stop - rows.start)
        if rows.stop == rows.start:
            continue
        Kc, Vc = gather_kv(k_pool, v_pool, np.asarray(block_tables)[s], c, num_kv_heads, head_dim)
        K = np.concatenate([Kc, k[rows]], axis=0)
        V = np.concatenate([Vc, v[rows]], axis=0)
        attn[rows] = attention_one_request(q[rows], K, V, c, scale)
    y = linear(attn.reshape(T, num_q_heads * head_dim), w_o)
    return y, q, k, v, attn


__all__ = ["LLAMA3_ROPE_THETA", "row_positions", "linear", "rope_angles", "rope", "qkv_rope", "layer_forward",
           "bf16_bits_to_f64"]
