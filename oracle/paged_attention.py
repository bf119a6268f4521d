"""Plain fp64 definition of one packed, ragged attention step over a paged
KV cache.  Slow and obviously correct; test infrastructure only.

Sources (page titles as given in the source material):

* [CB]  "Continuous Batching 深入实现: 从 attention mask 到 chunked prefill"
         (zoe.im), sections "Ragged Batch + cu_seqlens" and "一个 chunked
         prefill 请求怎么组织 attention".
* [K4I] "continuous batching" (k4i.top), sections "防止跨请求 attention"
         (the block-diagonal mask formula M_ij), "与 KV cache 的关系" (the
         decode formula softmax(q [K_cache; k_t]^T / sqrt(d_k)) [V_cache; v_t])
         and "为什么 packed forward 等价" (the visible set S(i)).
* [PA]  "连续批处理与 PagedAttention 原理" (plumephp.com), section
         "block table 与地址映射" (logical block p // 16, physical block b,
         offset b * 16 + p % 16).
* [YB]  "11.2 连续批处理与 PagedAttention" (yeasy gitbook), section 11.2.2
         (per-request attention inside one packed step, cu_seqlens of shape
         [requests + 1]) and section 11.2.3, Figure 11-4 (shared blocks).
* [MLM] "同时服务多位用户: 连续批处理如何保持 LLM 推理高效" (traeai.com),
         section "完整实现" (the dense block-diagonal mask built from per-key
         and per-query (sequence, position) tags; the printed mask grids).

Readings taken where the pages leave a step open (each is listed again in
the design notes):

* GQA: query head h reads kv head h // (Hq / Hkv) (contiguous groups).
* ``seq_lens[s]`` counts the keys visible to the sequence's last row after
  this step's rows are appended; the cached prefix is
  ``c_s = seq_lens[s] - q_len_s`` and the step's rows sit at positions
  ``c_s .. seq_lens[s] - 1``.
* Physical layout of a (block, kv head) tile of the pool (the pages fix the
  slot formula and that a block's 16 tokens are contiguous, and defer the
  tensor layout to a section that is not present): K tiles hold the
  dimensions in groups of W = min(32, D), each group token-major: element
  (o, d) at ``(d // W) * 16 * W + o * W + d % W`` (D = 128: four groups of
  32 dimensions); V tiles hold the 16 tokens in two halves of 8, each half
  dimension-major: element (o, d) at ``(o // 8) * 8 * D + d * 8 + o % 8``.
  Slot ``x`` is block ``x // 16``, offset ``x % 16``.
* Masked scores are -inf (the M_ij formula of [K4I]); every row sees at
  least its own key, so no row is fully masked.

Parity unpinned: none -- every function below has a pin in the CPU tests.
"""

from __future__ import annotations

from typing import Dict, List, Sequence, Tuple

import numpy as np

BLOCK = 16  # tokens per block ([PA]: the default block holds 16 tokens)


# ----------------------------------------------------------------------------
# numbers
# ----------------------------------------------------------------------------

def bf16_bits_to_f64(bits: np.ndarray) -> np.ndarray:
    """Exact widening of bf16 bit patterns (uint16) to float64: a bf16 value
    is the top half of the float32 with the same sign, exponent and leading
    mantissa bits."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return b.view(np.float32).astype(np.float64)


# ----------------------------------------------------------------------------
# slot translation ([PA] "block table 与地址映射")
# ----------------------------------------------------------------------------

def slot_of(block_table_row: Sequence[int], pos: int) -> int:
    """Physical slot of logical position ``pos``: the logical block is
    pos // 16, the table gives its physical block b, the slot is
    b * 16 + pos % 16."""
    b = int(block_table_row[pos // BLOCK])
    return b * BLOCK + pos % BLOCK


def slot_mapping(cu_seqlens_q, seq_lens, block_tables) -> np.ndarray:
    """Slot of every packed row, in packed order.  Row ``j`` of sequence s
    (0-based within the sequence) sits at position c_s + j."""
    cu = np.asarray(cu_seqlens_q, dtype=np.int64)
    sl = np.asarray(seq_lens, dtype=np.int64)
    out = np.empty(int(cu[-1]), dtype=np.int64)
    for s in range(sl.shape[0]):
        q_len = int(cu[s + 1] - cu[s])
        c = int(sl[s]) - q_len
        for j in range(q_len):
            out[cu[s] + j] = slot_of(block_tables[s], c + j)
    return out


# ----------------------------------------------------------------------------
# reading the pool (layout reading stated in the module docstring)
# ----------------------------------------------------------------------------

def k_group(D: int) -> int:
    """Width of the dimension groups of a K tile."""
    return min(32, D)


def read_k_token(k_pool: np.ndarray, slot: int, head: int, D: int) -> np.ndarray:
    """The D key elements at ``slot`` for kv head ``head`` (bf16 bits): in
    each group of W dimensions, token o's W elements start at o * W."""
    b, o = divmod(int(slot), BLOCK)
    W = k_group(D)
    tile = np.asarray(k_pool[b, head]).reshape(D // W, BLOCK, W)
    return tile[:, o, :].reshape(D)


V_HALF = 8  # tokens per half of a V tile


def read_v_token(v_pool: np.ndarray, slot: int, head: int, D: int) -> np.ndarray:
    """The D value elements at ``slot`` for kv head ``head`` (bf16 bits):
    in the half holding token o, they sit 8 elements apart."""
    b, o = divmod(int(slot), BLOCK)
    tile = np.asarray(v_pool[b, head])
    start = (o // V_HALF) * V_HALF * D + o % V_HALF
    return tile[start:start + V_HALF * D:V_HALF]


def gather_kv(k_pool, v_pool, block_table_row, n_tokens: int, H_kv: int, D: int):
    """Logical, contiguous K and V (fp64, [n_tokens, H_kv, D]) of positions
    0 .. n_tokens-1 of one sequence.  Logical block i (positions 16i ..
    16i+15) is physical block table[i]; position p is offset p % 16 of it,
    which is the slot formula applied a whole block at a time."""
    nblk = (n_tokens + BLOCK - 1) // BLOCK
    if nblk == 0:
        z = np.zeros((0, H_kv, D), dtype=np.float64)
        return z, z.copy()
    blocks = np.asarray(block_table_row[:nblk], dtype=np.int64)
    W = k_group(D)
    kt = k_pool[blocks].reshape(nblk, H_kv, D // W, BLOCK, W)   # (blk, h, group, o, d % W)
    vt = v_pool[blocks].reshape(nblk, H_kv, BLOCK // V_HALF, D, V_HALF)  # (blk, h, half, d, o % 8)
    K = kt.transpose(0, 3, 1, 2, 4).reshape(nblk * BLOCK, H_kv, D)[:n_tokens]
    V = vt.transpose(0, 2, 4, 1, 3).reshape(nblk * BLOCK, H_kv, D)[:n_tokens]
    return bf16_bits_to_f64(K), bf16_bits_to_f64(V)


def gather_kv_by_token(k_pool, v_pool, block_table_row, n_tokens: int, H_kv: int, D: int):
    """Same as gather_kv, one token and one head at a time through
    slot_of / read_k_token / read_v_token (the brute-force form)."""
    K = np.empty((n_tokens, H_kv, D), dtype=np.float64)
    V = np.empty((n_tokens, H_kv, D), dtype=np.float64)
    for p in range(n_tokens):
        x = slot_of(block_table_row, p)
        for h in range(H_kv):
            K[p, h] = bf16_bits_to_f64(read_k_token(k_pool, x, h, D))
            V[p, h] = bf16_bits_to_f64(read_v_token(v_pool, x, h, D))
    return K, V


def pools_after_append(k_pool, v_pool, slots, k_new, v_new):
    """The pool expected after the append: every row's K/V (all kv heads)
    written bit-for-bit into its slot; rows with a negative slot are skipped;
    nothing else changes."""
    k_out = k_pool.copy()
    v_out = v_pool.copy()
    T, H_kv, D = k_new.shape
    for t in range(T):
        x = int(slots[t])
        if x < 0:
            continue
        b, o = divmod(x, BLOCK)
        W = k_group(D)
        for h in range(H_kv):
            k_out[b, h].reshape(D // W, BLOCK, W)[:, o, :] = np.asarray(k_new[t, h]).reshape(D // W, W)
            start = (o // V_HALF) * V_HALF * D + o % V_HALF
            v_out[b, h, start:start + V_HALF * D:V_HALF] = v_new[t, h]
    return k_out, v_out


# ----------------------------------------------------------------------------
# attention
# ----------------------------------------------------------------------------

def attention_one_request(q, K, V, cached: int, scale: float) -> np.ndarray:
    """Dense causal attention of one request.

    q: [n, Hq, D] rows at positions cached .. cached+n-1.
    K, V: [cached+n, Hkv, D] keys/values at positions 0 .. cached+n-1
    (the [K_cache; k_t] stacking of [K4I]).
    Row j, head h sees keys i <= cached + j of kv head h // G (the visible
    set S(i) of [K4I]); out = softmax(scale * q K^T) V over those keys.
    """
    n, Hq, D = q.shape
    L, Hkv, _ = K.shape
    G = Hq // Hkv
    out = np.empty((n, Hq, D), dtype=np.float64)
    for h in range(Hq):
        g = h // G
        scores = (q[:, h, :] @ K[:, g, :].T) * scale          # [n, L]
        pos = cached + np.arange(n)[:, None]
        visible = np.arange(L)[None, :] <= pos
        scores = np.where(visible, scores, -np.inf)
        m = scores.max(axis=1, keepdims=True)
        p = np.exp(scores - m)
        out[:, h, :] = (p @ V[:, g, :]) / p.sum(axis=1, keepdims=True)
    return out


def step_from_batch(batch) -> Dict[str, object]:
    """fp64 views of a generated batch's inputs (shared by the formulations
    below)."""
    return dict(
        cu=np.asarray(batch.cu_seqlens_q, dtype=np.int64),
        seq_lens=np.asarray(batch.seq_lens, dtype=np.int64),
        bt=np.asarray(batch.block_tables, dtype=np.int64),
        q=bf16_bits_to_f64(batch.q),
        k_new=bf16_bits_to_f64(batch.k_new),
        v_new=bf16_bits_to_f64(batch.v_new),
        scale=float(np.float32(batch.scale)),
        H_kv=int(batch.num_kv_heads),
        D=int(batch.head_dim),
    )


def _request_kv(batch, st, s):
    cu, sl = st["cu"], st["seq_lens"]
    q_len = int(cu[s + 1] - cu[s])
    c = int(sl[s]) - q_len
    Kc, Vc = gather_kv(batch.k_pool, batch.v_pool, st["bt"][s], c, st["H_kv"], st["D"])
    rows = slice(int(cu[s]), int(cu[s + 1]))
    K = np.concatenate([Kc, st["k_new"][rows]], axis=0)
    V = np.concatenate([Vc, st["v_new"][rows]], axis=0)
    return rows, c, K, V


def packed_attention(batch, seqs: Sequence[int] | None = None) -> np.ndarray:
    """The whole step: every sequence's rows attend to that sequence's cached
    prefix (read through its block table from the pool as it was before the
    step) followed by its own new rows.  Output [T, Hq, D] fp64 in packed
    order; rows of sequences not in ``seqs`` (when given) are left NaN."""
    st = step_from_batch(batch)
    T = int(st["cu"][-1])
    out = np.full((T,) + st["q"].shape[1:], np.nan, dtype=np.float64)
    for s in (range(len(st["seq_lens"])) if seqs is None else seqs):
        rows, c, K, V = _request_kv(batch, st, s)
        if rows.stop > rows.start:
            out[rows] = attention_one_request(st["q"][rows], K, V, c, st["scale"])
    return out


def packed_attention_rows(batch, rows: Sequence[int]) -> Dict[int, np.ndarray]:
    """Output of selected packed rows only ({row: [Hq, D]}), for sampling
    large steps row by row."""
    st = step_from_batch(batch)
    cu = st["cu"]
    res = {}
    by_seq: Dict[int, List[int]] = {}
    for t in rows:
        s = int(np.searchsorted(cu, t, side="right") - 1)
        by_seq.setdefault(s, []).append(int(t))
    for s, ts in by_seq.items():
        r, c, K, V = _request_kv(batch, st, s)
        for t in ts:
            j = t - r.start
            # row j alone: same visible set (keys 0 .. c+j)
            o = attention_one_request(st["q"][t:t + 1], K[:c + j + 1], V[:c + j + 1], c + j, st["scale"])
            res[t] = o[0]
    return res


def _packed_key_axis(cached_lens, q_lens):
    """Sequence index and position of every key on one packed key axis that
    holds all sequences' cached keys, then all new rows, each part in
    sequence order; and the same two labels for the query rows (the new
    rows).  Sequence s's cached keys sit at positions 0 .. c_s - 1 and its
    new rows at c_s .. c_s + n_s - 1."""
    c = np.asarray(cached_lens, dtype=np.int64)
    n = np.asarray(q_lens, dtype=np.int64)
    ids = np.arange(c.shape[0], dtype=np.int64)
    # position inside a run = running index minus the index the run starts at
    cached_pos = np.arange(int(c.sum())) - np.repeat(np.cumsum(c) - c, c)
    row_pos = np.arange(int(n.sum())) - np.repeat(np.cumsum(n) - n, n) + np.repeat(c, n)
    row_seq = np.repeat(ids, n)
    key_seq = np.concatenate([np.repeat(ids, c), row_seq])
    key_pos = np.concatenate([cached_pos, row_pos])
    return key_seq, key_pos, row_seq, row_pos


def _block_diagonal_causal(key_seq, key_pos, row_seq, row_pos) -> np.ndarray:
    """[K4I] "防止跨请求 attention": row i may read key j exactly when both
    belong to the same request and j's position is not after i's."""
    return (row_seq[:, None] == key_seq[None, :]) & (key_pos[None, :] <= row_pos[:, None])


def dense_mask_attention(batch, seqs: Sequence[int] | None = None) -> np.ndarray:
    """Second, independent formulation ([MLM] "完整实现"; mask rule of [K4I]
    "防止跨请求 attention"): the selected sequences' cached keys, then their
    new rows, laid out as ONE key axis with a (sequence, position) label per
    key and per query; a dense block-diagonal causal mask over that axis;
    one softmax per query row over the whole key axis.  Returns
    [Tsel, Hq, D] for the selected sequences' rows in packed order."""
    st = step_from_batch(batch)
    cu, sl = st["cu"], st["seq_lens"]
    sel = np.arange(sl.shape[0]) if seqs is None else np.asarray(list(seqs), dtype=np.int64)
    Hq, D, Hkv = st["q"].shape[1], st["D"], st["H_kv"]
    G = Hq // Hkv
    q_lens = cu[sel + 1] - cu[sel]
    cached = sl[sel] - q_lens
    key_seq, key_pos, row_seq, row_pos = _packed_key_axis(cached, q_lens)
    # packed row index of every selected query row
    q_rows = np.concatenate([np.arange(cu[s], cu[s + 1]) for s in sel]) if len(sel) else np.zeros(0, np.int64)
    gathered = [gather_kv(batch.k_pool, batch.v_pool, st["bt"][s], int(c), Hkv, D) for s, c in zip(sel, cached)]
    K = np.concatenate([kv[0] for kv in gathered] + [st["k_new"][q_rows]], axis=0)
    V = np.concatenate([kv[1] for kv in gathered] + [st["v_new"][q_rows]], axis=0)
    mask = np.where(_block_diagonal_causal(key_seq, key_pos, row_seq, row_pos), 0.0, -np.inf)
    Q = st["q"][q_rows]
    out = np.empty((q_rows.shape[0], Hq, D), dtype=np.float64)
    for h in range(Hq):
        scores = (Q[:, h, :] @ K[:, h // G, :].T) * st["scale"] + mask
        m = scores.max(axis=1, keepdims=True)
        p = np.exp(scores - m)
        p /= p.sum(axis=1, keepdims=True)
        out[:, h, :] = p @ V[:, h // G, :]
    return out


def visibility_grid(kv_lens: Sequence[int], q_lens: Sequence[int]) -> np.ndarray:
    """Boolean [total_q, total_kv + total_q] grid of the dense mask of [MLM]
    for sequences with ``kv_lens`` cached and ``q_lens`` new tokens: key axis
    [all cached | all new], allowed iff same sequence and key position <=
    query position."""
    return _block_diagonal_causal(*_packed_key_axis(kv_lens, q_lens))


def score_shapes(cu_seqlens_q, seq_lens) -> List[Tuple[int, int]]:
    """Per-request, per-head score-matrix shape [q_len, keys] of [YB] 11.2.2:
    each request's queries against its own cached + new keys."""
    cu = np.asarray(cu_seqlens_q, dtype=np.int64)
    return [(int(cu[s + 1] - cu[s]), int(n)) for s, n in enumerate(seq_lens)]
