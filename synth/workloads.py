"""Seeded synthetic batches for one packed, ragged attention step over a
paged KV cache.

What a batch holds (all integer metadata is int32, all tensors are bf16 bit
patterns stored as uint16):

* ``cu_seqlens_q[S+1]``: cumulative query-row counts; sequence ``s`` owns
  packed rows ``cu[s] .. cu[s+1]-1`` (the ragged layout of "Continuous
  Batching 深入实现", section "Ragged Batch + cu_seqlens").
* ``seq_lens[S]``: keys visible to the sequence's last row after this step's
  rows are appended (cached prefix + this step's rows).
* ``block_tables[S, MB]``: physical block id of each logical 16-token block
  ("连续批处理与 PagedAttention 原理", section "block table 与地址映射");
  entries past a sequence's last block are -1.
* ``q[T, Hq, D]``, ``k_new / v_new[T, Hkv, D]``: this step's rows.
* ``k_pool / v_pool[NB, Hkv, 16*D]``: the pool's contents before the step,
  one 4 KiB tile per (block, kv head).  Every element of a referenced tile is
  an independent N(0,1) draw; the generator does not know or care how the
  2048 elements of a tile are ordered (token-major, dimension-major...).
  Tiles of blocks no table references are filled with a quiet-NaN pattern
  by default, so a reader that strays into them shows up at once.

Values are N(0,1) rounded to bf16 (nearest even), computed by the
counter-based generator of ``synth.counter`` from (seed, tensor, element
index), so every consumer sees the same bits and any block of a large pool
can be computed on its own (``Pool``); the whole pool can be generated on
the GPU from the same definition.  Lengths and block placement (a seeded
random permutation of the pool's block ids) come from
``numpy.random.Generator(PCG64(seed))``.  This module holds no attention
arithmetic.
"""

from __future__ import annotations

import dataclasses
import math
from typing import List, Optional, Sequence, Tuple

import numpy as np

from . import counter

BLOCK_SIZE = 16
HEAD_DIM = 128
NUM_Q_HEADS = 32
NUM_KV_HEADS = 8
QNAN_BF16 = np.uint16(counter.QNAN_BF16)

# seed of config i (1-based) is 149000 + i
CONFIG_SEEDS = {i: 149000 + i for i in range(1, 6)}


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bf16 (round to nearest, ties to even); return
    the 16-bit patterns.  Inputs here are finite."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    lsb = (u >> np.uint32(16)) & np.uint32(1)
    r = (u + np.uint32(0x7FFF) + lsb) >> np.uint32(16)
    return r.astype(np.uint16)


# counter-generator stream ids of the batch tensors
STREAM_Q, STREAM_K_NEW, STREAM_V_NEW, STREAM_K_POOL, STREAM_V_POOL = 1, 2, 3, 4, 5


class Pool:
    """The pool's contents, [num_blocks, Hkv, 16*D] bf16 bits, computed on
    demand: ``pool[blocks]`` gives the tiles of the listed blocks and
    ``pool[b, h]`` one tile.  Element (b, h, e) is counter element
    (b * Hkv + h) * 16D + e of this pool's stream; tiles of blocks no table
    references hold ``unused_fill`` instead."""

    def __init__(self, seed, stream, num_blocks, num_kv_heads, tile, referenced, unused_fill):
        self.seed, self.stream = seed, stream
        self.num_blocks, self.num_kv_heads, self.tile = num_blocks, num_kv_heads, tile
        self.referenced = referenced
        self.unused_fill = unused_fill
        self.shape = (num_blocks, num_kv_heads, tile)
        self.dtype = np.dtype(np.uint16)

    def tiles(self, blocks) -> np.ndarray:
        blocks = np.asarray(blocks, dtype=np.int64).reshape(-1)
        per = self.num_kv_heads * self.tile
        idx = blocks.astype(np.uint64)[:, None] * np.uint64(per) + np.arange(per, dtype=np.uint64)[None, :]
        out = counter.normal_bf16_np(self.seed, self.stream, idx)
        if self.unused_fill != "normal":
            free = ~self.referenced[blocks]
            out[free] = QNAN_BF16 if self.unused_fill == "nan" else 0
        return out.reshape(blocks.shape[0], self.num_kv_heads, self.tile)

    def __getitem__(self, key):
        if isinstance(key, tuple):
            b, h = key
            return self.tiles([int(b)])[0, h]
        a = np.asarray(key)
        if a.ndim == 0:
            return self.tiles([int(a)])[0]
        return self.tiles(a)

    def materialize(self) -> np.ndarray:
        return self.tiles(np.arange(self.num_blocks))

    def copy(self) -> np.ndarray:
        return self.materialize()

    def to_device(self, device):
        """int16 tensor [num_blocks, Hkv, tile] generated on ``device``."""
        import torch
        per = self.num_kv_heads * self.tile
        t = counter.normal_bf16_range_torch(self.seed, self.stream, 0, self.num_blocks * per, device)
        t = t.view(self.num_blocks, self.num_kv_heads, self.tile)
        if self.unused_fill != "normal":
            free = torch.from_numpy(np.nonzero(~self.referenced)[0]).to(device)
            if free.numel():
                t[free] = QNAN_BF16 if self.unused_fill == "nan" else 0
        return t


@dataclasses.dataclass
class Batch:
    name: str
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    cu_seqlens_q: np.ndarray
    seq_lens: np.ndarray
    block_tables: np.ndarray
    num_blocks: int
    q: np.ndarray
    k_new: np.ndarray
    v_new: np.ndarray
    k_pool: np.ndarray
    v_pool: np.ndarray
    scale: np.float32
    shared_groups: List[Tuple[Tuple[int, ...], int]] = dataclasses.field(default_factory=list)
    seed: int = 0

    @property
    def num_seqs(self) -> int:
        return int(self.seq_lens.shape[0])

    @property
    def num_rows(self) -> int:
        return int(self.cu_seqlens_q[-1])

    @property
    def q_lens(self) -> np.ndarray:
        return np.diff(self.cu_seqlens_q).astype(np.int64)

    @property
    def cached_lens(self) -> np.ndarray:
        return self.seq_lens.astype(np.int64) - self.q_lens

    @property
    def bt_stride(self) -> int:
        return int(self.block_tables.shape[1])


def _blocks_needed(n_tokens: int) -> int:
    return (n_tokens + BLOCK_SIZE - 1) // BLOCK_SIZE


def make_batch(
    name: str,
    seqs: Sequence[Tuple[int, int]],
    *,
    seed: int,
    num_q_heads: int = NUM_Q_HEADS,
    num_kv_heads: int = NUM_KV_HEADS,
    head_dim: int = HEAD_DIM,
    num_blocks: Optional[int] = None,
    pool_factor: float = 1.25,
    shared_groups: Sequence[Tuple[Sequence[int], int]] = (),
    unused_fill: str = "nan",
    pool: str = "lazy",
    rng: Optional[np.random.Generator] = None,
) -> Batch:
    """Draw one batch.

    ``seqs`` lists ``(cached, q_len)`` per sequence in packed order.
    ``pool`` is "lazy" (a ``Pool``) or "materialize" (numpy arrays).
    ``shared_groups`` lists ``(members, n_blocks)``: the first ``n_blocks``
    logical blocks of every member point at the same physical blocks (a
    read-only shared prefix; each member must hold at least that many full
    cached blocks).  ``num_blocks`` defaults to ``ceil(pool_factor * used)``.
    """
    if rng is None:
        rng = np.random.Generator(np.random.PCG64(seed))
    S = len(seqs)
    cached = np.array([c for c, _ in seqs], dtype=np.int64)
    qlen = np.array([n for _, n in seqs], dtype=np.int64)
    if (cached < 0).any() or (qlen < 0).any():
        raise ValueError("negative length")
    seq_lens = cached + qlen
    need = np.array([_blocks_needed(int(n)) for n in seq_lens], dtype=np.int64)

    shared_of = {}
    for gi, (members, nb) in enumerate(shared_groups):
        for m in members:
            if m in shared_of:
                raise ValueError("sequence in two shared groups")
            if cached[m] < nb * BLOCK_SIZE:
                raise ValueError("shared prefix must be full cached blocks")
            shared_of[m] = (gi, nb)
    n_shared = sum(nb for _, nb in shared_groups)
    used = int(need.sum()) - sum(shared_of[m][1] for m in shared_of) + n_shared
    if num_blocks is None:
        num_blocks = int(math.ceil(pool_factor * used))
    if used > num_blocks:
        raise ValueError(f"pool of {num_blocks} blocks cannot hold {used}")

    perm = rng.permutation(num_blocks).astype(np.int64)
    cursor = 0
    group_blocks = []
    for _, nb in shared_groups:
        group_blocks.append(perm[cursor:cursor + nb])
        cursor += nb
    mb = max(1, int(need.max()) if S else 1)
    bt = np.full((S, mb), -1, dtype=np.int64)
    for s in range(S):
        start = 0
        if s in shared_of:
            gi, nb = shared_of[s]
            bt[s, :nb] = group_blocks[gi]
            start = nb
        n_priv = int(need[s]) - start
        bt[s, start:start + n_priv] = perm[cursor:cursor + n_priv]
        cursor += n_priv

    T = int(qlen.sum())
    cu = np.zeros(S + 1, dtype=np.int64)
    cu[1:] = np.cumsum(qlen)
    q = counter.normal_bf16_range_np(seed, STREAM_Q, 0, T * num_q_heads * head_dim)
    q = q.reshape(T, num_q_heads, head_dim)
    k_new = counter.normal_bf16_range_np(seed, STREAM_K_NEW, 0, T * num_kv_heads * head_dim)
    k_new = k_new.reshape(T, num_kv_heads, head_dim)
    v_new = counter.normal_bf16_range_np(seed, STREAM_V_NEW, 0, T * num_kv_heads * head_dim)
    v_new = v_new.reshape(T, num_kv_heads, head_dim)

    tile = BLOCK_SIZE * head_dim
    referenced = np.zeros(num_blocks, dtype=bool)
    referenced[bt[bt >= 0]] = True
    if unused_fill not in ("nan", "zero", "normal"):
        raise ValueError(unused_fill)
    k_pool = Pool(seed, STREAM_K_POOL, num_blocks, num_kv_heads, tile, referenced, unused_fill)
    v_pool = Pool(seed, STREAM_V_POOL, num_blocks, num_kv_heads, tile, referenced, unused_fill)
    if pool == "materialize":
        k_pool, v_pool = k_pool.materialize(), v_pool.materialize()

    return Batch(
        name=name,
        num_q_heads=num_q_heads,
        num_kv_heads=num_kv_heads,
        head_dim=head_dim,
        cu_seqlens_q=cu.astype(np.int32),
        seq_lens=seq_lens.astype(np.int32),
        block_tables=bt.astype(np.int32),
        num_blocks=int(num_blocks),
        q=q,
        k_new=k_new,
        v_new=v_new,
        k_pool=k_pool,
        v_pool=v_pool,
        scale=np.float32(1.0 / math.sqrt(head_dim)),
        shared_groups=[(tuple(m), nb) for m, nb in shared_groups],
        seed=seed,
    )


def batch_from_metadata(name: str, cu_seqlens_q, seq_lens, block_tables, num_blocks: int, *, seed: int,
                        num_q_heads: int = NUM_Q_HEADS, num_kv_heads: int = NUM_KV_HEADS,
                        head_dim: int = HEAD_DIM, unused_fill: str = "nan") -> Batch:
    """A batch with given metadata (e.g. one step of the scheduler's trace)
    and freshly drawn values: the step's rows, and a pool whose every
    referenced tile is an N(0,1) draw."""
    cu = np.asarray(cu_seqlens_q, dtype=np.int32)
    sl = np.asarray(seq_lens, dtype=np.int32)
    bt = np.asarray(block_tables, dtype=np.int32)
    T = int(cu[-1])
    rows = lambda stream, H: counter.normal_bf16_range_np(seed, stream, 0, T * H * head_dim).reshape(T, H, head_dim)
    referenced = np.zeros(num_blocks, dtype=bool)
    for s_ in range(sl.shape[0]):
        nb = (int(sl[s_]) + BLOCK_SIZE - 1) // BLOCK_SIZE
        referenced[bt[s_, :nb]] = True
    tile = BLOCK_SIZE * head_dim
    return Batch(
        name=name, num_q_heads=num_q_heads, num_kv_heads=num_kv_heads, head_dim=head_dim,
        cu_seqlens_q=cu, seq_lens=sl, block_tables=bt, num_blocks=int(num_blocks),
        q=rows(STREAM_Q, num_q_heads), k_new=rows(STREAM_K_NEW, num_kv_heads),
        v_new=rows(STREAM_V_NEW, num_kv_heads),
        k_pool=Pool(seed, STREAM_K_POOL, num_blocks, num_kv_heads, tile, referenced, unused_fill),
        v_pool=Pool(seed, STREAM_V_POOL, num_blocks, num_kv_heads, tile, referenced, unused_fill),
        scale=np.float32(1.0 / math.sqrt(head_dim)), seed=seed)


def permute_placement(batch: Batch, seed: int) -> Batch:
    """Same logical K/V, new physical placement: whole tiles move to new block
    ids and every block-table entry is renamed the same way."""
    rng = np.random.Generator(np.random.PCG64(seed))
    perm = rng.permutation(batch.num_blocks)
    src_k, src_v = np.asarray(batch.k_pool.copy()), np.asarray(batch.v_pool.copy())
    k_pool = np.empty_like(src_k)
    v_pool = np.empty_like(src_v)
    k_pool[perm] = src_k
    v_pool[perm] = src_v
    bt = batch.block_tables.astype(np.int64)
    bt = np.where(bt >= 0, perm[np.maximum(bt, 0)], -1)
    return dataclasses.replace(batch, k_pool=k_pool, v_pool=v_pool,
                               block_tables=bt.astype(np.int32))


# ----------------------------------------------------------------------------
# The single-step workloads.  Shapes follow the pages' Llama-3-8B figures
# (32 query heads, 8 GQA KV heads, head_dim 128, bf16).
# ----------------------------------------------------------------------------

def config_worked_step(seed: int = CONFIG_SEEDS[1], **kw) -> Batch:
    """The selective-batching worked step of "11.2 连续批处理与 PagedAttention"
    (section 11.2.2): R1 prefills 5 tokens with nothing cached, R2 decodes
    with 7 cached (8 visible), R3 decodes with 3 cached (4 visible); 7 packed
    rows; a 64-block pool."""
    return make_batch("worked-step-3req-7rows", [(0, 5), (7, 1), (3, 1)],
                      seed=seed, num_blocks=64, **kw)


def config_decode64(seed: int = CONFIG_SEEDS[2], **kw) -> Batch:
    """Decode-only step: 64 sequences, one query row each, cached lengths
    uniform integers in [128, 4096]; pool = ceil(1.25 x blocks used)."""
    rng = np.random.Generator(np.random.PCG64(seed))
    cached = rng.integers(128, 4096, size=64, endpoint=True)
    return make_batch("decode-64seq-ctx128-4096", [(int(c), 1) for c in cached],
                      seed=seed, rng=rng, **kw)


def config_mixed_chunked(seed: int = CONFIG_SEEDS[3], n_decode: int = 1024, **kw) -> Batch:
    """Mixed chunked-prefill step at a 2048-token budget: four 256-row prefill
    chunks continuing cached prefixes of 0/1024/2048/3072 tokens, then 1024
    decode rows whose cached lengths are log-normal (median 1024, sigma 1.0)
    clipped to [16, 8192]."""
    rng = np.random.Generator(np.random.PCG64(seed))
    dec = np.clip(np.rint(np.exp(rng.normal(math.log(1024.0), 1.0, size=n_decode))), 16, 8192)
    seqs = [(p, 256) for p in (0, 1024, 2048, 3072)] + [(int(c), 1) for c in dec]
    return make_batch("mixed-4x256prefill-1024decode", seqs, seed=seed, rng=rng, **kw)


def config_long_shared(seed: int = CONFIG_SEEDS[4], n_seqs: int = 16, cached: int = 32768,
                       group: int = 8, shared_tokens: int = 2048, **kw) -> Batch:
    """Long-context decode with prefix sharing: 16 sequences x 32768 cached
    tokens, one query row each; each group of 8 sequences aliases the same
    physical blocks for its first 2048 tokens."""
    nb = shared_tokens // BLOCK_SIZE
    groups = [(tuple(range(g, min(g + group, n_seqs))), nb) for g in range(0, n_seqs, group)]
    return make_batch("longctx-16x32768-shared2048", [(cached, 1)] * n_seqs,
                      seed=seed, shared_groups=groups, **kw)


def config_prefill_chunk(seed: int = 149006, past: int = 30720, chunk: int = 2048, **kw) -> Batch:
    """Prefill-heavy: one 2048-token chunk continuing a 30,720-token cached
    prefix -- the sixteenth chunk of the 32,768-token prompt of "11.2 连续批处理
    与 PagedAttention", section 11.2.5."""
    return make_batch(f"prefill-chunk{chunk}-after{past}", [(past, chunk)], seed=seed, **kw)


def config_prefill_fresh(seed: int = 149007, n: int = 4, length: int = 2048, **kw) -> Batch:
    """Prefill-heavy: four 2048-token prompts with nothing cached (an 8192-token
    budget of fresh prefill)."""
    return make_batch(f"prefill-{n}x{length}-fresh", [(0, length)] * n, seed=seed, **kw)


def config_trace_step(index: int = 150, seed: int = 149008, **kw) -> Batch:
    """One step of the continuous-batching trace (default step 150: about 735
    decode rows beside ~7,460 rows of prefill chunks), with fresh N(0,1)
    values for its rows and every pool tile it references."""
    from synth import scheduler as sc
    steps, sch = sc.continuous_batching_trace(sc.TraceConfig(steps=index + 1))
    st = steps[index]
    return batch_from_metadata(f"trace-step{index}-{st.num_rows}rows-{st.n_decode}decode", st.cu_seqlens_q,
                               st.seq_lens, st.block_tables, sch.pool.num_blocks, seed=seed, **kw)
