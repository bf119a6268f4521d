"""Oracle for the block pool, copy-on-write and swap -- test infrastructure,
slow and plain; only the tests, the smoke check and the benchmark's CPU
baseline use it.  The library's product path never imports it.

What the pages fix (cited per function):

* [PA] "连续批处理与 PagedAttention 原理", section "块管理器": the physical
  block pool records which blocks are free and, for every block in use, a
  reference count; each sequence has a block table from logical to
  physical blocks; the operations are allocation, release and
  copy-on-write (when two sequences share a physical block and one of them
  must write a new token into it, the block is copied first and the other
  sequence is unaffected).
* [YB] "11.2 连续批处理与 PagedAttention", section 11.2.3 "共享" and Figure
  11-4: several logical blocks may map to one physical block; within one
  request, parallel samples share all of the prompt's blocks and only the
  last, not yet full block is copied when a sample writes into a block whose
  count is above 1; across requests only full, read-only blocks are shared.
  A request takes a new block only when it has filled its last one.
* [PA] section "抢占策略" and [CB] "Continuous Batching 深入实现", section
  "Preemption 与 Recompute vs Swap": a swapped-out sequence's KV cache is
  copied to CPU memory and copied back when it resumes.

Readings where the pages leave a choice open (also in the design notes):

* which free block an allocation returns: free blocks form a stack; a new
  pool has block 0 on top, then 1, 2, ...; allocation pops the top and a
  block whose count reaches zero is pushed on top.  (Any order is correct;
  this one makes two implementations comparable id for id.)
* a sequence that writes into its partially filled last block while it is
  the only holder writes in place (the pages copy only shared blocks).
* the host layout of swapped blocks: block p of the list occupies
  host[p][0] = its K slab (all kv heads, pool tile layout) and
  host[p][1] = its V slab.

Parity unpinned: none -- every function below has a pin in
``tests/test_block_pool_oracle.py``.
"""

from __future__ import annotations

from typing import List, Optional, Sequence, Tuple

import numpy as np

BLOCK = 16


class PoolModel:
    """The block pool as the pages describe it, one Python list per field."""

    def __init__(self, num_blocks: int):
        self.refcount = [0] * num_blocks
        self.free = list(range(num_blocks - 1, -1, -1))  # top of the stack at the end

    def num_free(self) -> int:
        return len(self.free)

    def allocate(self, n: int) -> List[int]:
        if n > len(self.free):
            raise MemoryError("not enough free blocks")
        out = []
        for _ in range(n):
            b = self.free.pop()
            self.refcount[b] = 1
            out.append(b)
        return out

    def share(self, blocks: Sequence[int]) -> None:
        for b in blocks:
            if self.refcount[b] <= 0:
                raise ValueError("sharing a free block")
        for b in blocks:
            self.refcount[b] += 1

    def release(self, blocks: Sequence[int]) -> None:
        for b in set(blocks):
            if self.refcount[b] < list(blocks).count(b):
                raise ValueError("more releases than references")
        for b in blocks:
            self.refcount[b] -= 1
            if self.refcount[b] == 0:
                self.free.append(b)

    def append_slots(self, row: List[int], num_tokens: int, num_new: int) -> Optional[Tuple[int, int]]:
        """Make room in block-table ``row`` (a list, changed in place) for
        num_new tokens after num_tokens.  A held block that the first new
        token falls in and that another sequence also maps is replaced by a
        copy; blocks beyond the held ones are allocated when needed."""
        if num_new == 0:
            return None
        held = -(-num_tokens // BLOCK)
        need = -(-(num_tokens + num_new) // BLOCK)
        first = num_tokens // BLOCK
        cow = first < held and self.refcount[row[first]] > 1
        if need - held + int(cow) > len(self.free):
            raise MemoryError("not enough free blocks")
        copy = None
        if cow:
            old = row[first]
            new = self.allocate(1)[0]
            self.release([old])
            row[first] = new
            copy = (old, new)
        for lb in range(held, need):
            row[lb] = self.allocate(1)[0]
        return copy


def pools_after_copy(k_pool: np.ndarray, v_pool: np.ndarray, pairs: Sequence[Tuple[int, int]],
                     num_blocks: int):
    """Both pools after copying block src onto block dst for every pair
    (every kv head, bit for bit); pairs with an id outside the pool or
    src == dst change nothing.  Sources are read before any write (the
    destinations of a valid list are distinct and not sources)."""
    k_out = np.array(k_pool, copy=True)
    v_out = np.array(v_pool, copy=True)
    for src, dst in pairs:
        if not (0 <= src < num_blocks and 0 <= dst < num_blocks) or src == dst:
            continue
        k_out[dst] = np.asarray(k_pool[src])
        v_out[dst] = np.asarray(v_pool[src])
    return k_out, v_out


def swap_out_image(k_pool: np.ndarray, v_pool: np.ndarray, blocks: Sequence[int]) -> np.ndarray:
    """The host buffer after swapping out ``blocks``: [n][2][block slab],
    K slab then V slab, each the pool's own bits for that block."""
    k = np.asarray(k_pool)
    v = np.asarray(v_pool)
    slab = k[0].size
    img = np.empty((len(blocks), 2, slab), dtype=k.dtype)
    for p, b in enumerate(blocks):
        img[p, 0] = k[b].reshape(-1)
        img[p, 1] = v[b].reshape(-1)
    return img


def pools_after_swap_in(k_pool: np.ndarray, v_pool: np.ndarray, image: np.ndarray, blocks: Sequence[int]):
    """Both pools after writing the host image's blocks back into ``blocks``."""
    k_out = np.array(k_pool, copy=True)
    v_out = np.array(v_pool, copy=True)
    for p, b in enumerate(blocks):
        k_out[b] = image[p, 0].reshape(k_out[b].shape)
        v_out[b] = image[p, 1].reshape(v_out[b].shape)
    return k_out, v_out
