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
* [YB] "11.2 连续批处理与 PagedAttention", section 11.2.3 (sharing) and Figure
  11-4: several logical blocks may map to one physical block; within one
  request, parallel samples share all of the prompt's blocks and only the
  last, not yet full block is copied when a sample writes into a block whose
  count is above 1; across requests only full, read-only blocks are shared.
  A request takes a new block only when it has filled its last one.
* [PA] section "抢占策略" and [CB] "Continuous Batching 深入实现", section
  "Preemption 与 Recompute vs Swap": a swapped-out sequence's KV cache is
  copied to CPU memory and copied back when it resumes.
* [YB] section 11.2.4 "前缀缓存": under causal attention a position's K and V
  depend only on it and the tokens left of it, so two requests that start
  with the same tokens have byte-identical KV there and the later one can
  map it and skip that prefill; only full blocks are shared; each full
  block is hashed from its parent block's hash, its tokens and extra keys;
  a finished request's blocks stay in an evictable queue until hit or
  pushed out; reuse needs a token-exact match (one differing token
  invalidates every later block); the key carries everything that changes
  the KV or its visibility.  Worked example: 2,010 shared tokens + 200 user
  tokens, blocks of 16: 125 blocks (2,000 tokens) hit, prefill drops from
  2,210 to 210 tokens, linear-layer work to 9.5%.

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
* the block hash: FNV-1a, 64 bits (the published offset basis and prime),
  over the little-endian bytes of the parent hash (8), the 16 token ids
  (4 each) and one 64-bit extra key into which the caller folds model,
  adapter, multimodal and tenant keys; block 0's parent hash is 0.
* token-exact hits: an entry stores its tokens, its extra key and the serial
  number of its parent entry (serials never repeat); a lookup accepts it
  only if all three equal the prompt's block and the entry matched one
  block before, so a hash collision can never alias other content.
* a prompt matches at most the full blocks that leave one token to compute
  (the step needs a query row to produce the next token).
* registration walks a computed sequence's full blocks from block 0: an
  entry already holding this content is kept (the walk goes on through
  it), an entry under the same hash with other content is replaced, and the
  walk stops at a block already registered under another hash.
* eviction: allocation takes a free block first, else the evictable block
  released longest ago (first in, first out), which loses its
  registration; blocks enter the queue in the order a release lists them.

Parity unpinned: none -- every function below has a pin in
``tests/test_block_pool_oracle.py``.
"""

from __future__ import annotations

import struct
from typing import List, Optional, Sequence, Tuple

import numpy as np

BLOCK = 16

FNV64_OFFSET = 0xCBF29CE484222325
FNV64_PRIME = 0x100000001B3


def fnv1a64(data: bytes) -> int:
    """FNV-1a, 64 bits (Fowler, Noll and Vo): start from the offset basis;
    for every byte, xor it in, then multiply by the prime modulo 2^64."""
    h = FNV64_OFFSET
    for byte in data:
        h ^= byte
        h = (h * FNV64_PRIME) % (1 << 64)
    return h


def block_hash(parent: int, tokens: Sequence[int], extra_key: int = 0) -> int:
    """[YB] 11.2.4: a full block's hash from its parent's hash, its tokens
    and the extra key (byte layout: see the readings above)."""
    assert len(tokens) == BLOCK
    data = struct.pack("<Q", parent % (1 << 64))
    data += b"".join(struct.pack("<I", t % (1 << 32)) for t in tokens)
    data += struct.pack("<Q", extra_key % (1 << 64))
    return fnv1a64(data)


class PoolModel:
    """The block pool as the pages describe it, one Python list per field."""

    def __init__(self, num_blocks: int):
        self.refcount = [0] * num_blocks
        self.free = list(range(num_blocks - 1, -1, -1))  # top of the stack at the end
        # prefix cache: hash -> entry dict(parent_serial, serial, tokens, extra, block)
        self.cache = {}
        self.hash_of = {}            # registered block -> its hash
        self.evictable = []          # registered blocks with count 0, oldest first
        self.next_serial = 1

    def num_free(self) -> int:
        return len(self.free) + len(self.evictable)

    def allocate(self, n: int) -> List[int]:
        if n > self.num_free():
            raise MemoryError("not enough free blocks")
        out = []
        for _ in range(n):
            if self.free:
                b = self.free.pop()
            else:                                    # evict the oldest cached block
                b = self.evictable.pop(0)
                del self.cache[self.hash_of.pop(b)]
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
                if b in self.hash_of:
                    self.evictable.append(b)
                else:
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
        if need - held + int(cow) > self.num_free():
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


    # ------------------------------------------------ prefix caching, [YB] 11.2.4

    def _entry_is(self, e, parent_serial, tokens, extra_key) -> bool:
        return e["parent_serial"] == parent_serial and e["tokens"] == tuple(tokens) and e["extra"] == extra_key

    def match_prefix(self, tokens: Sequence[int], row: List[int], extra_key: int = 0) -> int:
        """Map the prompt's leading cached full blocks into ``row``; each
        gains a reference.  Returns the number of cached tokens."""
        hits = []
        parent, parent_serial = 0, 0
        for b in range(min((len(tokens) - 1) // BLOCK if tokens else 0, len(row))):
            t = list(tokens[b * BLOCK:(b + 1) * BLOCK])
            h = block_hash(parent, t, extra_key)
            e = self.cache.get(h)
            if e is None or not self._entry_is(e, parent_serial, t, extra_key):
                break                                # the first miss ends the prefix
            hits.append(e["block"])
            parent, parent_serial = h, e["serial"]
        for lb, blk in enumerate(hits):
            if self.refcount[blk] == 0:
                self.evictable.remove(blk)
            self.refcount[blk] += 1
            row[lb] = blk
        return BLOCK * len(hits)

    def register_prefix(self, tokens: Sequence[int], row: Sequence[int], extra_key: int = 0) -> None:
        """Make a computed sequence's full blocks findable by content."""
        if any(self.refcount[row[b]] <= 0 for b in range(len(tokens) // BLOCK)):
            raise ValueError("registering a block that is not in use")
        parent, parent_serial = 0, 0
        for b in range(len(tokens) // BLOCK):
            t = list(tokens[b * BLOCK:(b + 1) * BLOCK])
            h = block_hash(parent, t, extra_key)
            blk = row[b]
            e = self.cache.get(h)
            if e is not None and self._entry_is(e, parent_serial, t, extra_key):
                parent_serial = e["serial"]
            else:
                if blk in self.hash_of:
                    break
                if e is not None:                    # other content under this hash
                    old = e["block"]
                    del self.hash_of[old]
                    del self.cache[h]
                    if self.refcount[old] == 0:
                        self.evictable.remove(old)
                        self.free.append(old)
                e = {"parent_serial": parent_serial, "serial": self.next_serial, "tokens": tuple(t),
                     "extra": extra_key, "block": blk}
                self.next_serial += 1
                self.cache[h] = e
                self.hash_of[blk] = h
                parent_serial = e["serial"]
            parent = h


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
