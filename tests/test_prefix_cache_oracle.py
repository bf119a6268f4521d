"""The prefix cache of the block-pool oracle pinned to the pages and to the
hash's published definition, and the library's pool checked against it id
for id (host code only, no GPU).  [YB] "11.2 连续批处理与 PagedAttention",
section 11.2.4."""

import numpy as np
import pytest

import paged_kv_cache_149_amd as pkv
from oracle import block_pool as bp

BLOCK = 16


# ------------------------------------------------- the hash: published test vectors

@pytest.mark.parametrize("data,expected", [
    (b"", 0xCBF29CE484222325),
    (b"a", 0xAF63DC4C8601EC8C),
    (b"foobar", 0x85944171F73967E8),
])
def test_fnv1a64_published_vectors(data, expected):
    """FNV-1a 64 of the empty string is the offset basis; "a" and "foobar"
    are the FNV authors' test vectors."""
    assert bp.fnv1a64(data) == expected


def test_block_hash_byte_layout():
    """Parent (8 bytes LE), 16 tokens (4 bytes LE each), extra key (8 bytes
    LE): the hash over that byte string, built here by hand."""
    toks = list(range(100, 116))
    data = (7).to_bytes(8, "little") + b"".join(t.to_bytes(4, "little") for t in toks) \
        + (9).to_bytes(8, "little")
    assert bp.block_hash(7, toks, 9) == bp.fnv1a64(data)
    assert bp.block_hash(0, [-1] * 16) == bp.fnv1a64(bytes(8) + b"\xff" * 64 + bytes(8))


# ------------------------------------------------- the worked example of 11.2.4

def _prompt(shared, own, seed):
    rng = np.random.default_rng(seed)
    return list(shared) + rng.integers(0, 50000, size=own).tolist()


def _run_request(pool, tokens, cap=256, extra=0):
    """Admit a request: match, then allocate the rest; returns (row, cached)."""
    row = [-1] * cap
    cached = pool.match_prefix(tokens, row, extra)
    assert pool.append_slots(row, cached, len(tokens) - cached) is None
    return row, cached


def _finish(pool, row, n_tokens):
    held = -(-n_tokens // BLOCK)
    pool.release(row[:held][::-1])           # last block first


def test_worked_example_2010_shared_200_own():
    """2,010 shared tokens + 200 own, blocks of 16: the second request hits
    floor(2010 / 16) = 125 blocks (2,000 tokens) and prefills 210 of its
    2,210 tokens, 9.5 % of the work of the linear layers."""
    shared = np.random.default_rng(0).integers(0, 50000, size=2010).tolist()
    pool = bp.PoolModel(400)
    a = _prompt(shared, 200, 1)
    row_a, cached_a = _run_request(pool, a)
    assert cached_a == 0
    pool.register_prefix(a, row_a)
    _finish(pool, row_a, len(a))
    b = _prompt(shared, 200, 2)
    assert b[2010] != a[2010]
    row_b, cached_b = _run_request(pool, b)
    assert cached_b == 2000 and cached_b // BLOCK == 125 == 2010 // BLOCK
    assert len(b) - cached_b == 210
    assert round(100 * (len(b) - cached_b) / len(b), 1) == 9.5
    assert row_b[:125] == row_a[:125] and row_b[125] != row_a[125]
    # the hit blocks are in use once more; A's other blocks stay evictable
    assert all(pool.refcount[x] == 1 for x in row_b[:139])


def test_one_differing_token_invalidates_every_later_block():
    rng = np.random.default_rng(3)
    a = rng.integers(0, 1000, size=160).tolist()        # ten full blocks
    for p in [0, 15, 16, 37, 100, 158]:
        pool = bp.PoolModel(64)
        row_a, _ = _run_request(pool, a, 16)
        pool.register_prefix(a, row_a)
        b = list(a)
        b[p] += 1
        row_b = [-1] * 16
        assert pool.match_prefix(b, row_b) == BLOCK * (p // BLOCK)


def test_extra_key_separates_equal_tokens():
    """The key carries whatever changes the KV or its visibility (model,
    adapter, tenant salt): equal tokens under another extra key never hit."""
    a = list(range(64))
    pool = bp.PoolModel(32)
    row_a, _ = _run_request(pool, a, 8, extra=1)
    pool.register_prefix(a, row_a, extra_key=1)
    assert pool.match_prefix(a + [0], [-1] * 8, extra_key=2) == 0
    assert pool.match_prefix(a + [0], [-1] * 8, extra_key=1) == 64


def test_a_prompt_keeps_one_token_to_compute():
    """A prompt that is exactly four registered full blocks hits three: the
    step needs the last prompt token as a query row."""
    a = list(range(64))
    pool = bp.PoolModel(16)
    row_a, _ = _run_request(pool, a, 8)
    pool.register_prefix(a, row_a)
    assert pool.match_prefix(a, [-1] * 8) == 48
    assert pool.match_prefix(a + [5], [-1] * 8) == 64


def test_eviction_takes_free_blocks_first_then_the_oldest_released():
    pool = bp.PoolModel(8)
    a = list(range(80))                                 # five full blocks
    row_a, _ = _run_request(pool, a, 8)
    pool.register_prefix(a, row_a)
    _finish(pool, row_a, 80)
    assert pool.num_free() == 8 and len(pool.evictable) == 5 and len(pool.free) == 3
    got = pool.allocate(4)                              # three free, then A's last block
    assert got[3] == row_a[4] and row_a[4] not in pool.hash_of
    row = [-1] * 8
    assert pool.match_prefix(a, row) == 64              # blocks 0..3 still cached
    assert row[:4] == row_a[:4] and pool.evictable == []
    with pytest.raises(MemoryError):
        pool.allocate(1)                                # hit blocks left the queue
    pool.release(got)
    _finish(pool, row, 64)
    assert pool.evictable == row_a[:4][::-1]


def test_a_hash_collision_never_aliases(monkeypatch):
    """With every block hashing alike, lookups still compare tokens, extra
    key and parent entry: no prompt ever maps a block of other content."""
    monkeypatch.setattr(bp, "block_hash", lambda parent, tokens, extra_key=0: 42)
    pool = bp.PoolModel(32)
    a = list(range(48))
    row_a, _ = _run_request(pool, a, 8)
    pool.register_prefix(a, row_a)
    assert pool.match_prefix([1000 + t for t in a] + [0], [-1] * 8) == 0
    # only one entry fits under the one hash: a prompt reaches at most block 0
    assert pool.match_prefix(a + [0], [-1] * 8) in (0, BLOCK)


# ------------------------------------------------- brute force over a content model

WORDS = [[w * 100 + i for i in range(BLOCK)] for w in range(3)]


def _family_prompt(rng):
    """Prompts built from three 16-token words, so that equal blocks follow
    different prefixes, plus a ragged tail."""
    n_words = int(rng.integers(0, 6))
    toks = []
    for _ in range(n_words):
        toks += WORDS[int(rng.integers(0, 3))]
    return toks + rng.integers(0, 3, size=int(rng.integers(1, 20))).tolist()


def simulate_prefix_cache(steps=600, seed=7, num_blocks=40):
    """Requests arrive (match, allocate, compute the rest), register their
    blocks and finish at random under block pressure.  A block's content is
    modelled as the whole token prefix its KV depends on (causal
    attention), written when computed.  Every hit must hold exactly the
    prompt's prefix, and live requests' blocks must never change."""
    rng = np.random.default_rng(seed)
    pool = bp.PoolModel(num_blocks)
    content = {}
    live = []                                           # (tokens, row)
    hits_total = 0
    for _ in range(steps):
        if live and rng.integers(0, 3) == 0:
            i = int(rng.integers(len(live)))
            toks, row = live.pop(i)
            _finish(pool, row, len(toks))
        else:
            toks = _family_prompt(rng)
            row = [-1] * 8
            cached = pool.match_prefix(toks, row)
            for lb in range(cached // BLOCK):
                assert content[row[lb]] == tuple(toks[:(lb + 1) * BLOCK])
            hits_total += cached // BLOCK
            try:
                assert pool.append_slots(row, cached, len(toks) - cached) is None
            except MemoryError:
                pool.release(row[:cached // BLOCK])
                continue
            for lb in range(cached // BLOCK, -(-len(toks) // BLOCK)):
                content[row[lb]] = tuple(toks[:min((lb + 1) * BLOCK, len(toks))])
            pool.register_prefix(toks, row)
            live.append((toks, row))
        refs = [0] * num_blocks
        for toks, row in live:
            for lb in range(-(-len(toks) // BLOCK)):
                refs[row[lb]] += 1
                assert content[row[lb]] == tuple(toks[:min((lb + 1) * BLOCK, len(toks))])
        assert refs == pool.refcount
        in_use = {b for b in range(num_blocks) if pool.refcount[b] > 0}
        assert set(pool.free).isdisjoint(in_use) and set(pool.evictable).isdisjoint(in_use)
        assert len(pool.free) + len(pool.evictable) + len(in_use) == num_blocks
        assert set(pool.evictable) <= set(pool.hash_of) <= set(pool.evictable) | in_use
        assert {e["block"] for e in pool.cache.values()} == set(pool.hash_of)
    return hits_total


def test_brute_force_hits_are_exact_and_live_blocks_stay_put():
    assert simulate_prefix_cache() > 50


def test_pins_catch_a_cache_that_ignores_the_parent(monkeypatch):
    monkeypatch.setattr(bp.PoolModel, "_entry_is",
                        lambda self, e, ps, t, x: e["tokens"] == tuple(t) and e["extra"] == x)
    orig = bp.block_hash
    monkeypatch.setattr(bp, "block_hash", lambda parent, tokens, extra_key=0: orig(0, tokens, extra_key))
    with pytest.raises(AssertionError):
        simulate_prefix_cache()


def test_pins_catch_a_hit_that_stays_evictable(monkeypatch):
    orig = bp.PoolModel.match_prefix

    def leaky(self, tokens, row, extra_key=0):
        queue = list(self.evictable)
        n = orig(self, tokens, row, extra_key)
        self.evictable[:] = [b for b in queue if b in self.evictable or b in row[:n // BLOCK]]
        return n

    monkeypatch.setattr(bp.PoolModel, "match_prefix", leaky)
    with pytest.raises(AssertionError):
        simulate_prefix_cache()


# ------------------------------------------------- the library's pool vs the model

def test_library_block_hash_matches_the_oracle():
    rng = np.random.default_rng(2)
    for _ in range(50):
        parent = int(rng.integers(0, 2**63)) * 2 + int(rng.integers(0, 2))
        toks = rng.integers(-2**31, 2**31, size=BLOCK).tolist()
        extra = int(rng.integers(0, 2**63))
        assert pkv.pkv_block_hash(parent, toks, extra) == bp.block_hash(parent, toks, extra)


def test_library_prefix_cache_matches_model_id_for_id():
    rng = np.random.default_rng(13)
    N = 40
    lib, model = pkv.BlockPool(N), bp.PoolModel(N)
    live = []                                           # (tokens, lib row, model row, extra)
    for step in range(700):
        op = int(rng.integers(0, 3))
        if live and op == 0:
            i = int(rng.integers(len(live)))
            toks, rl, rm, _ = live.pop(i)
            held = -(-len(toks) // BLOCK)
            order = slice(None, None, -1) if rng.integers(0, 2) else slice(None)
            model.release(rm[:held][order])
            lib.release(rl[:held][order])
        else:
            toks = _family_prompt(rng)
            extra = int(rng.integers(0, 2)) << 63
            rl, rm = np.full(8, -1, np.int32), [-1] * 8
            cm = model.match_prefix(toks, rm, extra)
            assert lib.match_prefix(toks, rl, extra) == cm
            assert rl.tolist() == rm
            try:
                pm = model.append_slots(rm, cm, len(toks) - cm)
            except MemoryError:
                with pytest.raises(pkv.PKVError):
                    lib.append_slots(rl, cm, len(toks) - cm)
                model.release(rm[:cm // BLOCK])
                lib.release(rl[:cm // BLOCK])
            else:
                assert lib.append_slots(rl, cm, len(toks) - cm) == pm
                if op == 1 or rng.integers(0, 4):
                    model.register_prefix(toks, rm, extra)
                    lib.register_prefix(toks, rl, extra)
                live.append((toks, rl, rm, extra))
        for _, rl, rm, _ in live:
            assert rl.tolist() == rm
        assert lib.num_free == model.num_free() and lib.num_cached == len(model.cache)
        assert [lib.refcount(b) for b in range(N)] == model.refcount


def test_library_prefix_cache_errors():
    p = pkv.BlockPool(4)
    row = np.full(4, -1, np.int32)
    with pytest.raises(pkv.PKVError):
        p.register_prefix(list(range(32)), row)         # blocks not in use
    with pytest.raises(TypeError):
        p.match_prefix(list(range(32)), np.full(4, -1, np.int64))
    assert p.match_prefix([], row) == 0 and p.match_prefix([1], row) == 0
    assert p.num_cached == 0 and p.num_free == 4
