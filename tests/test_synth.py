"""The seeded generator: determinism and the shapes the workloads state."""

import numpy as np

from synth import workloads as wl


def test_same_seed_same_batch():
    a = wl.config_decode64(unused_fill="zero")
    b = wl.config_decode64(unused_fill="zero")
    for f in ("cu_seqlens_q", "seq_lens", "block_tables", "q", "k_new", "v_new", "k_pool", "v_pool"):
        assert np.array_equal(getattr(a, f), getattr(b, f)), f


def test_worked_step():
    b = wl.config_worked_step()
    assert b.num_blocks == 64 and b.num_seqs == 3 and b.num_rows == 7
    assert list(b.cached_lens) == [0, 7, 3]
    used = b.block_tables[b.block_tables >= 0]
    assert len(set(used.tolist())) == used.size == 3


def test_decode64():
    b = wl.config_decode64(pool="skip")
    c = b.cached_lens
    assert b.num_seqs == 64 and b.num_rows == 64
    assert c.min() >= 128 and c.max() <= 4096
    need = ((b.seq_lens + 15) // 16).sum()
    assert b.num_blocks == int(np.ceil(1.25 * need))


def test_mixed_chunked():
    b = wl.config_mixed_chunked(pool="skip")
    assert b.num_rows == 2048 and b.num_seqs == 1028
    assert list(b.q_lens[:4]) == [256] * 4 and list(b.cached_lens[:4]) == [0, 1024, 2048, 3072]
    dec = b.cached_lens[4:]
    assert (b.q_lens[4:] == 1).all() and dec.min() >= 16 and dec.max() <= 8192
    assert 700 < np.median(dec) < 1400


def test_long_shared_aliasing():
    b = wl.config_long_shared(pool="skip")
    assert b.num_seqs == 16 and (b.seq_lens == 32769).all()
    bt = b.block_tables
    assert bt.shape[1] == 2049
    for g in (0, 8):
        assert (bt[g:g + 8, :128] == bt[g, :128]).all()
    assert not np.intersect1d(bt[0, :128], bt[8, :128]).size
    # private blocks are not shared with anyone
    priv = bt[:, 128:].ravel()
    assert np.unique(priv).size == priv.size
    assert not np.intersect1d(priv, bt[:, :128].ravel()).size
    assert b.num_blocks == int(np.ceil(1.25 * (2 * 128 + 16 * 1921)))


def test_new_rows_never_land_in_shared_blocks():
    b = wl.config_long_shared(pool="skip")
    last = b.block_tables[:, 2048]
    assert not np.isin(last, b.block_tables[:, :128]).any()


def test_permute_placement_keeps_tiles_with_their_table_entries():
    b = wl.make_batch("t", [(40, 2), (3, 1)], seed=5, num_q_heads=4, num_kv_heads=1, head_dim=8)
    p = wl.permute_placement(b, 9)
    for s in range(b.num_seqs):
        for i in range(b.block_tables.shape[1]):
            o, n = b.block_tables[s, i], p.block_tables[s, i]
            assert (o < 0) == (n < 0)
            if o >= 0:
                assert np.array_equal(b.k_pool[o], p.k_pool[n])
                assert np.array_equal(b.v_pool[o], p.v_pool[n])
