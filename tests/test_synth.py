"""The seeded generator: determinism and the shapes the workloads state."""

import numpy as np

from synth import workloads as wl


def test_same_seed_same_batch():
    a = wl.config_decode64(unused_fill="zero")
    b = wl.config_decode64(unused_fill="zero")
    for f in ("cu_seqlens_q", "seq_lens", "block_tables", "q", "k_new", "v_new"):
        assert np.array_equal(getattr(a, f), getattr(b, f)), f
    blocks = np.array([0, 5, 77, a.num_blocks - 1])
    assert np.array_equal(a.k_pool[blocks], b.k_pool[blocks])
    assert np.array_equal(a.v_pool[blocks], b.v_pool[blocks])
    assert not np.array_equal(a.k_pool[blocks], a.v_pool[blocks])


def test_worked_step():
    b = wl.config_worked_step()
    assert b.num_blocks == 64 and b.num_seqs == 3 and b.num_rows == 7
    assert list(b.cached_lens) == [0, 7, 3]
    used = b.block_tables[b.block_tables >= 0]
    assert len(set(used.tolist())) == used.size == 3


def test_decode64():
    b = wl.config_decode64(pool="lazy")
    c = b.cached_lens
    assert b.num_seqs == 64 and b.num_rows == 64
    assert c.min() >= 128 and c.max() <= 4096
    need = ((b.seq_lens + 15) // 16).sum()
    assert b.num_blocks == int(np.ceil(1.25 * need))


def test_mixed_chunked():
    b = wl.config_mixed_chunked(pool="lazy")
    assert b.num_rows == 2048 and b.num_seqs == 1028
    assert list(b.q_lens[:4]) == [256] * 4 and list(b.cached_lens[:4]) == [0, 1024, 2048, 3072]
    dec = b.cached_lens[4:]
    assert (b.q_lens[4:] == 1).all() and dec.min() >= 16 and dec.max() <= 8192
    assert 700 < np.median(dec) < 1400


def test_long_shared_aliasing():
    b = wl.config_long_shared(pool="lazy")
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
    b = wl.config_long_shared(pool="lazy")
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


def test_counter_numpy_and_torch_forms_agree():
    import torch
    from synth import counter
    rng = np.random.default_rng(0)
    idx = np.concatenate([np.arange(0, 5000), rng.integers(0, 2 ** 40, size=20000)]).astype(np.uint64)
    for seed, stream in ((149002, 4), (1, 1), (2 ** 31 + 7, 5)):
        a = counter.uniform16_np(seed, stream, idx)
        b = counter.uniform16_torch(seed, stream, torch.from_numpy(idx.astype(np.int64))).numpy()
        assert np.array_equal(a.astype(np.int64), b)
        start = 12345
        r_np = counter.normal_bf16_range_np(seed, stream, start, 3000)
        r_t = counter.normal_bf16_range_torch(seed, stream, start, 3000, "cpu").numpy().view(np.uint16)
        assert np.array_equal(r_np, r_t)


def test_counter_values_look_standard_normal():
    from synth import counter
    from oracle import bf16_bits_to_f64
    v = bf16_bits_to_f64(counter.normal_bf16_range_np(7, 3, 0, 1 << 20))
    assert abs(v.mean()) < 0.005 and abs(v.std() - 1) < 0.005
    assert abs((v > 1.0).mean() - 0.158655) < 0.002
    # neighbouring elements are uncorrelated
    assert abs(np.corrcoef(v[:-1], v[1:])[0, 1]) < 0.005


def test_lazy_pool_matches_materialized_and_fills_unused():
    b = wl.make_batch("t", [(40, 2), (3, 1)], seed=5, num_q_heads=4, num_kv_heads=2, head_dim=8,
                      num_blocks=12)
    full = b.k_pool.materialize()
    ref = np.zeros(12, dtype=bool)
    ref[b.block_tables[b.block_tables >= 0]] = True
    assert (full[~ref] == 0x7FC0).all() and not (full[ref] == 0x7FC0).any()
    for blk in range(12):
        assert np.array_equal(b.k_pool[blk], full[blk])
        assert np.array_equal(b.k_pool[blk, 1], full[blk, 1])
