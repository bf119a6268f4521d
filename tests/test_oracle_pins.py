"""Pins of the fp64 oracle against what the pages and the mathematics fix.

None of these compares the oracle with itself: each checks it against a
printed worked example, a closed form, a textbook routine (torch's
scaled_dot_product_attention in float64 on the CPU), a second formulation
written differently, or brute force on tiny inputs.
"""

import math
import os

import numpy as np
import pytest
import torch

import oracle
from oracle import paged_attention as pa
from synth import workloads as wl

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def small_batch(seqs, seed=7, Hq=8, Hkv=2, D=16, **kw):
    return wl.make_batch("t", seqs, seed=seed, num_q_heads=Hq, num_kv_heads=Hkv,
                         head_dim=D, **kw)


# ---------------------------------------------------------------- numbers

def test_bf16_widening_known_patterns():
    bits = np.array([0x3F80, 0xC000, 0x3F00, 0x0000, 0x8000, 0x0001, 0x7F80, 0x4049], dtype=np.uint16)
    v = oracle.bf16_bits_to_f64(bits)
    assert v[0] == 1.0 and v[1] == -2.0 and v[2] == 0.5
    assert v[3] == 0.0 and math.copysign(1.0, v[4]) == -1.0
    assert v[5] == 2.0 ** -133          # smallest bf16 subnormal
    assert v[6] == math.inf
    assert v[7] == 3.140625             # 0x4049: 1.5703125 * 2


def test_generator_rounds_to_nearest_even():
    # 1 + 2^-8 is halfway between bf16 1.0 and 1.0078125: ties go to even (1.0);
    # 1 + 3*2^-8 is halfway between 1.0078125 and 1.015625: goes to even 1.015625
    x = np.array([1 + 2 ** -8, 1 + 3 * 2 ** -8, 1 + 2 ** -8 + 2 ** -20], dtype=np.float32)
    v = oracle.bf16_bits_to_f64(wl.f32_to_bf16_bits(x))
    assert list(v) == [1.0, 1.015625, 1.0078125]


# ---------------------------------------------------------------- slots

def _simulate_paging(tables, lengths, num_blocks):
    """Brute force: walk each sequence's block list and write its token
    numbers into a flat physical memory, 16 cells per block, in order."""
    mem = {}
    for s, (row, n) in enumerate(zip(tables, lengths)):
        p = 0
        for b in row:
            for cell in range(16):
                if p >= n:
                    break
                mem[(s, p)] = b * 16 + cell
                p += 1
    return mem


def test_slot_formula_matches_paging_simulation():
    rng = np.random.default_rng(3)
    nb = 40
    perm = rng.permutation(nb)
    lengths = [1, 16, 17, 33, 70, 5]
    tables, cur = [], 0
    for n in lengths:
        k = (n + 15) // 16
        tables.append(list(perm[cur:cur + k]))
        cur += k
    mem = _simulate_paging(tables, lengths, nb)
    for s, n in enumerate(lengths):
        for p in range(n):
            assert oracle.slot_of(tables[s], p) == mem[(s, p)]


def test_figure_11_4_shared_blocks():
    # [YB] Figure 11-4: A holds 50 tokens in blocks 1, 4, 7, 2; B holds 40 in
    # 1, 4, 8; the first two blocks are full, read-only and shared.
    A, B = [1, 4, 7, 2], [1, 4, 8]
    sa = [oracle.slot_of(A, p) for p in range(50)]
    sb = [oracle.slot_of(B, p) for p in range(40)]
    assert sa[:32] == sb[:32] == list(range(16, 32)) + list(range(64, 80))
    assert sa[49] == 33 and sb[39] == 135
    assert len(set(sa)) == 50 and len(set(sb)) == 40
    assert set(sa[32:]).isdisjoint(sb[32:])


def test_slot_mapping_packed_rows():
    # three sequences: prefill of 3 (nothing cached), decode with 17 cached,
    # chunk of 2 continuing 30 cached
    cu = np.array([0, 3, 4, 6])
    seq_lens = np.array([3, 18, 32])
    bt = np.array([[5, -1], [2, 9], [7, 0]])
    got = oracle.slot_mapping(cu, seq_lens, bt)
    assert list(got) == [80, 81, 82, 9 * 16 + 1, 0 * 16 + 14, 0 * 16 + 15]


# ---------------------------------------------------------------- pool reading

def test_gather_blockwise_equals_token_by_token():
    b = small_batch([(37, 2), (16, 1), (0, 5)], D=16)
    for s in range(b.num_seqs):
        n = int(b.seq_lens[s])
        K1, V1 = pa.gather_kv(b.k_pool, b.v_pool, b.block_tables[s], n, 2, 16)
        K2, V2 = pa.gather_kv_by_token(b.k_pool, b.v_pool, b.block_tables[s], n, 2, 16)
        assert np.array_equal(K1, K2) and np.array_equal(V1, V2)


def test_gather_grouped_k_tiles():
    """D = 64: two 32-dimension groups per K tile.  The block-wise gather
    equals the token-by-token reads, and token o's dimensions 32..63 sit in
    the second group at o * 32 (written out by hand for one token)."""
    b = small_batch([(37, 2), (0, 5)], D=64, pool="materialize")
    for s in range(b.num_seqs):
        n = int(b.seq_lens[s])
        K1, V1 = pa.gather_kv(b.k_pool, b.v_pool, b.block_tables[s], n, 2, 64)
        K2, V2 = pa.gather_kv_by_token(b.k_pool, b.v_pool, b.block_tables[s], n, 2, 64)
        assert np.array_equal(K1, K2) and np.array_equal(V1, V2)
    blk, o, h = int(b.block_tables[0, 1]), 5, 1          # position 21 of sequence 0
    tile = b.k_pool[blk, h]
    by_hand = np.concatenate([tile[o * 32:(o + 1) * 32], tile[512 + o * 32:512 + (o + 1) * 32]])
    K, _ = pa.gather_kv(b.k_pool, b.v_pool, b.block_tables[0], 37, 2, 64)
    assert np.array_equal(K[21, h], oracle.bf16_bits_to_f64(by_hand))


def test_append_round_trip_and_untouched_tiles():
    b = small_batch([(37, 3), (15, 1), (0, 16)], D=16, unused_fill="normal", pool="materialize")
    slots = oracle.slot_mapping(b.cu_seqlens_q, b.seq_lens, b.block_tables)
    slots_skip = slots.copy()
    slots_skip[1] = -1
    k2, v2 = oracle.pools_after_append(b.k_pool, b.v_pool, slots_skip, b.k_new, b.v_new)
    touched = set()
    for s in range(b.num_seqs):
        n = int(b.seq_lens[s])
        q_len = int(b.cu_seqlens_q[s + 1] - b.cu_seqlens_q[s])
        K, V = pa.gather_kv(k2, v2, b.block_tables[s], n, 2, 16)
        for j in range(q_len):
            t = int(b.cu_seqlens_q[s]) + j
            if t == 1:
                continue
            assert np.array_equal(K[n - q_len + j], oracle.bf16_bits_to_f64(b.k_new[t]))
            assert np.array_equal(V[n - q_len + j], oracle.bf16_bits_to_f64(b.v_new[t]))
    # exactly the written elements changed
    changed_k = np.argwhere(k2 != b.k_pool)
    for blk, h, e in changed_k:
        touched.add((int(blk), int(h), int(e) // 16))
    expect = set()
    for t, x in enumerate(slots_skip):
        if x < 0:
            continue
        for h in range(2):
            expect.add((int(x) // 16, h, int(x) % 16))
    assert touched <= expect  # identical values may coincide; nothing else moved
    changed_v = np.argwhere(v2 != b.v_pool)
    for blk, h, e in changed_v:  # V tile: halves of 8 tokens, each [D][8]
        o = (int(e) // (8 * 16)) * 8 + int(e) % 8
        assert (int(blk), int(h), o) in expect
    # the skipped row's slot kept its old contents
    x = int(slots[1])
    assert np.array_equal(k2[x // 16, :, (x % 16) * 16:(x % 16 + 1) * 16],
                          b.k_pool[x // 16, :, (x % 16) * 16:(x % 16 + 1) * 16])


# ---------------------------------------------------------------- worked examples

def test_worked_step_shapes():
    # [YB] 11.2.2: R1 prefill 5 (0 cached), R2 decode (7 cached), R3 decode
    # (3 cached): 7 packed rows, per-head scores [5,5], [1,8], [1,4]
    b = wl.config_worked_step()
    assert list(b.cu_seqlens_q) == [0, 5, 6, 7]
    assert list(b.seq_lens) == [5, 8, 4]
    assert b.num_rows == 7 and b.q.shape == (7, 32, 128) and b.k_new.shape == (7, 8, 128)
    assert oracle.score_shapes(b.cu_seqlens_q, b.seq_lens) == [(5, 5), (1, 8), (1, 4)]
    grid = oracle.visibility_grid([0, 7, 3], [5, 1, 1])
    # R1's block of the grid is the 5x5 lower triangle; R2 sees 8 keys, R3 4
    assert grid.sum(axis=1).tolist() == [1, 2, 3, 4, 5, 8, 4]


def _render(grid, kv_lens, q_lens, labels):
    total_kv = sum(kv_lens)
    key_seq = [s for s, c in enumerate(kv_lens) for _ in range(c)]
    key_seq += [s for s, n in enumerate(q_lens) for _ in range(n)]
    q_seq = [s for s, n in enumerate(q_lens) for _ in range(n)]
    q_pos = [kv_lens[s] + j for s, n in enumerate(q_lens) for j in range(n)]
    lines = []
    for qi in range(grid.shape[0]):
        out = []
        for ki in range(grid.shape[1]):
            if total_kv > 0 and ki == total_kv:
                out.append(" | ")
            elif ki > 0 and key_seq[ki] != key_seq[ki - 1]:
                out.append(" ")
            out.append("#" if grid[qi, ki] else ".")
        lines.append(f"{labels[q_seq[qi]]} p{q_pos[qi]} " + "".join(out))
    return lines


def _load_grid(name):
    meta, rows = {}, []
    with open(os.path.join(GOLDEN, name), encoding="utf-8") as f:
        for line in f:
            line = line.rstrip("\n")
            if line.startswith("# ") and ":" in line and line[2:].split(":")[0] in ("kv_lens", "q_lens", "labels"):
                k, v = line[2:].split(":", 1)
                meta[k] = v.split()
            elif line and not line.startswith("#"):
                rows.append(line)
    return [int(x) for x in meta["kv_lens"]], [int(x) for x in meta["q_lens"]], meta["labels"], rows


@pytest.mark.parametrize("name", ["mlm_mask_step1.txt", "mlm_mask_step7.txt"])
def test_printed_mask_grids(name):
    kv, ql, labels, rows = _load_grid(name)
    grid = oracle.visibility_grid(kv, ql)
    got = _render(grid, kv, ql, labels)
    assert [r.split() for r in got] == [r.split() for r in rows]


def test_mixed_iteration_visibility():
    # [K4I] "一个完整的 mixed iteration": A 3 prefill rows, B one decode row at
    # position 5 (B1..B4 cached), C 2 prefill rows; 6 packed rows
    grid = oracle.visibility_grid([0, 4, 0], [3, 1, 2])
    assert grid.shape == (6, 4 + 6)
    assert grid.sum(axis=1).tolist() == [1, 2, 3, 5, 1, 2]
    # B's row sees exactly B's 4 cached keys and its own new key
    assert np.nonzero(grid[3])[0].tolist() == [0, 1, 2, 3, 7]


def test_cu_seqlens_example():
    # [CB] "Ragged Batch + cu_seqlens": a 500-token prefill and one decode row
    # over a 2048-token history give cu_seqlens_q [0,500,501] and cumulative
    # key counts [0,500,2548]
    q_lens = [500, 1]
    seq_lens = [500, 2048]
    assert list(np.concatenate([[0], np.cumsum(q_lens)])) == [0, 500, 501]
    assert list(np.concatenate([[0], np.cumsum(seq_lens)])) == [0, 500, 2548]
    assert oracle.score_shapes([0, 500, 501], seq_lens) == [(500, 500), (1, 2048)]


def test_chunked_prefill_offset_shape():
    # [CB] chunked prefill, iteration 2: Q of 512 rows against K/V of 1024
    grid = oracle.visibility_grid([512], [512])
    assert grid.shape == (512, 1024)
    assert grid.sum(axis=1).tolist() == list(range(513, 1025))


# ---------------------------------------------------------------- attention

def _sdpa_causal(q, K, V, scale):
    """torch SDPA (float64, CPU) on one request with GQA expanded."""
    n, Hq, D = q.shape
    G = Hq // K.shape[1]
    qt = torch.from_numpy(q).permute(1, 0, 2)[None]
    kt = torch.from_numpy(K).permute(1, 0, 2).repeat_interleave(G, dim=0)[None]
    vt = torch.from_numpy(V).permute(1, 0, 2).repeat_interleave(G, dim=0)[None]
    return None, qt, kt, vt


def sdpa(q, K, V, scale, causal_offset):
    """q rows sit at positions causal_offset .. ; keys at 0 .. len(K)-1."""
    _, qt, kt, vt = _sdpa_causal(q, K, V, scale)
    n, L = q.shape[0], K.shape[0]
    mask = torch.arange(L)[None, :] <= (causal_offset + torch.arange(n))[:, None]
    out = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, attn_mask=mask, scale=scale)
    return out[0].permute(1, 0, 2).numpy()


def test_textbook_single_request_no_cache():
    rng = np.random.default_rng(11)
    n, Hq, Hkv, D = 9, 8, 2, 32
    q, K, V = rng.standard_normal((n, Hq, D)), rng.standard_normal((n, Hkv, D)), rng.standard_normal((n, Hkv, D))
    s = 1 / math.sqrt(D)
    ours = oracle.attention_one_request(q, K, V, 0, s)
    qt = torch.from_numpy(q).permute(1, 0, 2)[None]
    kt = torch.from_numpy(K).permute(1, 0, 2).repeat_interleave(Hq // Hkv, dim=0)[None]
    vt = torch.from_numpy(V).permute(1, 0, 2).repeat_interleave(Hq // Hkv, dim=0)[None]
    ref = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, is_causal=True, scale=s)
    assert np.abs(ours - ref[0].permute(1, 0, 2).numpy()).max() < 1e-12


def test_chunk_with_prefix_equals_rows_of_full_causal():
    # a chunk continuing c cached tokens gives the last rows of one causal
    # pass over the whole sequence ([CB] chunked prefill)
    rng = np.random.default_rng(12)
    c, n, Hq, Hkv, D = 21, 6, 8, 2, 32
    L = c + n
    qf, K, V = rng.standard_normal((L, Hq, D)), rng.standard_normal((L, Hkv, D)), rng.standard_normal((L, Hkv, D))
    s = 0.3
    ours = oracle.attention_one_request(qf[c:], K, V, c, s)
    qt = torch.from_numpy(qf).permute(1, 0, 2)[None]
    kt = torch.from_numpy(K).permute(1, 0, 2).repeat_interleave(4, dim=0)[None]
    vt = torch.from_numpy(V).permute(1, 0, 2).repeat_interleave(4, dim=0)[None]
    full = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, is_causal=True, scale=s)
    assert np.abs(ours - full[0].permute(1, 0, 2).numpy()[c:]).max() < 1e-12


def test_mha_reduction():
    rng = np.random.default_rng(13)
    n, H, D = 5, 3, 16
    q, K, V = rng.standard_normal((n, H, D)), rng.standard_normal((n, H, D)), rng.standard_normal((n, H, D))
    ours = oracle.attention_one_request(q, K, V, 0, 0.25)
    for h in range(H):
        ref = oracle.attention_one_request(q[:, h:h + 1], K[:, h:h + 1], V[:, h:h + 1], 0, 0.25)
        assert np.array_equal(ours[:, h], ref[:, 0])
    qt = torch.from_numpy(q).permute(1, 0, 2)[None]
    kt = torch.from_numpy(K).permute(1, 0, 2)[None]
    vt = torch.from_numpy(V).permute(1, 0, 2)[None]
    ref = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, is_causal=True, scale=0.25)
    assert np.abs(ours - ref[0].permute(1, 0, 2).numpy()).max() < 1e-12


def test_packed_step_against_sdpa_per_request():
    b = small_batch([(37, 3), (0, 7), (16, 1), (5, 1), (31, 2)], D=32, Hq=8, Hkv=2)
    out = oracle.packed_attention(b)
    st = oracle.step_from_batch(b)
    for s in range(b.num_seqs):
        r = slice(int(b.cu_seqlens_q[s]), int(b.cu_seqlens_q[s + 1]))
        n = r.stop - r.start
        c = int(b.seq_lens[s]) - n
        Kc, Vc = pa.gather_kv_by_token(b.k_pool, b.v_pool, b.block_tables[s], c, 2, 32)
        K = np.concatenate([Kc, st["k_new"][r]])
        V = np.concatenate([Vc, st["v_new"][r]])
        ref = sdpa(st["q"][r], K, V, st["scale"], c)
        assert np.abs(out[r] - ref).max() < 1e-12


def test_two_formulations_agree_worked_step():
    b = wl.config_worked_step()
    a1 = oracle.packed_attention(b)
    a2 = oracle.dense_mask_attention(b)
    assert np.abs(a1 - a2).max() < 1e-12


def test_two_formulations_agree_mixed_subsample():
    b = wl.config_mixed_chunked(n_decode=24)
    sel = [0, 1, 4, 9, 17, 27]      # two chunks (prefix 0, 1024) + four decode rows
    a2 = oracle.dense_mask_attention(b, sel)
    a1 = oracle.packed_attention(b, sel)
    rows = np.concatenate([np.arange(b.cu_seqlens_q[s], b.cu_seqlens_q[s + 1]) for s in sel])
    assert np.abs(a1[rows] - a2).max() < 1e-12


def test_packed_equals_separate():
    b = small_batch([(20, 3), (0, 4), (9, 1)], D=16)
    packed = oracle.packed_attention(b)
    for s in range(b.num_seqs):
        r = slice(int(b.cu_seqlens_q[s]), int(b.cu_seqlens_q[s + 1]))
        sub = wl.Batch(**{**b.__dict__,
                          "cu_seqlens_q": np.array([0, r.stop - r.start], dtype=np.int32),
                          "seq_lens": b.seq_lens[s:s + 1], "block_tables": b.block_tables[s:s + 1],
                          "q": b.q[r], "k_new": b.k_new[r], "v_new": b.v_new[r]})
        alone = oracle.packed_attention(sub)
        assert np.array_equal(alone, packed[r])


def test_rows_sampler_matches_full():
    b = small_batch([(20, 3), (0, 4), (9, 1)], D=16)
    full = oracle.packed_attention(b)
    got = oracle.packed_attention_rows(b, [0, 2, 5, 7])
    for t, o in got.items():
        assert np.abs(o - full[t]).max() < 1e-13


def test_placement_invariance():
    b = small_batch([(40, 2), (3, 1), (0, 6)], D=16, unused_fill="normal")
    base = oracle.packed_attention(b)
    for seed in (1, 2, 3):
        p = wl.permute_placement(b, seed)
        assert not np.array_equal(p.block_tables, b.block_tables)
        assert np.array_equal(oracle.packed_attention(p), base)


def test_single_visible_key_returns_its_value():
    # position 0 sees only itself (first row of the printed grids)
    b = small_batch([(0, 4), (0, 1)], D=16)
    out = oracle.packed_attention(b)
    v = oracle.bf16_bits_to_f64(b.v_new)
    for t in (0, 4):
        for h in range(8):
            assert np.array_equal(out[t, h], v[t, h // 4])


def test_constant_values_give_the_constant():
    b = small_batch([(33, 2), (7, 1)], D=16, pool="materialize")
    c = wl.f32_to_bf16_bits(np.array([1.25, -0.5], dtype=np.float32))
    b.v_pool[:, 0, :] = c[0]
    b.v_pool[:, 1, :] = c[1]
    b.v_new[:, 0, :] = c[0]
    b.v_new[:, 1, :] = c[1]
    out = oracle.packed_attention(b)
    assert np.abs(out[:, :4] - 1.25).max() < 1e-15
    assert np.abs(out[:, 4:] + 0.5).max() < 1e-15


def test_zero_query_gives_mean_of_visible_values():
    b = small_batch([(29, 3)], D=16)
    b.q[:] = 0
    out = oracle.packed_attention(b)
    K, V = pa.gather_kv_by_token(b.k_pool, b.v_pool, b.block_tables[0], 29, 2, 16)
    V = np.concatenate([V, oracle.bf16_bits_to_f64(b.v_new)])
    for j in range(3):
        mean = V[:29 + j + 1].mean(axis=0)
        for h in range(8):
            assert np.abs(out[j, h] - mean[h // 4]).max() < 1e-14
