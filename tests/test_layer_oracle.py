"""The packed-layer oracle pinned to the pages and to closed forms (host
only, no GPU): positions of the worked step, projections against explicit
sums, RoPE against its complex-number form and its invariants, and the
layer's wiring against the attention oracle."""

import numpy as np
import pytest

import oracle
from oracle import layer as L
from synth import workloads as wl

D = 128


def test_positions_of_the_worked_step():
    """[YB] 11.2.2: R1 prefills positions 0..4, R2 decodes at 7 (7 cached),
    R3 at 3 (3 cached); cu_seqlens [0, 5, 6, 7], seq_lens [5, 8, 4]."""
    assert L.row_positions([0, 5, 6, 7], [5, 8, 4]).tolist() == [0, 1, 2, 3, 4, 7, 3]
    # a chunk continuing a 1024-token prefix, and an empty sequence
    assert L.row_positions([0, 3, 3], [1027, 9]).tolist() == [1024, 1025, 1026]


def test_projection_shapes_of_the_worked_step():
    """[YB] 11.2.2: X[7, 4096] x W_Q -> Q[7, 4096]; X x W_K -> K[7, 1024]
    (32 query heads, 8 kv heads of 128)."""
    rng = np.random.default_rng(0)
    x = rng.standard_normal((7, 4096))
    w = rng.standard_normal((6144, 4096)) / 64
    q, k, v = L.qkv_rope(x, w, L.row_positions([0, 5, 6, 7], [5, 8, 4]), 32, 8, D)
    assert q.reshape(7, -1).shape == (7, 4096) and k.reshape(7, -1).shape == (7, 1024)
    assert v.shape == (7, 8, D)


def test_linear_is_the_explicit_sum():
    rng = np.random.default_rng(1)
    x = rng.standard_normal((3, 5))
    w = rng.standard_normal((4, 5))
    y = L.linear(x, w)
    for m in range(3):
        for n in range(4):
            assert y[m, n] == pytest.approx(sum(x[m, k] * w[n, k] for k in range(5)), abs=1e-12)


def test_rope_matches_its_complex_form():
    """RoFormer's rotation written independently: the pair (x_i, x_{i+D/2})
    as the complex number x_i + 1j x_{i+D/2}, multiplied by
    exp(1j * p * theta^(-2i/D))."""
    rng = np.random.default_rng(2)
    x = rng.standard_normal((6, 3, D))
    pos = np.array([0, 1, 7, 100, 4095, 32768])
    got = L.rope(x, pos)
    half = D // 2
    for r in range(6):
        for h in range(3):
            for i in range(half):
                z = complex(x[r, h, i], x[r, h, i + half])
                z *= np.exp(1j * pos[r] * L.LLAMA3_ROPE_THETA ** (-2.0 * i / D))
                assert got[r, h, i] == pytest.approx(z.real, abs=1e-9)
                assert got[r, h, i + half] == pytest.approx(z.imag, abs=1e-9)


def test_rope_invariants():
    rng = np.random.default_rng(3)
    x = rng.standard_normal((4, 2, D))
    # position 0 leaves the vector unchanged
    assert np.allclose(L.rope(x, np.zeros(4, int)), x, atol=0)
    # every pair keeps its length
    y = L.rope(x, np.array([3, 50, 999, 8191]))
    half = D // 2
    assert np.allclose(np.hypot(y[..., :half], y[..., half:]), np.hypot(x[..., :half], x[..., half:]))
    # a query-key dot product depends only on the distance of their positions
    q, k = rng.standard_normal((1, 1, D)), rng.standard_normal((1, 1, D))
    dot = lambda m, n: float((L.rope(q, np.array([m])) * L.rope(k, np.array([n]))).sum())
    assert dot(10, 3) == pytest.approx(dot(1010, 1003), abs=1e-9)
    assert dot(10, 3) != pytest.approx(dot(10, 4), abs=1e-6)
    # the first pair turns by exactly p radians (theta^0 = 1)
    e = np.zeros((1, 1, D))
    e[0, 0, 0] = 1.0
    r = L.rope(e, np.array([2]))
    assert r[0, 0, 0] == pytest.approx(np.cos(2.0)) and r[0, 0, half] == pytest.approx(np.sin(2.0))


def test_layer_wiring_reduces_to_the_attention_oracle():
    """With identity blocks for W_QKV (x holds q, k and v side by side) and
    identity for W_O, the layer is rope on q and k, then the packed step's
    attention on the rotated rows, bit for bit in fp64."""
    b = wl.config_worked_step(pool="materialize")
    T = b.num_rows
    Hq, Hkv = b.num_q_heads, b.num_kv_heads
    width = (Hq + 2 * Hkv) * D
    rng = np.random.default_rng(4)
    x = rng.standard_normal((T, width))
    w_qkv = np.eye(width)
    w_o = np.eye(Hq * D)
    kp, vp = np.asarray(b.k_pool), np.asarray(b.v_pool)
    y, q, k, v, attn = L.layer_forward(x, w_qkv, w_o, b.cu_seqlens_q, b.seq_lens, b.block_tables, kp, vp,
                                       Hq, Hkv, D, float(b.scale))
    pos = L.row_positions(b.cu_seqlens_q, b.seq_lens)
    assert np.array_equal(q, L.rope(x[:, :Hq * D].reshape(T, Hq, D), pos))
    assert np.array_equal(v, x[:, (Hq + Hkv) * D:].reshape(T, Hkv, D))
    ref = np.empty((T, Hq, D))
    for s in range(len(b.seq_lens)):
        rows = slice(int(b.cu_seqlens_q[s]), int(b.cu_seqlens_q[s + 1]))
        c = int(b.seq_lens[s]) - (rows.stop - rows.start)
        Kc, Vc = oracle.gather_kv(kp, vp, b.block_tables[s], c, Hkv, D)
        ref[rows] = oracle.attention_one_request(q[rows], np.concatenate([Kc, k[rows]]),
                                                 np.concatenate([Vc, v[rows]]), c, float(b.scale))
    assert np.array_equal(attn, ref)
    assert np.allclose(y, attn.reshape(T, -1), atol=0)


def test_pins_catch_adjacent_pairs(monkeypatch):
    """A RoPE pairing (2i, 2i+1) instead of (i, i + D/2) fails the complex form."""
    def adjacent(x, positions, theta=L.LLAMA3_ROPE_THETA):
        x = np.asarray(x, dtype=np.float64)
        a = L.rope_angles(positions, x.shape[-1], theta)[:, None, :]
        c, s = np.cos(a), np.sin(a)
        x1, x2 = x[..., 0::2], x[..., 1::2]
        out = np.empty_like(x)
        out[..., 0::2], out[..., 1::2] = x1 * c - x2 * s, x2 * c + x1 * s
        return out
    monkeypatch.setattr(L, "rope", adjacent)
    with pytest.raises(AssertionError):
        test_rope_matches_its_complex_form()


def test_pins_catch_a_backward_rotation(monkeypatch):
    orig = L.rope
    monkeypatch.setattr(L, "rope", lambda x, p, theta=L.LLAMA3_ROPE_THETA: orig(x, -np.asarray(p), theta))
    with pytest.raises(AssertionError):
        test_rope_matches_its_complex_form()


def test_pins_catch_positions_off_by_one(monkeypatch):
    orig = L.row_positions
    monkeypatch.setattr(L, "row_positions", lambda cu, sl: orig(cu, sl) + 1)
    with pytest.raises(AssertionError):
        test_positions_of_the_worked_step()
