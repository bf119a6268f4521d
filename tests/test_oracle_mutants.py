"""Plant plausible mistakes in the oracle (on the CPU) and check that the
pins catch every one of them: a pin set that a wrong oracle also passes
would prove nothing."""

import numpy as np
import pytest

import oracle
from oracle import paged_attention as pa
import tests.test_oracle_pins as pins


def _attn(q, K, V, cached, scale, *, gqa="div", causal="le", use_scale=True,
          swap_kv=False, norm_axis=1, offset=0):
    n, Hq, D = q.shape
    L, Hkv, _ = K.shape
    G = Hq // Hkv
    if swap_kv:
        K, V = V, K
    out = np.empty((n, Hq, D))
    for h in range(Hq):
        g = h // G if gqa == "div" else h % Hkv
        sc = q[:, h, :] @ K[:, g, :].T
        if use_scale:
            sc = sc * scale
        pos = cached + offset + np.arange(n)[:, None]
        vis = (np.arange(L)[None, :] <= pos) if causal == "le" else (np.arange(L)[None, :] < pos)
        sc = np.where(vis, sc, -np.inf)
        m = sc.max(axis=1, keepdims=True)
        m = np.where(np.isfinite(m), m, 0.0)
        p = np.exp(sc - m)
        den = p.sum(axis=norm_axis, keepdims=True)
        out[:, h, :] = (p @ V[:, g, :]) / den
    return out


MUTANTS = {
    "gqa_modulo": dict(gqa="mod"),
    "causal_strict": dict(causal="lt"),
    "no_scale": dict(use_scale=False),
    "k_v_swapped": dict(swap_kv=True),
    "normalised_over_queries": dict(norm_axis=0),
    "offset_off_by_one": dict(offset=-1),
}

PIN_CHECKS = [
    pins.test_textbook_single_request_no_cache,
    pins.test_chunk_with_prefix_equals_rows_of_full_causal,
    pins.test_packed_step_against_sdpa_per_request,
    pins.test_single_visible_key_returns_its_value,
    pins.test_zero_query_gives_mean_of_visible_values,
]


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_pins_catch_planted_mistake(name, monkeypatch):
    kw = MUTANTS[name]

    def mutant(q, K, V, cached, scale):
        return _attn(q, K, V, cached, scale, **kw)

    monkeypatch.setattr(pa, "attention_one_request", mutant)
    monkeypatch.setattr(oracle, "attention_one_request", mutant)
    caught = []
    for check in PIN_CHECKS:
        try:
            with np.errstate(all="ignore"):
                check()
        except (AssertionError, ValueError, IndexError):
            caught.append(check.__name__)
    assert caught, f"no pin caught mutant {name}"


def test_unmutated_reference_passes_every_check(monkeypatch):
    def same(q, K, V, cached, scale):
        return _attn(q, K, V, cached, scale)

    monkeypatch.setattr(pa, "attention_one_request", same)
    monkeypatch.setattr(oracle, "attention_one_request", same)
    for check in PIN_CHECKS:
        check()


def test_pins_catch_wrong_v_tile_reading(monkeypatch):
    def token_major_v(v_pool, slot, head, D):
        b, o = divmod(int(slot), 16)
        return v_pool[b, head][o * D:(o + 1) * D]

    monkeypatch.setattr(pa, "read_v_token", token_major_v)
    with pytest.raises(AssertionError):
        pins.test_gather_blockwise_equals_token_by_token()


def test_pins_catch_whole_tile_dimension_major_v_reading(monkeypatch):
    # the V tile as one [D][16] dimension-major block instead of two halves
    def whole_tile_v(v_pool, slot, head, D):
        b, o = divmod(int(slot), 16)
        return np.asarray(v_pool[b, head])[o::16][:D]

    monkeypatch.setattr(pa, "read_v_token", whole_tile_v)
    with pytest.raises(AssertionError):
        pins.test_gather_blockwise_equals_token_by_token()


def test_pins_catch_token_major_k_reading(monkeypatch):
    def token_major_k(k_pool, slot, head, D):
        b, o = divmod(int(slot), 16)
        return k_pool[b, head][o * D:(o + 1) * D]

    monkeypatch.setattr(pa, "read_k_token", token_major_k)
    with pytest.raises(AssertionError):
        pins.test_gather_grouped_k_tiles()


def test_pins_catch_wrong_slot_offset(monkeypatch):
    def bad_slot(row, pos):
        return int(row[pos // 16]) * 16 + (pos % 16 + 1) % 16

    monkeypatch.setattr(pa, "slot_of", bad_slot)
    monkeypatch.setattr(oracle, "slot_of", bad_slot)
    with pytest.raises(AssertionError):
        pins.test_slot_formula_matches_paging_simulation()
    with pytest.raises(AssertionError):
        pins.test_figure_11_4_shared_blocks()
