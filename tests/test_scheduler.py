"""The iteration-level scheduler that drives the continuous-batching trace,
pinned by the schedules the pages print."""

import numpy as np
import pytest

import oracle
from synth import scheduler as sc


def test_static_batching_worked_examples():
    # [YB] Figure 11-2: A2 B5 C3 D8 E4 F3 G5 H6 on 4 rows: 14 steps, 64% useful
    steps, frac = sc.static_batching([2, 5, 3, 8, 4, 3, 5, 6], 4)
    assert steps == 14 and round(frac, 2) == 0.64
    # [YB] 11.2.1: outputs 10, 50, 200, 2000 in one batch: 2260 / 8000 = 28.25%
    steps, frac = sc.static_batching([10, 50, 200, 2000], 4)
    assert steps == 2000 and frac == pytest.approx(0.2825)


def test_continuous_batching_figure_11_2():
    # [YB] Figure 11-2: continuous batching needs 12 steps (75% useful) and E
    # starts at step 3 instead of step 9
    steps, first, done = sc.slot_schedule([2, 5, 3, 8, 4, 3, 5, 6], 4)
    assert steps == 12
    assert first[4] == 3
    assert sum([2, 5, 3, 8, 4, 3, 5, 6]) / (4 * steps) == 0.75


def test_continuous_batching_run_log():
    # [MLM] run log: caps 6, 50, 300, 30, 180, 45 on 3 slots finish at steps
    # 6, 50, 300, 36, 216, 95; request 3 is admitted after step 6 and its
    # prefill runs in step 7 together with the others' decode rows
    steps, first, done = sc.slot_schedule([6, 50, 300, 30, 180, 45], 3)
    assert done == [6, 50, 300, 36, 216, 95]
    assert first[3] == 7 and first[4] == 37 and first[5] == 51
    assert steps == 300


def test_budget_and_chunked_prefill():
    sch = sc.Scheduler(num_blocks=1000, token_budget=100)
    sch.add(sc.Request(0, prompt_len=250, output_len=3))
    sch.add(sc.Request(1, prompt_len=30, output_len=2))
    s0 = sch.schedule()
    assert s0.rows == [(0, 0, 100)]                     # first chunk fills the budget
    s1 = sch.schedule()
    assert s1.rows == [(0, 100, 100)]
    s2 = sch.schedule()
    assert s2.rows == [(0, 200, 50), (1, 0, 30)]       # last chunk, then admission
    s3 = sch.schedule()
    # both prompts are done: decode rows of both
    assert s3.rows == [(0, 250, 1), (1, 30, 1)]
    for st in (s0, s1, s2, s3):
        assert st.num_rows <= 100
        assert list(st.seq_lens) == [c + q for _, c, q in st.rows]


def test_recompute_preemption_returns_blocks_and_requeues():
    # two requests fill a 6-block pool; when both need a fourth block the
    # least recently scheduled, most recently admitted one is evicted
    sch = sc.Scheduler(num_blocks=6, token_budget=1000)
    sch.add(sc.Request(0, prompt_len=32, output_len=40))
    sch.add(sc.Request(1, prompt_len=32, output_len=40))
    evicted_at = None
    for _ in range(30):
        st = sch.schedule()
        if st.preempted:
            evicted_at = st
            break
    assert evicted_at is not None and evicted_at.preempted == [1]
    victim = sch.waiting[0]
    assert victim.rid == 1 and victim.computed == 0 and victim.blocks == []
    assert victim.known == 32 + victim.generated and victim.generated > 0
    owned = [b for r in sch.running for b in r.blocks]
    assert len(owned) + len(sch.pool.free) == 6 and len(set(owned)) == len(owned)
    # it comes back later and is prefilled again from position 0 with every
    # token it holds (prompt + generated)
    known_at_eviction = victim.known
    for _ in range(200):
        st = sch.schedule()
        mine = [row for row in st.rows if row[0] == 1]
        if mine:
            assert mine[0][1] == 0 and mine[0][2] == known_at_eviction
            break
    else:
        raise AssertionError("victim never re-admitted")


def test_trace_invariants():
    steps, sch = sc.continuous_batching_trace(sc.TraceConfig(steps=120))
    assert len(steps) == 120
    total_rows = 0
    for st in steps:
        assert 0 < st.num_rows <= 8192
        total_rows += st.num_rows
        q = np.diff(st.cu_seqlens_q)
        # decode rows come first in the packed order
        dec = [i for i, (_, c, n) in enumerate(st.rows) if n == 1]
        assert dec == list(range(len(dec))) or st.n_decode == 0 or dec[:st.n_decode] == list(range(st.n_decode))
        slots = oracle.slot_mapping(st.cu_seqlens_q, st.seq_lens, st.block_tables)
        assert np.unique(slots).size == slots.size          # no two rows write one slot
        bt = st.block_tables
        used = np.concatenate([bt[i, :(int(n) + 15) // 16] for i, n in enumerate(st.seq_lens)])
        assert used.min() >= 0 and used.max() < 65536
        assert np.unique(used).size == used.size            # no block shared between sequences
        assert (q >= 1).all()
    # the budget is saturated once the queue has built up
    assert np.mean([st.num_rows for st in steps[20:]]) > 0.95 * 8192
