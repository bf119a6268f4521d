"""Parity of the HIP path with the fp64 oracle, through the C ABI.

Slot translation and append: bit-exact.  Attention: max-abs <= 2e-2 and
mean-abs <= 2e-3 against the fp64 oracle over every compared element.
Every config is compared whole (every element); only the 32K-prefix chunk,
a diagnostic workload, is sampled.  Default plan options, as the bench runs.
"""

import dataclasses
import math
import sys

import numpy as np
import pytest
import torch

import oracle
import paged_kv_cache_149_amd as pkv
from synth import workloads as wl
from synth.device import to_device

pytestmark = pytest.mark.gpu

MAX_ABS = 2e-2
MEAN_ABS = 2e-3


@pytest.fixture(scope="module")
def dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    pkv.load_library()
    return torch.device("cuda", 0)


def note(msg):
    print(f"[gpu-parity] {msg}", flush=True)
    sys.stdout.flush()


def run_step(batch, dev, options=None, tensors=None):
    """Plan + slot mapping + append + attention on the device; returns host
    copies of out (bf16 bits), slots and the device tensors."""
    t = tensors or to_device(batch, dev)
    plan = pkv.pkv_plan(batch.cu_seqlens_q, batch.seq_lens, batch.num_q_heads, batch.num_kv_heads,
                        batch.head_dim, block_tables=batch.block_tables, num_blocks=batch.num_blocks,
                        options=options, device=dev)
    out, slots = pkv.pkv_paged_step(t["q"], t["k_new"], t["v_new"], t["k_cache"], t["v_cache"],
                                    t["cu_seqlens_q"], t["seq_lens"], t["block_tables"], t["scale"], plan)
    torch.cuda.synchronize()
    return pkv.bf16_bits(out), slots.cpu().numpy(), t, plan


def attn_error(gpu_bits, ref):
    g = oracle.bf16_bits_to_f64(gpu_bits)
    err = np.abs(g - ref)
    assert np.isfinite(g).all(), "non-finite output"
    return float(err.max()), float(err.mean())


def check_attention(gpu_bits, ref, label):
    mx, mean = attn_error(gpu_bits, ref)
    note(f"{label}: max-abs {mx:.3e} mean-abs {mean:.3e}")
    assert mx <= MAX_ABS and mean <= MEAN_ABS, (label, mx, mean)


def check_append(batch, slots, t, blocks=None):
    """Every appended row's K/V bits sit in its slot; other slots of the
    touched blocks keep the pool's original bits."""
    ref_slots = oracle.slot_mapping(batch.cu_seqlens_q, batch.seq_lens, batch.block_tables)
    assert np.array_equal(slots, ref_slots)
    touched = np.unique(ref_slots // 16)
    if blocks is not None:
        touched = np.unique(np.concatenate([touched, blocks]))
    tb = torch.from_numpy(touched).to(t["k_cache"].device)
    k_dev = t["k_cache"][tb].contiguous().view(torch.int16).cpu().numpy().view(np.uint16)
    v_dev = t["v_cache"][tb].contiguous().view(torch.int16).cpu().numpy().view(np.uint16)
    k_exp = np.asarray(batch.k_pool[touched]).copy()
    v_exp = np.asarray(batch.v_pool[touched]).copy()
    pos = {int(b): i for i, b in enumerate(touched)}
    D = batch.head_dim
    W = oracle.k_group(D)
    for row, x in enumerate(ref_slots):
        b, o = divmod(int(x), 16)
        for h in range(batch.num_kv_heads):
            k_exp[pos[b], h].reshape(D // W, 16, W)[:, o, :] = batch.k_new[row, h].reshape(D // W, W)
            start = (o // 8) * 8 * D + o % 8  # V tile: halves of 8 tokens, each [D][8]
            v_exp[pos[b], h, start:start + 8 * D:8] = batch.v_new[row, h]
    assert np.array_equal(k_dev.reshape(k_exp.shape), k_exp)
    assert np.array_equal(v_dev.reshape(v_exp.shape), v_exp)


# ------------------------------------------------------------------ configs

def test_worked_step_full(dev):
    b = wl.config_worked_step()
    note("worked step: 3 requests, 7 rows")
    out, slots, t, plan = run_step(b, dev)
    check_append(b, slots, t)
    ref = oracle.packed_attention(b)
    check_attention(out, ref, "worked step")
    # R1 row 0 sees only its own key: the output is that value exactly
    for h in range(32):
        assert np.array_equal(out[0, h], b.v_new[0, h // 4])


def test_decode64_full(dev):
    b = wl.config_decode64()
    note("decode step: 64 sequences, contexts 128..4096")
    out, slots, t, plan = run_step(b, dev)
    check_append(b, slots, t)
    check_attention(out, oracle.packed_attention(b), "decode64")


def host_pools(batch, t):
    """The batch with its pools replaced by host copies of what the seeded
    generator wrote on the device (synth's torch form of the counter
    generator, before any library call touched the pools), so the oracle
    reads a whole multi-GB pool without generating it again on the CPU.
    A sample of referenced tiles is checked against the numpy form of the
    same generator first."""
    nb, hkv = batch.num_blocks, batch.num_kv_heads
    k = t["k_cache"].view(torch.int16).cpu().numpy().view(np.uint16).reshape(nb, hkv, -1)
    v = t["v_cache"].view(torch.int16).cpu().numpy().view(np.uint16).reshape(nb, hkv, -1)
    used = np.unique(batch.block_tables[batch.block_tables >= 0])
    probe = np.random.default_rng(7).choice(used, size=min(16, used.size), replace=False)
    assert np.array_equal(k[probe], batch.k_pool[probe]) and np.array_equal(v[probe], batch.v_pool[probe])
    return dataclasses.replace(batch, k_pool=k, v_pool=v)


def run_whole(batch, dev, label, plan_check=None):
    """The step on the device, then the append and every output element
    against the oracle."""
    t = to_device(batch, dev)
    b = host_pools(batch, t)
    out, slots, t, plan = run_step(b, dev, tensors=t)
    if plan_check is not None:
        plan_check(plan)
    check_append(b, slots, t)
    del t
    torch.cuda.empty_cache()
    check_attention(out, oracle.packed_attention(b), label)


def test_mixed_chunked_full(dev):
    """Mixed chunked-prefill step, whole: 4 x 256 prefill rows after
    prefixes 0/1024/2048/3072 and 1024 decode rows (2048 rows, every
    element against the oracle)."""
    note("mixed chunked-prefill step: 2048 rows (whole)")

    def wide_and_narrow(plan):
        assert plan.num_wide_items > 0 and plan.num_waves > 0

    run_whole(wl.config_mixed_chunked(), dev, "mixed chunked (whole)", wide_and_narrow)


def test_long_shared_full(dev):
    """Long-context decode with shared prefixes, whole: 16 x 32769 keys,
    two groups of 8 aliasing their first 128 blocks; contexts are split
    over wavefronts and merged."""
    note("long-context decode with shared prefixes: 16 x 32769 keys (whole)")

    def merged(plan):
        assert plan.num_merge > 0

    run_whole(wl.config_long_shared(), dev, "long shared (whole)", merged)


def test_prefill_chunk_sampled_rows(dev):
    """The 2048-row chunk after 30,720 cached tokens (wide workgroup tiles)."""
    b = wl.config_prefill_chunk()
    note("prefill chunk: 2048 rows after 30720 cached (sampled)")
    out, slots, t, plan = run_step(b, dev)
    assert plan.num_wide_items > 0
    check_append(b, slots, t)
    rows = [0, 1, 15, 16, 63, 64, 100, 511, 1000, 1024, 1535, 2000, 2046, 2047]
    ref = oracle.packed_attention_rows(b, rows)
    check_attention(out[rows], np.stack([ref[r] for r in rows]), "prefill chunk (sampled)")


def test_prefill_fresh_full(dev):
    b = wl.make_batch("prefill-3x300", [(0, 300), (0, 257), (0, 64)], seed=35)
    note("fresh prefills 300/257/64 (whole)")
    out, slots, t, plan = run_step(b, dev)
    assert plan.num_wide_items > 0
    check_append(b, slots, t)
    check_attention(out, oracle.packed_attention(b), "fresh prefills")


# ------------------------------------------------------------------ invariants

def test_placement_invariance_bitwise(dev):
    b = wl.make_batch("perm", [(300, 1), (0, 37), (129, 5), (31, 1), (1000, 3)], seed=21,
                      unused_fill="normal")
    note("placement invariance: 3 permutations")
    base, _, _, _ = run_step(b, dev)
    for seed in (1, 2, 3):
        p = wl.permute_placement(b, seed)
        o, _, _, _ = run_step(p, dev)
        assert np.array_equal(o, base), seed
    check_attention(base, oracle.packed_attention(b), "permutation base")


def test_constant_values(dev):
    b = wl.make_batch("const", [(77, 1), (0, 20), (33, 4)], seed=22, num_blocks=40, pool="materialize")
    c = wl.f32_to_bf16_bits(np.linspace(-2, 2, 8).astype(np.float32))
    for h in range(8):
        b.v_pool[:, h, :] = c[h]
        b.v_new[:, h, :] = c[h]
    out, _, _, _ = run_step(b, dev)
    got = oracle.bf16_bits_to_f64(out)
    want = oracle.bf16_bits_to_f64(c)[np.arange(32) // 4]
    assert np.abs(got - want[None, :, None]).max() <= 2 ** -8 * 2


def test_zero_query_gives_mean(dev):
    b = wl.make_batch("zq", [(45, 2), (0, 9)], seed=23)
    b.q[:] = 0
    out, _, _, _ = run_step(b, dev)
    check_attention(out, oracle.packed_attention(b), "zero query")


# ------------------------------------------------------------------ edge cases

EDGE = {
    "single-key": [(0, 1)],
    "block-edges": [(15, 1), (16, 1), (31, 1), (32, 1), (33, 1), (47, 1), (0, 16), (0, 17), (0, 32), (0, 33)],
    "empty-seqs": [(10, 1), (20, 0), (0, 0), (5, 3), (64, 0), (7, 1)],
    "short-prefills": [(0, 2), (3, 3), (10, 4), (0, 5), (100, 7)],
    "long-prefill": [(50, 100), (0, 130)],
    "ragged-tail": [(1023, 1), (0, 65), (4000, 17), (3, 1)],
    # rows of one 16-row append group more than 63 sequence boundaries apart
    # (runs of empty sequences): the slot translation's fallback search
    "many-empty-seqs": [(3, 1)] + [(7, 0)] * 80 + [(30, 2)] + [(1, 0)] * 70 + [(0, 5), (40, 1)] + [(2, 0)] * 3000,
}


@pytest.mark.parametrize("name", sorted(EDGE))
def test_edge_batches(dev, name):
    b = wl.make_batch(name, EDGE[name], seed=31)
    note(f"edge batch {name}")
    out, slots, t, _ = run_step(b, dev)
    check_append(b, slots, t)
    check_attention(out, oracle.packed_attention(b), name)


@pytest.mark.parametrize("Hq,Hkv", [(8, 8), (16, 8), (64, 8), (32, 2), (16, 1)])
def test_gqa_ratios(dev, Hq, Hkv):
    b = wl.make_batch(f"gqa{Hq}x{Hkv}", [(40, 1), (0, 23), (70, 6), (200, 1)], seed=32,
                      num_q_heads=Hq, num_kv_heads=Hkv)
    note(f"GQA Hq={Hq} Hkv={Hkv}")
    out, slots, t, _ = run_step(b, dev)
    check_append(b, slots, t)
    check_attention(out, oracle.packed_attention(b), f"gqa {Hq}/{Hkv}")


@pytest.mark.parametrize("opts", [
    {"min_wave_keys": 32, "narrow_waves": 1 << 20},   # one 32-key chunk per wavefront
    {"min_wave_keys": 64, "narrow_waves": 3, "wide_tiles": 0},  # three wavefronts walk everything
    {"wide_tiles": 1},
    {"workgroups": 8},                                 # long wide lists: many tile boundaries
    {"workgroups": 16, "narrow_waves": 64, "wide_tiles": 1},
])
def test_plan_options_same_result(dev, opts):
    b = wl.make_batch("opts", [(700, 1), (0, 50), (90, 3), (2000, 1), (129, 20)], seed=33)
    note(f"plan options {opts}")
    out, _, _, plan = run_step(b, dev, options=opts)
    check_attention(out, oracle.packed_attention(b), f"options {opts}")


@pytest.mark.parametrize("narrow_waves", [8, 64, 1000])
def test_narrow_stream_many_items(dev, narrow_waves):
    """Decode rows and short prefill tails dealt to few wavefronts, so each
    walks hundreds of items as one chunk stream: finished outputs (bf16 rows
    and fp32 partials) overflow the wavefront's 64 parked records many times
    and are written out mid-stream, and the items cut at share boundaries
    write partials."""
    rng = np.random.default_rng(71)
    seqs = [(int(c), 1) for c in rng.integers(1, 300, size=500)]
    seqs += [(int(c), int(n)) for c, n in zip(rng.integers(0, 200, size=12), rng.integers(2, 14, size=12))]
    b = wl.make_batch("narrow-stream", seqs, seed=72)
    note(f"narrow stream, {narrow_waves} wavefronts")
    out, _, _, plan = run_step(b, dev, options={"narrow_waves": narrow_waves, "min_wave_keys": 32, "wide_tiles": 0})
    assert plan.num_merge > 0
    check_attention(out, oracle.packed_attention(b), f"narrow stream {narrow_waves}")


@pytest.mark.parametrize("opts", [None, {"workgroups": 8}, {"workgroups": 16, "narrow_waves": 64}])
def test_wide_lists_with_interior_chunks(dev, opts):
    """Prefill tiles long enough to have interior (unmasked) chunks beside
    partial tiles and one-chunk tiles, dealt to few workgroups so one
    workgroup walks many tiles: every tile's Q operands are loaded while the
    previous tile finishes, and interior steps take the branch-free path."""
    seqs = [(300, 70), (0, 200), (1000, 64), (65, 1), (129, 33), (2000, 128), (0, 5), (96, 17)]
    b = wl.make_batch("wide-lists", seqs, seed=36)
    note(f"wide lists {opts}")
    out, _, _, _ = run_step(b, dev, options=opts)
    check_attention(out, oracle.packed_attention(b), f"wide lists {opts}")


@pytest.mark.parametrize("scale", [0.01, 0.0883883, 0.3, 1.0])
def test_softmax_scales(dev, scale):
    """Scales other than 1/sqrt(128), against the oracle at each scale:
    prefill tiles and decode items both apply the scale in fp32 inside each
    exponent's argument."""
    import dataclasses
    b = wl.make_batch("scales", [(300, 70), (0, 130), (900, 1), (64, 1)], seed=37)
    b = dataclasses.replace(b, scale=np.float32(scale))
    note(f"softmax scale {scale}")
    out, _, _, _ = run_step(b, dev)
    check_attention(out, oracle.packed_attention(b), f"scale {scale}")


def _scaled_bits(bits, factor):
    """bf16 bits of factor x value, rounded to nearest even (exact when the
    factor is a power of two); NaN and infinity patterns are kept."""
    x = np.asarray(bits, dtype=np.uint16)
    special = (x & 0x7F80) == 0x7F80
    y = wl.f32_to_bf16_bits((oracle.bf16_bits_to_f64(x) * factor).astype(np.float32))
    return np.where(special, x, y).astype(np.uint16)


@pytest.mark.parametrize("std", [2.0, 3.0])
def test_large_queries_and_keys_at_the_default_scale(dev, std):
    """Q and K drawn with standard deviation 2 and 3 instead of 1 (logits
    4 and 9 times larger) at the default scale 1/sqrt(128): prefill tiles
    and decode items both stay within the tolerance."""
    b = wl.make_batch("large-qk", [(300, 70), (0, 130), (900, 1), (64, 1), (0, 600), (40, 3)], seed=38,
                      pool="materialize")
    b.q[:] = _scaled_bits(b.q, std)
    b.k_new[:] = _scaled_bits(b.k_new, std)
    b.k_pool[:] = _scaled_bits(b.k_pool, std)
    note(f"Q/K std {std}")
    out, slots, t, plan = run_step(b, dev)
    assert plan.num_wide_items > 0
    check_append(b, slots, t)
    check_attention(out, oracle.packed_attention(b), f"Q/K std {std}")


def test_nan_in_unused_slots_does_not_leak(dev):
    """Slots past each sequence's end in its last block hold NaN bits."""
    b = wl.make_batch("nan-tail", [(20, 1), (0, 7), (37, 2)], seed=34, pool="materialize")
    D = b.head_dim
    for s in range(b.num_seqs):
        n = int(b.seq_lens[s])
        last = int(b.block_tables[s, (n - 1) // 16])
        W = oracle.k_group(D)
        for o in range(n % 16 or 16, 16):
            b.k_pool[last].reshape(b.num_kv_heads, D // W, 16, W)[:, :, o, :] = 0x7FC0
            b.v_pool[last, :, (o // 8) * 8 * D + o % 8::8][:, :D] = 0x7FC0
    out, _, _, _ = run_step(b, dev)
    check_attention(out, oracle.packed_attention(b), "nan tails")


def test_growing_scores_recompute(dev):
    """Scores that grow by ~2 (log2 units) every 32 keys: a prefill tile's
    first-chunk reference is exceeded by more than 2^100 after ~50 chunks,
    so the wavefronts of such tiles recompute their columns with the
    running-maximum softmax.  Every query is 1.0; key p is 0.125 * (p // 32)
    in every dimension."""
    seqs = [(0, 3000), (2900, 100), (3100, 1)]
    b = wl.make_batch("growing-scores", seqs, seed=35, pool="materialize")
    D = b.head_dim
    one = wl.f32_to_bf16_bits(np.float32(1.0))
    b.q[:] = one
    kval = lambda p: wl.f32_to_bf16_bits(np.float32(0.125 * (p // 32)))
    cu = b.cu_seqlens_q
    W = oracle.k_group(D)
    for s, (c, ql) in enumerate(seqs):
        for p in range(c):
            blk = int(b.block_tables[s, p // 16])
            b.k_pool[blk].reshape(b.num_kv_heads, D // W, 16, W)[:, :, p % 16, :] = kval(p)
        for j in range(ql):
            b.k_new[cu[s] + j] = kval(c + j)
    note("growing scores")
    out, slots, t, plan = run_step(b, dev)
    assert plan.num_wide_items > 0
    check_append(b, slots, t)
    check_attention(out, oracle.packed_attention(b), "growing scores")


def test_growing_scores_with_large_values(dev):
    """The growing-scores batch with every value multiplied by 2^30 (exact
    in bf16): a tile whose probabilities still sum below the recompute bound
    can then overflow its output accumulators (2^99 x 2^32 > 2^128), so the
    accumulators must be checked too.  Scaling values by a power of two
    scales the exact result by the same power, so the outputs divided by
    2^30 must meet the usual tolerance."""
    seqs = [(0, 3000), (2900, 100), (3100, 1)]
    b = wl.make_batch("growing-scores-big-v", seqs, seed=35, pool="materialize")
    D = b.head_dim
    one = wl.f32_to_bf16_bits(np.float32(1.0))
    b.q[:] = one
    kval = lambda p: wl.f32_to_bf16_bits(np.float32(0.125 * (p // 32)))
    cu = b.cu_seqlens_q
    W = oracle.k_group(D)
    for s, (c, ql) in enumerate(seqs):
        for p in range(c):
            blk = int(b.block_tables[s, p // 16])
            b.k_pool[blk].reshape(b.num_kv_heads, D // W, 16, W)[:, :, p % 16, :] = kval(p)
        for j in range(ql):
            b.k_new[cu[s] + j] = kval(c + j)
    big = 2.0 ** 30
    b.v_pool[:] = _scaled_bits(b.v_pool, big)
    b.v_new[:] = _scaled_bits(b.v_new, big)
    note("growing scores, values x 2^30")
    out, slots, t, plan = run_step(b, dev)
    assert plan.num_wide_items > 0
    check_append(b, slots, t)
    got = oracle.bf16_bits_to_f64(out) / big
    ref = oracle.packed_attention(b) / big
    assert np.isfinite(got).all(), "non-finite output"
    err = np.abs(got - ref)
    note(f"growing scores x 2^30: max-abs {err.max():.3e} mean-abs {err.mean():.3e} (after / 2^30)")
    assert err.max() <= MAX_ABS and err.mean() <= MEAN_ABS


def test_attention_entry_points_agree(dev):
    """main + reduce called separately == the combined call == the step."""
    b = wl.config_decode64()
    t = to_device(b, dev)
    plan = pkv.pkv_plan(b.cu_seqlens_q, b.seq_lens, 32, 8, 128, block_tables=b.block_tables,
                        num_blocks=b.num_blocks, options={"min_wave_keys": 64, "narrow_waves": 1 << 16},
                        device=dev)
    assert plan.num_merge > 0
    slots = pkv.pkv_slot_mapping(t["cu_seqlens_q"], t["seq_lens"], t["block_tables"], b.num_blocks)
    pkv.pkv_paged_kv_append(t["k_new"], t["v_new"], slots, t["k_cache"], t["v_cache"])
    o1 = pkv.pkv_varlen_attention_main(t["q"], t["k_cache"], t["v_cache"], t["block_tables"], t["scale"], plan)
    pkv.pkv_split_kv_reduce(plan, o1)
    o2 = pkv.pkv_paged_varlen_attention(t["q"], t["k_cache"], t["v_cache"], t["block_tables"], t["scale"], plan)
    torch.cuda.synchronize()
    assert torch.equal(o1.view(torch.int16), o2.view(torch.int16))
    check_attention(pkv.bf16_bits(o2), oracle.packed_attention(b), "split entry points")


@pytest.fixture(scope="module")
def trace_steps():
    from synth import scheduler as sc
    steps, _ = sc.continuous_batching_trace(sc.TraceConfig(steps=200))
    return steps


@pytest.mark.parametrize("index", [0, 5, 60, 150, 199])
def test_trace_step_full(dev, trace_steps, index):
    """Steps of the continuous-batching trace (65,536-block pool, 8192-token
    budget), whole: each step's metadata with freshly drawn values, every
    row of every kind against the oracle.  Step 0 is prefill only; steps
    150 and 199 carry 700+ decode rows beside prefill chunks in a nearly
    full pool."""
    st = trace_steps[index]
    b = wl.batch_from_metadata(f"trace-step{index}", st.cu_seqlens_q, st.seq_lens, st.block_tables,
                               65536, seed=149005 + 1000 * index)
    note(f"trace step {index}: {b.num_rows} rows, {b.num_seqs} sequences, {st.n_decode} decode (whole)")
    run_whole(b, dev, f"trace step {index} (whole)")


def test_trace_steps_around_a_preemption(dev):
    """The trace with a 16,384-block pool, where recompute preemption fires:
    the step that evicts a request and the next one, in which the evicted
    request is admitted again and prefills its prompt and generated tokens
    from scratch, both compared whole."""
    from synth import scheduler as sc
    steps, sch = sc.continuous_batching_trace(sc.TraceConfig(steps=120, num_blocks=16384))
    assert sch.preemptions > 0
    first = next(st for st in steps if st.preempted)
    victims = set(first.preempted)
    again = next(st for st in steps[first.index + 1:]
                 if any(rid in victims and cached == 0 for rid, cached, _ in st.rows))
    for st in (first, again):
        readmitted = [(rid, q) for rid, cached, q in st.rows if rid in victims and cached == 0]
        note(f"preemption trace step {st.index}: {st.num_rows} rows, preempted {st.preempted}, "
             f"re-admitted {readmitted}")
        b = wl.batch_from_metadata(f"preempt-step{st.index}", st.cu_seqlens_q, st.seq_lens, st.block_tables,
                                   16384, seed=149500 + st.index)
        run_whole(b, dev, f"preemption trace step {st.index} (whole)")


@pytest.mark.parametrize("name", ["trace-step150", "edge-runs"])
def test_planned_append_equals_plain_append(dev, trace_steps, name):
    """pkv_slot_append_planned (the step's append, on the planner's row
    groups) writes the same slots and leaves both pools bit-identical to
    pkv_slot_append (16-row groups); both checked against the oracle."""
    if name == "trace-step150":
        st = trace_steps[150]
        b = wl.batch_from_metadata("trace-step150-append", st.cu_seqlens_q, st.seq_lens, st.block_tables,
                                   65536, seed=149777)
    else:
        # (cached, new rows): runs that start and end inside blocks, a
        # block-aligned run, empty sequences and lone decode rows between them
        b = wl.make_batch("edge-runs-append", [(0, 16), (3, 0), (8, 1), (15, 33), (16, 1), (16, 16), (967, 33),
                                               (6, 1), (0, 0), (5, 39), (1, 1)], seed=149778)
    note(f"planned append {name}: {b.num_rows} rows, {b.num_seqs} sequences")
    plan = pkv.pkv_plan(b.cu_seqlens_q, b.seq_lens, b.num_q_heads, b.num_kv_heads, b.head_dim,
                        block_tables=b.block_tables, num_blocks=b.num_blocks, device=dev)
    assert plan.num_append_groups > 0
    results = []
    for planned in (False, True):
        t = to_device(b, dev)
        if planned:
            slots = pkv.pkv_slot_append_planned(t["k_new"], t["v_new"], t["cu_seqlens_q"], t["seq_lens"],
                                                t["block_tables"], t["k_cache"], t["v_cache"], plan)
        else:
            slots = pkv.pkv_slot_append(t["k_new"], t["v_new"], t["cu_seqlens_q"], t["seq_lens"],
                                        t["block_tables"], t["k_cache"], t["v_cache"])
        torch.cuda.synchronize()
        s = slots.cpu().numpy()
        check_append(b, s, t)
        results.append((s, t["k_cache"].view(torch.int16).clone(), t["v_cache"].view(torch.int16).clone()))
        del t
    assert np.array_equal(results[0][0], results[1][0])
    assert torch.equal(results[0][1], results[1][1]) and torch.equal(results[0][2], results[1][2])
