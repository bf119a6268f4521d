"""pkv_paged_step_static (the library's fixed device workspace) against
pkv_paged_step (a caller-owned workspace), through the C ABI: two calls in a
row on one stream, the second with a smaller batch, each compared bit for
bit with the existing entry point on its own copy of the pools (slots,
appended caches and attention output), and with the fp64 oracle."""

import sys

import numpy as np
import pytest
import torch

import oracle
import paged_kv_cache_149_amd as pkv
from synth import workloads as wl
from synth.device import to_device

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    pkv.load_library()
    return torch.device("cuda", 0)


def note(msg):
    print(f"[no-alloc] {msg}", flush=True)
    sys.stdout.flush()


def _both(b, dev, options):
    """Plan once (host staging only), then the step through both entry
    points, each on its own device copy of the batch."""
    plan = pkv.pkv_plan(b.cu_seqlens_q, b.seq_lens, b.num_q_heads, b.num_kv_heads, b.head_dim,
                        block_tables=b.block_tables, num_blocks=b.num_blocks, options=options, host_only=True)
    assert 0 < plan.ws_bytes <= pkv.STATIC_WS_BYTES
    ref_plan = pkv.pkv_plan(b.cu_seqlens_q, b.seq_lens, b.num_q_heads, b.num_kv_heads, b.head_dim,
                            block_tables=b.block_tables, num_blocks=b.num_blocks, options=options, device=dev)
    ta, tb = to_device(b, dev), to_device(b, dev)
    out_a, slots_a = pkv.pkv_paged_step(ta["q"], ta["k_new"], ta["v_new"], ta["k_cache"], ta["v_cache"],
                                        ta["cu_seqlens_q"], ta["seq_lens"], ta["block_tables"], ta["scale"],
                                        ref_plan)
    out_b, slots_b = pkv.pkv_paged_step_static(tb["q"], tb["k_new"], tb["v_new"], tb["k_cache"], tb["v_cache"],
                                               tb["cu_seqlens_q"], tb["seq_lens"], tb["block_tables"],
                                               tb["scale"], plan)
    torch.cuda.synchronize()
    return plan, (out_a, slots_a, ta), (out_b, slots_b, tb)


@pytest.mark.parametrize("options", [None, {"min_wave_keys": 64, "narrow_waves": 1 << 16}])
def test_static_workspace_matches_the_caller_workspace(dev, options):
    big = wl.make_batch("static-big", [(300, 70), (0, 130), (900, 1), (2000, 1), (64, 1), (3000, 1)], seed=41)
    small = wl.make_batch("static-small", [(40, 1), (0, 23), (129, 1)], seed=42)
    for b in (big, small):
        note(f"{b.name}: {b.num_rows} rows, options {options}")
        plan, (oa, sa, ta), (ob, sb, tb) = _both(b, dev, options)
        if options is not None:
            assert plan.num_merge > 0
        assert torch.equal(sa, sb)
        assert torch.equal(ta["k_cache"].view(torch.int16), tb["k_cache"].view(torch.int16))
        assert torch.equal(ta["v_cache"].view(torch.int16), tb["v_cache"].view(torch.int16))
        assert torch.equal(oa.view(torch.int16), ob.view(torch.int16))
        got = oracle.bf16_bits_to_f64(pkv.bf16_bits(ob))
        err = np.abs(got - oracle.packed_attention(b))
        note(f"{b.name}: max-abs {err.max():.3e} mean-abs {err.mean():.3e}")
        assert np.isfinite(got).all() and err.max() <= 2e-2 and err.mean() <= 2e-3
