"""The weight layers around the step on the GPU, through the C ABI, against
the fp64 oracle: the linear layer (ragged row counts, several tiles, the
full inner dimension), the fused QKV projection with RoPE (positions from
0 to past 30,000), and one whole packed layer (projection, paged step,
output projection) on the worked step and on a mixed chunk + decode step.

Tolerances.  A projection output is rounded once to bf16 (relative error at
most 2^-9) after an fp32 sum of K products (error far below that for
K <= 4096); RoPE's angle is formed in double and reduced to one turn before
the float sine and cosine (error ~1e-7 each).  Hence
|gpu - ref| <= 2^-8 |ref| + 2e-3 per element.  Row counts up to 64 take
the weight-streaming kernel (K a multiple of 128), larger ones the tiled
one; both are covered.  The layer's attention output
and final projection are held to the step's bar: max-abs 2e-2, mean-abs
2e-3, with inputs scaled so that q, k, v have unit variance.
"""

import sys

import numpy as np
import pytest
import torch

import oracle
import paged_kv_cache_149_amd as pkv
from oracle import layer as L
from synth import workloads as wl
from synth.device import to_device

pytestmark = pytest.mark.gpu

D = 128


@pytest.fixture(scope="module")
def dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    pkv.load_library()
    return torch.device("cuda", 0)


def note(msg):
    print(f"[gpu-layer] {msg}", flush=True)
    sys.stdout.flush()


def _bf16(rng, shape, scale=1.0):
    return wl.f32_to_bf16_bits((rng.standard_normal(shape) * scale).astype(np.float32))


def _close(got_bits, ref, label):
    got = oracle.bf16_bits_to_f64(got_bits)
    assert np.isfinite(got).all(), label
    err = np.abs(got - ref)
    bound = 2.0 ** -8 * np.abs(ref) + 2e-3
    note(f"{label}: max-abs {err.max():.3e}, worst err/bound {(err / bound).max():.3f}")
    assert (err <= bound).all(), (label, float(err.max()))


@pytest.mark.parametrize("M,N,K", [(1, 128, 64), (37, 256, 128), (64, 384, 4096), (5, 4096, 4096), (65, 256, 256), (300, 384, 512),
                                   (513, 128, 4096), (4096, 4096, 64), (4000, 4224, 128),
                                   # few rows, inner dimension a multiple of 256: rows and weights staged
                                   # through LDS (one chunk, two chunks, an odd count, rows not a
                                   # multiple of 16)
                                   (1, 128, 256), (33, 256, 512), (17, 128, 768), (63, 512, 1280)])
def test_linear_matches_oracle(dev, M, N, K):
    rng = np.random.default_rng(M * 7 + N + K)
    x, w = _bf16(rng, (M, K)), _bf16(rng, (N, K), 1.0 / np.sqrt(K))
    note(f"linear M={M} N={N} K={K}")
    y = pkv.pkv_linear(pkv.bf16_tensor(x, dev).view(M, K), pkv.bf16_tensor(w, dev).view(N, K))
    torch.cuda.synchronize()
    ref = L.linear(oracle.bf16_bits_to_f64(x), oracle.bf16_bits_to_f64(w))
    _close(pkv.bf16_bits(y), ref, f"linear {M}x{N}x{K}")


def test_linear_rejects_unsupported_shapes(dev):
    x = torch.zeros(4, 64, dtype=torch.bfloat16, device=dev)
    with pytest.raises(pkv.PKVError):
        pkv.pkv_linear(x, torch.zeros(100, 64, dtype=torch.bfloat16, device=dev))   # N % 128
    with pytest.raises(pkv.PKVError):
        pkv.pkv_linear(torch.zeros(4, 96, dtype=torch.bfloat16, device=dev),
                       torch.zeros(128, 96, dtype=torch.bfloat16, device=dev))      # K % 64


@pytest.mark.parametrize("name,seqs", [
    ("worked", [(0, 5), (7, 1), (3, 1)]),
    ("chunks-and-decode", [(30720, 70), (0, 33), (5000, 1), (4095, 1), (1, 2)]),
    ("long-prefill", [(0, 1500), (100, 547), (9000, 1)]),
    ("decode-h384", [(5000, 1), (10, 1), (0, 3), (77, 1)]),   # few rows, hidden 384: four-wavefront form
    ("decode-h1024", [(3000, 1), (5, 1), (0, 2), (31000, 1)]),  # few rows, hidden 1024: LDS-staged form
])
def test_qkv_rope_matches_oracle(dev, name, seqs):
    hidden, Hq, Hkv = {"long-prefill": 64, "decode-h384": 384, "decode-h1024": 1024}.get(name, 512), 32, 8
    cu = np.concatenate([[0], np.cumsum([n for _, n in seqs])]).astype(np.int32)
    sl = np.array([c + n for c, n in seqs], dtype=np.int32)
    T = int(cu[-1])
    rng = np.random.default_rng(5)
    x = _bf16(rng, (T, hidden))
    w = _bf16(rng, ((Hq + 2 * Hkv) * D, hidden), 1.0 / np.sqrt(hidden))
    note(f"qkv+rope {name}: {T} rows")
    q, k, v = pkv.pkv_qkv_rope(pkv.bf16_tensor(x, dev).view(T, hidden), pkv.bf16_tensor(w, dev).view(-1, hidden),
                               torch.from_numpy(cu).to(dev), torch.from_numpy(sl).to(dev), Hq, Hkv)
    torch.cuda.synchronize()
    pos = L.row_positions(cu, sl)
    rq, rk, rv = L.qkv_rope(oracle.bf16_bits_to_f64(x), oracle.bf16_bits_to_f64(w), pos, Hq, Hkv, D)
    _close(pkv.bf16_bits(q), rq, f"{name} q")
    _close(pkv.bf16_bits(k), rk, f"{name} k")
    _close(pkv.bf16_bits(v), rv, f"{name} v")


@pytest.mark.parametrize("name", ["worked", "chunk-and-decode"])
def test_layer_forward_matches_oracle(dev, name):
    if name == "worked":
        b = wl.config_worked_step(pool="materialize")
    else:
        b = wl.make_batch("layer-mix", [(100, 40), (700, 1), (0, 9), (33, 1)], seed=41, pool="materialize")
    T, Hq, Hkv, hidden = b.num_rows, b.num_q_heads, b.num_kv_heads, 512
    rng = np.random.default_rng(6)
    x = _bf16(rng, (T, hidden))
    w_qkv = _bf16(rng, ((Hq + 2 * Hkv) * D, hidden), 1.0 / np.sqrt(hidden))
    w_o = _bf16(rng, (hidden, Hq * D), 1.0 / np.sqrt(Hq * D))
    t = to_device(b, dev)
    plan = pkv.pkv_plan(b.cu_seqlens_q, b.seq_lens, Hq, Hkv, D, block_tables=b.block_tables,
                        num_blocks=b.num_blocks, device=dev)
    note(f"layer {name}: {T} rows, hidden {hidden}")
    y, buf = pkv.pkv_layer_forward(pkv.bf16_tensor(x, dev).view(T, hidden),
                                   pkv.bf16_tensor(w_qkv, dev).view(-1, hidden),
                                   pkv.bf16_tensor(w_o, dev).view(hidden, -1), t["k_cache"], t["v_cache"],
                                   t["cu_seqlens_q"], t["seq_lens"], t["block_tables"], t["scale"], plan)
    torch.cuda.synchronize()
    f64 = oracle.bf16_bits_to_f64
    ry, rq, rk, rv, rattn = L.layer_forward(f64(x), f64(w_qkv), f64(w_o), b.cu_seqlens_q, b.seq_lens,
                                            b.block_tables, b.k_pool, b.v_pool, Hq, Hkv, D, float(b.scale))
    _close(pkv.bf16_bits(buf["k_new"]), rk, f"{name} k_new")
    for got, ref, label in ((buf["attn"], rattn, "attn"), (y, ry, "y")):
        err = np.abs(f64(pkv.bf16_bits(got)).reshape(ref.shape) - ref)
        note(f"layer {name} {label}: max-abs {err.max():.3e} mean-abs {err.mean():.3e}")
        assert err.max() <= 2e-2 and err.mean() <= 2e-3, (label, err.max(), err.mean())
    # the new rows went into the pool at their slots, bit for bit as the step writes them
    slots = buf["slot_mapping"].cpu().numpy()
    assert np.array_equal(slots, oracle.slot_mapping(b.cu_seqlens_q, b.seq_lens, b.block_tables))
    k_pool = pkv.bf16_bits(t["k_cache"]).reshape(b.num_blocks, Hkv, -1)
    kexp, _ = oracle.pools_after_append(b.k_pool, b.v_pool, slots, pkv.bf16_bits(buf["k_new"]),
                                        pkv.bf16_bits(buf["v_new"]))
    assert np.array_equal(k_pool, kexp)
