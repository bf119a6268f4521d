"""ctypes binding of libpkv (include/pkv.h).  Argument marshalling only:
every step of the path runs in the library's HIP kernels.

The library must be built (``python -m paged_kv_cache_149_amd._build`` or
``__graft_entry__.build()``); there is no fallback.  torch is imported before
the library is loaded so that both use the one HIP runtime already in the
process (libamdhip64.so.7), which makes torch's device pointers and stream
handles valid arguments.
"""

from __future__ import annotations

import ctypes
import os
import re
import time
from typing import Optional

import numpy as np
import torch

from ._build import LIB_PATH, INCLUDE

BLOCK_SIZE = 16
HEAD_DIM = 128
V_HALF = 8  # a V tile holds its block's tokens in two halves of 8, each [D][8]


def v_cache_shape(num_blocks: int, num_kv_heads: int, head_dim: int = HEAD_DIM) -> tuple:
    """Shape of the V pool tensor: [NB][Hkv][2][D][8] (see include/pkv.h)."""
    return (num_blocks, num_kv_heads, BLOCK_SIZE // V_HALF, head_dim, V_HALF)
ITEM_INTS = 8
MERGE_INTS = 4

PKV_OK = 0
_STATUS = {0: "PKV_OK", 1: "PKV_EINVAL", 2: "PKV_ERANGE", 3: "PKV_EUNSUPPORTED",
           4: "PKV_EWORKSPACE", 5: "PKV_EHIP"}


class PKVError(RuntimeError):
    def __init__(self, func: str, status: int):
        self.status = status
        super().__init__(f"{func} failed: {_STATUS.get(status, status)}")


class PlanOptions(ctypes.Structure):
    _fields_ = [("narrow_waves", ctypes.c_int32), ("min_wave_keys", ctypes.c_int32),
                ("wide_tiles", ctypes.c_int32), ("workgroups", ctypes.c_int32)]


class PlanStruct(ctypes.Structure):
    _fields_ = [("num_seqs", ctypes.c_int32), ("num_rows", ctypes.c_int32),
                ("num_q_heads", ctypes.c_int32), ("num_kv_heads", ctypes.c_int32),
                ("head_dim", ctypes.c_int32), ("num_items", ctypes.c_int32),
                ("num_wide_items", ctypes.c_int32), ("num_waves", ctypes.c_int32),
                ("num_merge", ctypes.c_int32), ("num_part_cols", ctypes.c_int32),
                ("wave_keys", ctypes.c_int32), ("narrow_rows", ctypes.c_int32),
                ("items_off", ctypes.c_int64), ("waves_off", ctypes.c_int64),
                ("merge_off", ctypes.c_int64), ("ml_off", ctypes.c_int64), ("o_off", ctypes.c_int64),
                ("zero_off", ctypes.c_int64),
                ("ws_bytes", ctypes.c_size_t), ("host_bytes", ctypes.c_size_t),
                ("kv_keys", ctypes.c_int64), ("visible_pairs", ctypes.c_int64),
                ("num_workgroups", ctypes.c_int32), ("num_append_groups", ctypes.c_int32),
                ("wg_off", ctypes.c_int64), ("append_off", ctypes.c_int64)]


_P = ctypes.c_void_p
_I32 = ctypes.c_int32
_I64 = ctypes.c_int64
_F = ctypes.c_float
_SZ = ctypes.c_size_t

_SIGNATURES = {
    "pkv_status_string": (ctypes.c_char_p, [ctypes.c_int]),
    "pkv_version": (ctypes.c_int, []),
    "pkv_slot_mapping": (ctypes.c_int, [_P, _P, _P, _I32, _I32, _I32, _I64, _P, _P]),
    "pkv_paged_kv_append": (ctypes.c_int, [_P, _P, _P, _I32, _P, _P, _I64, _I32, _I32, _P]),
    "pkv_slot_append": (ctypes.c_int, [_P, _P, _P, _P, _P, _I32, _I32, _I32, _I64, _P, _P, _P,
                                       _I32, _I32, _P]),
    "pkv_plan": (ctypes.c_int, [_P, _P, _I32, _I32, _I32, _I32, _I32, _P, _I32, _I64,
                                ctypes.POINTER(PlanOptions), _P, _SZ, _P, _SZ,
                                ctypes.POINTER(PlanStruct), _P]),
    "pkv_varlen_attention_main": (ctypes.c_int, [_P, _P, _P, _P, _I32, _I64, _F,
                                                 ctypes.POINTER(PlanStruct), _P, _SZ, _P, _P]),
    "pkv_split_kv_reduce": (ctypes.c_int, [ctypes.POINTER(PlanStruct), _P, _SZ, _P, _P]),
    "pkv_paged_varlen_attention": (ctypes.c_int, [_P, _P, _P, _P, _I32, _I64, _F,
                                                  ctypes.POINTER(PlanStruct), _P, _SZ, _P, _P]),
    "pkv_slot_append_planned": (ctypes.c_int, [_P, _P, _P, _P, _P, _I32, _I64, _P, _P, _P, _P, _P, _SZ, _P]),
    "pkv_paged_step": (ctypes.c_int, [_P, _P, _P, _P, _P, _P, _P, _P, _I32, _I64, _P, _F,
                                      ctypes.POINTER(PlanStruct), _P, _SZ, _P, _P]),
    "pkv_paged_step_static": (ctypes.c_int, [_P, _P, _P, _P, _P, _P, _P, _P, _I32, _I64, _P, _F,
                                             ctypes.POINTER(PlanStruct), _P, _P, _P]),
    "pkv_linear": (ctypes.c_int, [_P, _P, _I32, _I32, _I32, _P, _P]),
    "pkv_qkv_rope": (ctypes.c_int, [_P, _P, _I32, _I32, _P, _P, _I32, _I32, _I32, _F, _P, _P, _P, _P]),
    "pkv_layer_forward": (ctypes.c_int, [_P, _P, _P, _I32, _P, _P, _P, _P, _P, _I32, _I64, _P, _F, _F,
                                         ctypes.POINTER(PlanStruct), _P, _SZ, _P, _P, _P, _P, _P, _P]),
    "pkv_block_pool_create": (ctypes.c_int, [_I64, ctypes.POINTER(ctypes.c_void_p)]),
    "pkv_block_pool_destroy": (None, [_P]),
    "pkv_block_pool_num_free": (_I64, [_P]),
    "pkv_block_pool_num_cached": (_I64, [_P]),
    "pkv_block_hash": (ctypes.c_uint64, [ctypes.c_uint64, _P, ctypes.c_uint64]),
    "pkv_block_pool_match_prefix": (ctypes.c_int, [_P, _P, _I32, ctypes.c_uint64, _P, _I32, ctypes.POINTER(_I32)]),
    "pkv_block_pool_register_prefix": (ctypes.c_int, [_P, _P, _I32, ctypes.c_uint64, _P]),
    "pkv_block_pool_refcount": (_I32, [_P, _I32]),
    "pkv_block_pool_allocate": (ctypes.c_int, [_P, _I32, _P]),
    "pkv_block_pool_share": (ctypes.c_int, [_P, _P, _I32]),
    "pkv_block_pool_release": (ctypes.c_int, [_P, _P, _I32]),
    "pkv_block_pool_append_slots": (ctypes.c_int, [_P, _P, _I32, _I32, _I32, _P, ctypes.POINTER(_I32)]),
    "pkv_copy_blocks": (ctypes.c_int, [_P, _P, _I64, _I32, _I32, _P, _I32, _P]),
    "pkv_swap_out": (ctypes.c_int, [_P, _P, _I64, _I32, _I32, _P, _I32, _P, _P]),
    "pkv_swap_in": (ctypes.c_int, [_P, _P, _I32, _P, _P, _I64, _I32, _I32, _P]),
}

_lib = None


def load_library(path: str = LIB_PATH) -> ctypes.CDLL:
    """Load libpkv once; raise if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(path):
            raise RuntimeError(f"{path} is missing: build it with __graft_entry__.build()")
        lib = ctypes.CDLL(path)
        for name, (res, args) in _SIGNATURES.items():
            fn = getattr(lib, name)
            fn.restype = res
            fn.argtypes = args
        _lib = lib
    return _lib


def header_functions() -> list:
    """Names of the functions include/pkv.h declares."""
    txt = open(os.path.join(INCLUDE, "pkv.h")).read()
    txt = re.sub(r"/\*.*?\*/", "", txt, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\s*\*?\s*(pkv_\w+)\s*\(", txt, flags=re.M)))


def _check(name: str, status: int):
    if status != PKV_OK:
        raise PKVError(name, status)


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream, device) -> ctypes.c_void_p:
    if stream is None:
        stream = torch.cuda.current_stream(device)
    return ctypes.c_void_p(stream.cuda_stream)


def _need(t: torch.Tensor, name: str, dtype, dev=None):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a tensor")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dev is not None and (t.device.type != "cuda" or (dev.index is not None and t.device != dev)):
        raise ValueError(f"{name} must live on {dev}")


# ---------------------------------------------------------------------------
# host <-> device helpers for bf16 bit patterns
# ---------------------------------------------------------------------------

def bf16_tensor(bits: np.ndarray, device) -> torch.Tensor:
    """bf16 tensor on ``device`` from uint16 bit patterns."""
    a = np.ascontiguousarray(bits, dtype=np.uint16)
    return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).to(device)


def bf16_bits(t: torch.Tensor) -> np.ndarray:
    """uint16 bit patterns of a bf16 tensor (copied to the host)."""
    return t.detach().contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


# ---------------------------------------------------------------------------
# entry points (same names as the C ABI)
# ---------------------------------------------------------------------------

def pkv_slot_mapping(cu_seqlens_q, seq_lens, block_tables, num_blocks, out=None, stream=None):
    lib = load_library()
    dev = cu_seqlens_q.device
    for n, t in (("cu_seqlens_q", cu_seqlens_q), ("seq_lens", seq_lens), ("block_tables", block_tables)):
        _need(t, n, torch.int32, dev)
    S = seq_lens.shape[0]
    T = int(cu_seqlens_q[-1].item()) if out is None else out.shape[0]
    if out is None:
        out = torch.empty(T, dtype=torch.int64, device=dev)
    _need(out, "slot_mapping", torch.int64, dev)
    _check("pkv_slot_mapping", lib.pkv_slot_mapping(
        _ptr(cu_seqlens_q), _ptr(seq_lens), _ptr(block_tables), block_tables.shape[1], S, T,
        int(num_blocks), _ptr(out), _stream(stream, dev)))
    return out


def pkv_paged_kv_append(k_new, v_new, slot_mapping, k_cache, v_cache, stream=None):
    lib = load_library()
    dev = k_cache.device
    for n, t in (("k_new", k_new), ("v_new", v_new), ("k_cache", k_cache), ("v_cache", v_cache)):
        _need(t, n, torch.bfloat16, dev)
    _need(slot_mapping, "slot_mapping", torch.int64, dev)
    T, Hkv, D = k_new.shape
    nb = k_cache.shape[0]
    if k_cache.shape != (nb, Hkv, BLOCK_SIZE, D) or v_cache.shape != v_cache_shape(nb, Hkv, D):
        raise ValueError("cache shapes must be [NB,Hkv,16,D] (K) and [NB,Hkv,2,D,8] (V)")
    if v_new.shape != k_new.shape or slot_mapping.shape[0] != T:
        raise ValueError("row counts differ")
    _check("pkv_paged_kv_append", lib.pkv_paged_kv_append(
        _ptr(k_new), _ptr(v_new), _ptr(slot_mapping), T, _ptr(k_cache), _ptr(v_cache), nb, Hkv, D,
        _stream(stream, dev)))


def pkv_slot_append(k_new, v_new, cu_seqlens_q, seq_lens, block_tables, k_cache, v_cache,
                    slot_mapping=None, stream=None):
    """Slot translation and append in one launch; returns slot_mapping."""
    lib = load_library()
    dev = k_cache.device
    for n, t in (("k_new", k_new), ("v_new", v_new), ("k_cache", k_cache), ("v_cache", v_cache)):
        _need(t, n, torch.bfloat16, dev)
    for n, t in (("cu_seqlens_q", cu_seqlens_q), ("seq_lens", seq_lens), ("block_tables", block_tables)):
        _need(t, n, torch.int32, dev)
    T, Hkv, D = k_new.shape
    nb = k_cache.shape[0]
    if k_cache.shape != (nb, Hkv, BLOCK_SIZE, D) or v_cache.shape != v_cache_shape(nb, Hkv, D):
        raise ValueError("cache shapes must be [NB,Hkv,16,D] (K) and [NB,Hkv,2,D,8] (V)")
    if slot_mapping is None:
        slot_mapping = torch.empty(T, dtype=torch.int64, device=dev)
    _need(slot_mapping, "slot_mapping", torch.int64, dev)
    _check("pkv_slot_append", lib.pkv_slot_append(
        _ptr(k_new), _ptr(v_new), _ptr(cu_seqlens_q), _ptr(seq_lens), _ptr(block_tables),
        block_tables.shape[1], seq_lens.shape[0], T, nb, _ptr(slot_mapping), _ptr(k_cache),
        _ptr(v_cache), Hkv, D, _stream(stream, dev)))
    return slot_mapping


class Plan:
    """A work plan in a device workspace.  Keeps its pinned host staging
    buffer alive (and its copy event) as long as the plan lives."""

    def __init__(self, st: PlanStruct, workspace: torch.Tensor, staging: torch.Tensor, event):
        self.st = st
        self.workspace = workspace
        self.staging = staging
        self.event = event
        self.host_us = 0.0

    def __getattr__(self, k):
        return getattr(self.st, k)

    def items(self) -> np.ndarray:
        n = self.st.num_items
        return self.staging[:n * ITEM_INTS * 4].numpy().view(np.int32).reshape(n, ITEM_INTS).copy()

    def waves(self) -> np.ndarray:
        """Item offsets of the narrow wavefronts (num_waves + 1 entries,
        relative to item num_wide_items)."""
        n = self.st.num_waves + 1
        off = self.st.waves_off
        return self.staging[off:off + n * 4].numpy().view(np.int32).copy()

    def wg_lists(self) -> np.ndarray:
        """Item offsets of the persistent workgroups' wide-tile lists
        (num_workgroups + 1 entries)."""
        n = self.st.num_workgroups + 1 if self.st.num_workgroups > 0 else 0
        off = self.st.wg_off
        return self.staging[off:off + n * 4].numpy().view(np.int32).copy()

    def append_groups(self) -> np.ndarray:
        """The append's row groups: [num_append_groups, 2] (first packed row,
        row count)."""
        n = self.st.num_append_groups
        off = self.st.append_off
        return self.staging[off:off + n * 8].numpy().view(np.int32).reshape(n, 2).copy()

    def merges(self) -> np.ndarray:
        n = self.st.num_merge
        off = self.st.merge_off
        return self.staging[off:off + n * MERGE_INTS * 4].numpy().view(np.int32).reshape(n, MERGE_INTS).copy()


def pkv_plan(cu_seqlens_q: np.ndarray, seq_lens: np.ndarray, num_q_heads: int, num_kv_heads: int,
             head_dim: int = HEAD_DIM, block_tables: Optional[np.ndarray] = None,
             num_blocks: int = 0, options: Optional[dict] = None, device=None,
             workspace: Optional[torch.Tensor] = None, stream=None, host_only: bool = False,
             staging: Optional[torch.Tensor] = None) -> Plan:
    """Build the work plan from HOST copies of the metadata.  With
    host_only=True nothing touches a GPU (the plan stays in host memory).
    ``staging`` (a pinned uint8 tensor) is used instead of a new pinned
    buffer when it is large enough; the caller must not reuse it until the
    plan's ``event`` has completed.  ``plan.host_us`` is the time the
    planning call itself took on the host."""
    lib = load_library()
    cu = np.ascontiguousarray(cu_seqlens_q, dtype=np.int32)
    sl = np.ascontiguousarray(seq_lens, dtype=np.int32)
    S = sl.shape[0]
    T = int(cu[-1]) if cu.size else 0
    bt = None if block_tables is None else np.ascontiguousarray(block_tables, dtype=np.int32)
    opts = PlanOptions(**(options or {"wide_tiles": -1}))
    if options is not None and "wide_tiles" not in options:
        opts.wide_tiles = -1
    st = PlanStruct()
    args = [cu.ctypes.data_as(_P), sl.ctypes.data_as(_P), S, T, num_q_heads, num_kv_heads, head_dim,
            None if bt is None else bt.ctypes.data_as(_P), 0 if bt is None else bt.shape[1],
            int(num_blocks), ctypes.byref(opts)]
    _check("pkv_plan", lib.pkv_plan(*args, None, 0, None, 0, ctypes.byref(st), None))
    host_bytes = max(int(st.host_bytes), 1)
    if host_only:
        staging = torch.empty(host_bytes, dtype=torch.uint8)
        _check("pkv_plan", lib.pkv_plan(*args, _P(staging.data_ptr()), host_bytes, None, 0,
                                         ctypes.byref(st), None))
        return Plan(st, None, staging, None)
    dev = torch.device(device if device is not None else "cuda")
    if dev.index is None:
        dev = torch.device("cuda", torch.cuda.current_device())
    if staging is None or staging.numel() < host_bytes or not staging.is_pinned():
        staging = torch.empty(host_bytes, dtype=torch.uint8, pin_memory=True)
    need = max(int(st.ws_bytes), 256)
    if workspace is None or workspace.numel() < need:
        workspace = torch.empty(need, dtype=torch.uint8, device=dev)
    s = stream if stream is not None else torch.cuda.current_stream(dev)
    t0 = time.perf_counter()
    rc = lib.pkv_plan(*args, _P(staging.data_ptr()), staging.numel(), _P(workspace.data_ptr()),
                      workspace.numel(), ctypes.byref(st), ctypes.c_void_p(s.cuda_stream))
    host_us = (time.perf_counter() - t0) * 1e6
    _check("pkv_plan", rc)
    ev = torch.cuda.Event()
    ev.record(s)
    plan = Plan(st, workspace, staging, ev)
    plan.host_us = host_us
    return plan


def _attn_args(q, k_cache, v_cache, block_tables, plan: Plan, out):
    dev = q.device
    _need(q, "q", torch.bfloat16, dev)
    _need(k_cache, "k_cache", torch.bfloat16, dev)
    _need(v_cache, "v_cache", torch.bfloat16, dev)
    _need(block_tables, "block_tables", torch.int32, dev)
    T, Hq, D = q.shape
    if T != plan.st.num_rows or Hq != plan.st.num_q_heads or D != plan.st.head_dim:
        raise ValueError("q does not match the plan")
    nb, Hkv = k_cache.shape[0], k_cache.shape[1]
    if Hkv != plan.st.num_kv_heads:
        raise ValueError("kv heads do not match the plan")
    if k_cache.shape != (nb, Hkv, BLOCK_SIZE, D) or v_cache.shape != v_cache_shape(nb, Hkv, D):
        raise ValueError("cache shapes must be [NB,Hkv,16,D] (K) and [NB,Hkv,2,D,8] (V)")
    if block_tables.shape[0] != plan.st.num_seqs:
        raise ValueError("block_tables rows do not match the plan")
    if out is None:
        out = torch.empty_like(q)
    _need(out, "out", torch.bfloat16, dev)
    if out.shape != q.shape:
        raise ValueError("out shape")
    return dev, nb, out


def pkv_varlen_attention_main(q, k_cache, v_cache, block_tables, scale, plan: Plan, out=None, stream=None):
    lib = load_library()
    dev, nb, out = _attn_args(q, k_cache, v_cache, block_tables, plan, out)
    ws = plan.workspace
    _check("pkv_varlen_attention_main", lib.pkv_varlen_attention_main(
        _ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(block_tables), block_tables.shape[1], nb,
        float(scale), ctypes.byref(plan.st), _ptr(ws), ws.numel(), _ptr(out), _stream(stream, dev)))
    return out


def pkv_split_kv_reduce(plan: Plan, out, stream=None):
    lib = load_library()
    _need(out, "out", torch.bfloat16, out.device)
    ws = plan.workspace
    _check("pkv_split_kv_reduce", lib.pkv_split_kv_reduce(
        ctypes.byref(plan.st), _ptr(ws), ws.numel(), _ptr(out), _stream(stream, out.device)))
    return out


def pkv_paged_varlen_attention(q, k_cache, v_cache, block_tables, scale, plan: Plan, out=None, stream=None):
    lib = load_library()
    dev, nb, out = _attn_args(q, k_cache, v_cache, block_tables, plan, out)
    ws = plan.workspace
    _check("pkv_paged_varlen_attention", lib.pkv_paged_varlen_attention(
        _ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(block_tables), block_tables.shape[1], nb,
        float(scale), ctypes.byref(plan.st), _ptr(ws), ws.numel(), _ptr(out), _stream(stream, dev)))
    return out


def pkv_slot_append_planned(k_new, v_new, cu_seqlens_q, seq_lens, block_tables, k_cache, v_cache, plan: Plan,
                            slot_mapping=None, stream=None):
    """pkv_slot_append on the plan's row groups (the step's first launch);
    returns slot_mapping."""
    lib = load_library()
    dev = k_cache.device
    for n, t in (("k_new", k_new), ("v_new", v_new), ("k_cache", k_cache), ("v_cache", v_cache)):
        _need(t, n, torch.bfloat16, dev)
    for n, t in (("cu_seqlens_q", cu_seqlens_q), ("seq_lens", seq_lens), ("block_tables", block_tables)):
        _need(t, n, torch.int32, dev)
    T, Hkv, D = k_new.shape
    nb = k_cache.shape[0]
    if k_cache.shape != (nb, Hkv, BLOCK_SIZE, D) or v_cache.shape != v_cache_shape(nb, Hkv, D):
        raise ValueError("cache shapes must be [NB,Hkv,16,D] (K) and [NB,Hkv,2,D,8] (V)")
    if T != plan.num_rows or Hkv != plan.num_kv_heads:
        raise ValueError("k_new does not match the plan")
    if slot_mapping is None:
        slot_mapping = torch.empty(T, dtype=torch.int64, device=dev)
    _need(slot_mapping, "slot_mapping", torch.int64, dev)
    ws = plan.workspace
    _check("pkv_slot_append_planned", lib.pkv_slot_append_planned(
        _ptr(k_new), _ptr(v_new), _ptr(cu_seqlens_q), _ptr(seq_lens), _ptr(block_tables), block_tables.shape[1],
        nb, _ptr(slot_mapping), _ptr(k_cache), _ptr(v_cache), ctypes.byref(plan.st), _ptr(ws), ws.numel(),
        _stream(stream, dev)))
    return slot_mapping


def pkv_paged_step(q, k_new, v_new, k_cache, v_cache, cu_seqlens_q, seq_lens, block_tables, scale,
                   plan: Plan, slot_mapping=None, out=None, stream=None):
    lib = load_library()
    dev, nb, out = _attn_args(q, k_cache, v_cache, block_tables, plan, out)
    _need(k_new, "k_new", torch.bfloat16, dev)
    _need(v_new, "v_new", torch.bfloat16, dev)
    _need(cu_seqlens_q, "cu_seqlens_q", torch.int32, dev)
    _need(seq_lens, "seq_lens", torch.int32, dev)
    if slot_mapping is None:
        slot_mapping = torch.empty(q.shape[0], dtype=torch.int64, device=dev)
    _need(slot_mapping, "slot_mapping", torch.int64, dev)
    ws = plan.workspace
    _check("pkv_paged_step", lib.pkv_paged_step(
        _ptr(q), _ptr(k_new), _ptr(v_new), _ptr(k_cache), _ptr(v_cache), _ptr(cu_seqlens_q),
        _ptr(seq_lens), _ptr(block_tables), block_tables.shape[1], nb, _ptr(slot_mapping),
        float(scale), ctypes.byref(plan.st), _ptr(ws), ws.numel(), _ptr(out), _stream(stream, dev)))
    return out, slot_mapping


STATIC_WS_BYTES = 32 << 20


def pkv_paged_step_static(q, k_new, v_new, k_cache, v_cache, cu_seqlens_q, seq_lens, block_tables, scale,
                          plan: Plan, slot_mapping=None, out=None, stream=None):
    """pkv_paged_step with the library's fixed device workspace: the plan's
    host staging buffer is copied there by the call, and nothing is
    allocated on the device by the library (plan.workspace is not used;
    build the plan with host_only=True).  Calls that overlap on one GPU
    share the array and race."""
    lib = load_library()
    dev, nb, out = _attn_args(q, k_cache, v_cache, block_tables, plan, out)
    _need(k_new, "k_new", torch.bfloat16, dev)
    _need(v_new, "v_new", torch.bfloat16, dev)
    _need(cu_seqlens_q, "cu_seqlens_q", torch.int32, dev)
    _need(seq_lens, "seq_lens", torch.int32, dev)
    if slot_mapping is None:
        slot_mapping = torch.empty(q.shape[0], dtype=torch.int64, device=dev)
    _need(slot_mapping, "slot_mapping", torch.int64, dev)
    if plan.staging is None or plan.staging.device.type != "cpu":
        raise ValueError("the plan needs its host staging buffer")
    _check("pkv_paged_step_static", lib.pkv_paged_step_static(
        _ptr(q), _ptr(k_new), _ptr(v_new), _ptr(k_cache), _ptr(v_cache), _ptr(cu_seqlens_q),
        _ptr(seq_lens), _ptr(block_tables), block_tables.shape[1], nb, _ptr(slot_mapping),
        float(scale), ctypes.byref(plan.st), _ptr(plan.staging), _ptr(out), _stream(stream, dev)))
    return out, slot_mapping


# ---------------------------------------------------------------------------
# the weight layers around the step
# ---------------------------------------------------------------------------

ROPE_THETA = 500000.0


def pkv_linear(x, w, out=None, stream=None):
    """y = x w^T over all rows: x bf16 [M, K], w bf16 [N, K] -> y bf16 [M, N]."""
    lib = load_library()
    dev = x.device
    _need(x, "x", torch.bfloat16, dev)
    _need(w, "w", torch.bfloat16, dev)
    M, K = x.shape
    N = w.shape[0]
    if w.shape[1] != K:
        raise ValueError("w must be [N, K] with x's K")
    if out is None:
        out = torch.empty(M, N, dtype=torch.bfloat16, device=dev)
    _need(out, "out", torch.bfloat16, dev)
    if tuple(out.shape) != (M, N):
        raise ValueError("out must be [M, N]")
    _check("pkv_linear", lib.pkv_linear(_ptr(x), _ptr(w), M, N, K, _ptr(out), _stream(stream, dev)))
    return out


def _qkv_out(T, Hq, Hkv, dev):
    return (torch.empty(T, Hq, HEAD_DIM, dtype=torch.bfloat16, device=dev),
            torch.empty(T, Hkv, HEAD_DIM, dtype=torch.bfloat16, device=dev),
            torch.empty(T, Hkv, HEAD_DIM, dtype=torch.bfloat16, device=dev))


def pkv_qkv_rope(x, w_qkv, cu_seqlens_q, seq_lens, num_q_heads: int, num_kv_heads: int,
                 rope_theta: float = ROPE_THETA, stream=None):
    """The fused QKV projection with RoPE by each row's position; returns
    (q [T, Hq, 128], k_new [T, Hkv, 128], v_new [T, Hkv, 128])."""
    lib = load_library()
    dev = x.device
    _need(x, "x", torch.bfloat16, dev)
    _need(w_qkv, "w_qkv", torch.bfloat16, dev)
    _need(cu_seqlens_q, "cu_seqlens_q", torch.int32, dev)
    _need(seq_lens, "seq_lens", torch.int32, dev)
    T, hidden = x.shape
    if tuple(w_qkv.shape) != ((num_q_heads + 2 * num_kv_heads) * HEAD_DIM, hidden):
        raise ValueError("w_qkv must be [(Hq + 2 Hkv) * 128, hidden]")
    q, k, v = _qkv_out(T, num_q_heads, num_kv_heads, dev)
    _check("pkv_qkv_rope", lib.pkv_qkv_rope(
        _ptr(x), _ptr(w_qkv), T, hidden, _ptr(cu_seqlens_q), _ptr(seq_lens), seq_lens.numel(), num_q_heads,
        num_kv_heads, float(rope_theta), _ptr(q), _ptr(k), _ptr(v), _stream(stream, dev)))
    return q, k, v


def pkv_layer_forward(x, w_qkv, w_o, k_cache, v_cache, cu_seqlens_q, seq_lens, block_tables, scale, plan: Plan,
                      rope_theta: float = ROPE_THETA, buffers=None, stream=None):
    """One packed layer: QKV projection with RoPE, the paged step, output
    projection.  Returns (y [T, hidden], buffers) where buffers holds the
    q, k_new, v_new, attn and slot_mapping tensors it wrote (pass them back
    in to reuse them)."""
    lib = load_library()
    dev = x.device
    T, hidden = x.shape
    Hq, Hkv = plan.st.num_q_heads, plan.st.num_kv_heads
    for t, name in ((x, "x"), (w_qkv, "w_qkv"), (w_o, "w_o"), (k_cache, "k_cache"), (v_cache, "v_cache")):
        _need(t, name, torch.bfloat16, dev)
    for t, name in ((cu_seqlens_q, "cu_seqlens_q"), (seq_lens, "seq_lens"), (block_tables, "block_tables")):
        _need(t, name, torch.int32, dev)
    if T != plan.st.num_rows:
        raise ValueError("x does not match the plan")
    if tuple(w_o.shape) != (hidden, Hq * HEAD_DIM):
        raise ValueError("w_o must be [hidden, Hq * 128]")
    if buffers is None:
        q, k, v = _qkv_out(T, Hq, Hkv, dev)
        buffers = {"q": q, "k_new": k, "v_new": v, "attn": torch.empty_like(q),
                   "slot_mapping": torch.empty(T, dtype=torch.int64, device=dev),
                   "y": torch.empty(T, hidden, dtype=torch.bfloat16, device=dev)}
    nb = k_cache.shape[0]
    ws = plan.workspace
    bf = buffers
    _check("pkv_layer_forward", lib.pkv_layer_forward(
        _ptr(x), _ptr(w_qkv), _ptr(w_o), hidden, _ptr(k_cache), _ptr(v_cache), _ptr(cu_seqlens_q), _ptr(seq_lens),
        _ptr(block_tables), block_tables.shape[1], nb, _ptr(bf["slot_mapping"]), float(scale), float(rope_theta),
        ctypes.byref(plan.st), _ptr(ws), ws.numel(), _ptr(bf["q"]), _ptr(bf["k_new"]), _ptr(bf["v_new"]),
        _ptr(bf["attn"]), _ptr(bf["y"]), _stream(stream, dev)))
    return bf["y"], bf


# ---------------------------------------------------------------------------
# block pool, copy-on-write and swap
# ---------------------------------------------------------------------------

def _i32(a) -> np.ndarray:
    return np.ascontiguousarray(a, dtype=np.int32)


class BlockPool:
    """The library's host block pool (reference counts, a stack of free
    blocks, copy-on-write of a shared partial block before an append, and a
    prefix cache of registered full blocks with an evictable queue)."""

    def __init__(self, num_blocks: int):
        self._lib = load_library()
        h = ctypes.c_void_p()
        _check("pkv_block_pool_create", self._lib.pkv_block_pool_create(int(num_blocks), ctypes.byref(h)))
        self._h = h
        self.num_blocks = int(num_blocks)

    def __del__(self):
        h = getattr(self, "_h", None)
        if h is not None and h.value:
            self._lib.pkv_block_pool_destroy(h)
            self._h = None

    @property
    def num_free(self) -> int:
        return int(self._lib.pkv_block_pool_num_free(self._h))

    @property
    def num_cached(self) -> int:
        return int(self._lib.pkv_block_pool_num_cached(self._h))

    def refcount(self, block: int) -> int:
        return int(self._lib.pkv_block_pool_refcount(self._h, int(block)))

    def match_prefix(self, tokens, row: np.ndarray, extra_key: int = 0) -> int:
        """Map the prompt's leading registered full blocks into ``row``
        (int32, modified in place); returns the number of cached tokens."""
        if row.dtype != np.int32 or not row.flags.c_contiguous:
            raise TypeError("row must be a contiguous int32 array")
        t = _i32(tokens)
        n = _I32()
        _check("pkv_block_pool_match_prefix", self._lib.pkv_block_pool_match_prefix(
            self._h, t.ctypes.data_as(_P), t.size, int(extra_key) & (2**64 - 1), row.ctypes.data_as(_P),
            row.size, ctypes.byref(n)))
        return int(n.value)

    def register_prefix(self, tokens, row, extra_key: int = 0) -> None:
        """Register the full blocks of a computed sequence for later hits."""
        t = _i32(tokens)
        r = _i32(row)
        if r.size < t.size // BLOCK_SIZE:
            raise ValueError("row shorter than the sequence's full blocks")
        _check("pkv_block_pool_register_prefix", self._lib.pkv_block_pool_register_prefix(
            self._h, t.ctypes.data_as(_P), t.size, int(extra_key) & (2**64 - 1), r.ctypes.data_as(_P)))

    def allocate(self, n: int) -> np.ndarray:
        out = np.empty(int(n), dtype=np.int32)
        _check("pkv_block_pool_allocate", self._lib.pkv_block_pool_allocate(
            self._h, int(n), out.ctypes.data_as(_P)))
        return out

    def share(self, blocks) -> None:
        b = _i32(blocks)
        _check("pkv_block_pool_share", self._lib.pkv_block_pool_share(self._h, b.ctypes.data_as(_P), b.size))

    def release(self, blocks) -> None:
        b = _i32(blocks)
        _check("pkv_block_pool_release", self._lib.pkv_block_pool_release(self._h, b.ctypes.data_as(_P), b.size))

    def append_slots(self, row: np.ndarray, num_tokens: int, num_new: int):
        """Prepare a block-table row (int32, modified in place) for num_new
        tokens after num_tokens; returns the (src, dst) copy to make first,
        or None."""
        if row.dtype != np.int32 or not row.flags.c_contiguous:
            raise TypeError("row must be a contiguous int32 array")
        copies = np.empty(2, dtype=np.int32)
        n = _I32()
        _check("pkv_block_pool_append_slots", self._lib.pkv_block_pool_append_slots(
            self._h, row.ctypes.data_as(_P), row.size, int(num_tokens), int(num_new),
            copies.ctypes.data_as(_P), ctypes.byref(n)))
        return (int(copies[0]), int(copies[1])) if n.value else None


def pkv_block_hash(parent: int, tokens16, extra_key: int = 0) -> int:
    """The library's hash of one full block (16 token ids)."""
    t = _i32(tokens16)
    if t.size != BLOCK_SIZE:
        raise ValueError("a block holds 16 tokens")
    return int(load_library().pkv_block_hash(int(parent) & (2**64 - 1), t.ctypes.data_as(_P),
                                              int(extra_key) & (2**64 - 1)))


def _pool_shapes(k_cache, v_cache):
    nb, Hkv, _, D = k_cache.shape
    if k_cache.shape != (nb, Hkv, BLOCK_SIZE, D) or v_cache.shape != v_cache_shape(nb, Hkv, D):
        raise ValueError("cache shapes must be [NB,Hkv,16,D] (K) and [NB,Hkv,2,D,8] (V)")
    return nb, Hkv, D


def pkv_copy_blocks(k_cache, v_cache, pairs, stream=None):
    """Copy block pairs[p, 0] onto pairs[p, 1] in both pools (device int32 [n, 2])."""
    lib = load_library()
    dev = k_cache.device
    _need(k_cache, "k_cache", torch.bfloat16, dev)
    _need(v_cache, "v_cache", torch.bfloat16, dev)
    _need(pairs, "pairs", torch.int32, dev)
    nb, Hkv, D = _pool_shapes(k_cache, v_cache)
    n = pairs.shape[0] if pairs.numel() else 0
    _check("pkv_copy_blocks", lib.pkv_copy_blocks(_ptr(k_cache), _ptr(v_cache), nb, Hkv, D, _ptr(pairs), n,
                                                  _stream(stream, dev)))


def swap_bytes(num_kv_heads: int, num: int, head_dim: int = HEAD_DIM) -> int:
    """Host bytes that num swapped blocks take (K and V)."""
    return int(num) * 2 * num_kv_heads * BLOCK_SIZE * head_dim * 2


def pkv_swap_out(k_cache, v_cache, blocks, host, stream=None):
    """Copy the listed blocks (device int32) into the pinned host tensor."""
    lib = load_library()
    dev = k_cache.device
    _need(k_cache, "k_cache", torch.bfloat16, dev)
    _need(v_cache, "v_cache", torch.bfloat16, dev)
    _need(blocks, "blocks", torch.int32, dev)
    nb, Hkv, D = _pool_shapes(k_cache, v_cache)
    if not host.is_pinned() or host.numel() * host.element_size() < swap_bytes(Hkv, blocks.numel(), D):
        raise ValueError("host must be a pinned tensor of at least swap_bytes() bytes")
    _check("pkv_swap_out", lib.pkv_swap_out(_ptr(k_cache), _ptr(v_cache), nb, Hkv, D, _ptr(blocks),
                                            blocks.numel(), _ptr(host), _stream(stream, dev)))


def pkv_swap_in(host, blocks, k_cache, v_cache, stream=None):
    """Copy the pinned host tensor's blocks back into the listed blocks."""
    lib = load_library()
    dev = k_cache.device
    _need(k_cache, "k_cache", torch.bfloat16, dev)
    _need(v_cache, "v_cache", torch.bfloat16, dev)
    _need(blocks, "blocks", torch.int32, dev)
    nb, Hkv, D = _pool_shapes(k_cache, v_cache)
    if not host.is_pinned() or host.numel() * host.element_size() < swap_bytes(Hkv, blocks.numel(), D):
        raise ValueError("host must be a pinned tensor of at least swap_bytes() bytes")
    _check("pkv_swap_in", lib.pkv_swap_in(_ptr(host), _ptr(blocks), blocks.numel(), _ptr(k_cache),
                                          _ptr(v_cache), nb, Hkv, D, _stream(stream, dev)))
