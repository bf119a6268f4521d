"""Counter-based N(0,1) bf16 values: value = f(seed, stream, element index).

Any element of any tensor (in particular any block of a huge paged pool) can
be computed on its own, so the CPU oracle computes only the blocks it reads
while the device fills a whole pool on the GPU from the same definition.

Definition.  For element index e (uint64) of stream ``stream`` under ``seed``:
  w  = e >> 1                          (one 32-bit hash serves two elements)
  s1 = H(seed * 0x9E3779B1 + stream * 0x85EBCA77 mod 2^32)
  s2 = H(s1 xor 0x27D4EB2F)
  h  = H(H((w mod 2^32) xor s1) xor (w >> 32) xor s2)
  u  = (h >> 16 * (e & 1)) & 0xFFFF     (uniform 16-bit integer)
  value = the bf16 pattern of the N(0,1) quantile at (u + 0.5) / 65536
with H the 32-bit integer hash
  x ^= x >> 16; x *= 0x7FEB352D; x ^= x >> 15; x *= 0x846CA68B; x ^= x >> 16
(all mod 2^32; multiplier constants of the "lowbias32" hash found by
C. Wellons' hash-prospector).  The numpy form uses native uint32
wraparound; the torch form computes the same products mod 2^32 in int64
in 16-bit halves so nothing overflows, and runs on CPU or GPU.
"""

from __future__ import annotations

import numpy as np

M32 = 0xFFFFFFFF
_C1, _C2 = 0x7FEB352D, 0x846CA68B

QNAN_BF16 = 0x7FC0


def _h32_int(x: int) -> int:
    x &= M32
    x ^= x >> 16
    x = (x * _C1) & M32
    x ^= x >> 15
    x = (x * _C2) & M32
    x ^= x >> 16
    return x


def stream_keys(seed: int, stream: int):
    s1 = _h32_int((seed * 0x9E3779B1 + stream * 0x85EBCA77) & M32)
    s2 = _h32_int(s1 ^ 0x27D4EB2F)
    return s1, s2


_TABLE = None


def normal_table() -> np.ndarray:
    """uint16[65536]: bf16 bits of the N(0,1) quantile at (u + 0.5) / 65536."""
    global _TABLE
    if _TABLE is None:
        from scipy.special import ndtri
        z = ndtri((np.arange(65536, dtype=np.float64) + 0.5) / 65536.0).astype(np.float32)
        u = z.view(np.uint32)
        r = (u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))) >> np.uint32(16)
        _TABLE = r.astype(np.uint16)
    return _TABLE


# ---------------------------------------------------------------- numpy

def _h32_np(x: np.ndarray) -> np.ndarray:
    x = x ^ (x >> np.uint32(16))
    x = x * np.uint32(_C1)
    x = x ^ (x >> np.uint32(15))
    x = x * np.uint32(_C2)
    x = x ^ (x >> np.uint32(16))
    return x


def uniform16_np(seed: int, stream: int, idx: np.ndarray) -> np.ndarray:
    s1, s2 = stream_keys(seed, stream)
    e = np.asarray(idx, dtype=np.uint64)
    w = e >> np.uint64(1)
    lo = (w & np.uint64(M32)).astype(np.uint32)
    hi = (w >> np.uint64(32)).astype(np.uint32)
    with np.errstate(over="ignore"):
        h = _h32_np(lo ^ np.uint32(s1))
        h = _h32_np(h ^ hi ^ np.uint32(s2))
    sh = ((e & np.uint64(1)) * np.uint64(16)).astype(np.uint32)
    return ((h >> sh) & np.uint32(0xFFFF)).astype(np.uint16)


def normal_bf16_np(seed: int, stream: int, idx: np.ndarray, chunk: int = 1 << 22) -> np.ndarray:
    """uint16 bf16 bits for the given element indices (any shape)."""
    idx = np.asarray(idx, dtype=np.uint64)
    flat = idx.reshape(-1)
    out = np.empty(flat.shape[0], dtype=np.uint16)
    tab = normal_table()
    for s in range(0, flat.shape[0], chunk):
        out[s:s + chunk] = tab[uniform16_np(seed, stream, flat[s:s + chunk])]
    return out.reshape(idx.shape)


def normal_bf16_range_np(seed: int, stream: int, start: int, count: int, chunk: int = 1 << 22) -> np.ndarray:
    out = np.empty(count, dtype=np.uint16)
    tab = normal_table()
    for s in range(0, count, chunk):
        n = min(chunk, count - s)
        idx = np.arange(start + s, start + s + n, dtype=np.uint64)
        out[s:s + n] = tab[uniform16_np(seed, stream, idx)]
    return out


# ---------------------------------------------------------------- torch

def _mulmod32_t(x, c: int):
    lo = (x & 0xFFFF) * c
    hi = ((x >> 16) * c) & 0xFFFF
    return (lo + (hi << 16)) & M32


def _h32_t(x):
    x = x ^ (x >> 16)
    x = _mulmod32_t(x, _C1)
    x = x ^ (x >> 15)
    x = _mulmod32_t(x, _C2)
    x = x ^ (x >> 16)
    return x


def uniform16_torch(seed: int, stream: int, idx):
    """Same function as uniform16_np on an int64 torch tensor of
    non-negative indices (CPU or GPU); returns int64 in [0, 65536)."""
    s1, s2 = stream_keys(seed, stream)
    w = idx >> 1
    h = _h32_t((w & M32) ^ s1)
    h = _h32_t(h ^ (w >> 32) ^ s2)
    return (h >> ((idx & 1) * 16)) & 0xFFFF


def normal_bf16_range_torch(seed: int, stream: int, start: int, count: int, device, chunk: int = 1 << 25):
    """int16 tensor (bf16 bits) of ``count`` values starting at element
    ``start``, generated on ``device``."""
    import torch
    tab = torch.from_numpy(normal_table().view(np.int16).astype(np.int64)).to(device)
    out = torch.empty(count, dtype=torch.int16, device=device)
    for s in range(0, count, chunk):
        n = min(chunk, count - s)
        idx = torch.arange(start + s, start + s + n, dtype=torch.int64, device=device)
        out[s:s + n] = tab[uniform16_torch(seed, stream, idx)].to(torch.int16)
    return out
