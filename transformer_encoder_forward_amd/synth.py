"""Seeded synthetic inputs shared by the HIP path's tests/bench and the oracle.

This module holds random draws only: no step of the encoder forward is computed
here. Every tensor is drawn from its own counter-based stream, so any element
can be regenerated alone (the full-size parity tests recompute sampled rows on
the host) and the same integer draws come out of numpy on the host and torch on
the device.

Stream definition (splitmix64 used as a counter-based generator):
  key      = mix64(master_seed ^ fnv1a64(name))          one key per tensor
  u64[i]   = mix64(key + (i + 1) * 0x9E3779B97F4A7C15)    mod 2**64
  mix64(z) = the splitmix64 output finaliser (Steele, Lea, Flood 2014):
             z ^= z >> 30; z *= 0xBF58476D1CE4E5B9; z ^= z >> 27;
             z *= 0x94D049BB133111EB; z ^= z >> 31
Derived draws:
  uniform (0,1]    ((u64 >> 11) + 1) * 2**-53
  normal           Box-Muller, cos branch, from uniforms at 2i and 2i+1
  int8 [-127,127]  ((u64 >> 32) * 255 >> 32) - 127     (integer only)
  length [lo,hi]   lo + ((u64 >> 32) * (hi - lo + 1) >> 32)
"""
from __future__ import annotations

import numpy as np

GAMMA = 0x9E3779B97F4A7C15
M1 = 0xBF58476D1CE4E5B9
M2 = 0x94D049BB133111EB
MASK64 = (1 << 64) - 1


def _mix64_int(z: int) -> int:
    z &= MASK64
    z ^= z >> 30
    z = (z * M1) & MASK64
    z ^= z >> 27
    z = (z * M2) & MASK64
    z ^= z >> 31
    return z


def fnv1a64(s: str) -> int:
    h = 0xCBF29CE484222325
    for b in s.encode("utf-8"):
        h ^= b
        h = (h * 0x100000001B3) & MASK64
    return h


def tensor_key(master_seed: int, name: str) -> int:
    """The 64-bit stream key of one named tensor under a master seed."""
    return _mix64_int((master_seed & MASK64) ^ fnv1a64(name))


# ----------------------------------------------------------------------------- numpy (host)

def _mix64_np(z: np.ndarray) -> np.ndarray:
    z = z ^ (z >> np.uint64(30))
    z = z * np.uint64(M1)
    z = z ^ (z >> np.uint64(27))
    z = z * np.uint64(M2)
    z = z ^ (z >> np.uint64(31))
    return z


def u64_np(key: int, start: int, count: int) -> np.ndarray:
    idx = np.arange(start + 1, start + 1 + count, dtype=np.uint64)
    with np.errstate(over="ignore"):
        x = np.uint64(key) + idx * np.uint64(GAMMA)
        return _mix64_np(x)


def uniform_np(key: int, start: int, count: int) -> np.ndarray:
    u = u64_np(key, start, count)
    return ((u >> np.uint64(11)).astype(np.float64) + 1.0) * (2.0 ** -53)


def normal_np(key: int, start: int, count: int) -> np.ndarray:
    """Standard normals n[start : start+count] of the stream (float64)."""
    u = uniform_np(key, 2 * start, 2 * count)
    u1, u2 = u[0::2], u[1::2]
    return np.sqrt(-2.0 * np.log(u1)) * np.cos(2.0 * np.pi * u2)


def int8_np(key: int, start: int, count: int) -> np.ndarray:
    u = u64_np(key, start, count) >> np.uint64(32)
    return (((u * np.uint64(255)) >> np.uint64(32)).astype(np.int64) - 127).astype(np.int8)


def ints_np(key: int, count: int, lo: int, hi: int) -> np.ndarray:
    """Integers uniform in [lo, hi] (inclusive), draws 0..count-1."""
    u = u64_np(key, 0, count) >> np.uint64(32)
    span = np.uint64(hi - lo + 1)
    return ((u * span) >> np.uint64(32)).astype(np.int64) + lo


# ----------------------------------------------------------------------------- torch (device)
# Only the integer-valued draws have a device twin: they are bit-identical to
# the numpy ones because they use integer arithmetic alone.

def _torch_mix64(z):
    import torch

    def lsr(v, s):  # logical shift right of int64 bit patterns
        return (v >> s) & ((1 << (64 - s)) - 1)

    z = z ^ lsr(z, 30)
    z = z * torch.tensor(M1 - (1 << 64), dtype=torch.int64, device=z.device)
    z = z ^ lsr(z, 27)
    z = z * torch.tensor(M2 - (1 << 64), dtype=torch.int64, device=z.device)
    z = z ^ lsr(z, 31)
    return z


def int8_torch(key: int, start: int, count: int, device, chunk: int = 1 << 26):
    """int8 draws start..start+count-1 generated on `device` (same values as int8_np)."""
    import torch

    out = torch.empty(count, dtype=torch.int8, device=device)
    k = key - (1 << 64) if key >= (1 << 63) else key
    g = GAMMA - (1 << 64)
    for c0 in range(0, count, chunk):
        c1 = min(count, c0 + chunk)
        idx = torch.arange(start + c0 + 1, start + c1 + 1, dtype=torch.int64, device=device)
        z = _torch_mix64(idx * g + k)
        u = (z >> 32) & 0xFFFFFFFF
        out[c0:c1] = (((u * 255) >> 32) - 127).to(torch.int8)
    return out
