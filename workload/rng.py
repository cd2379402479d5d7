"""Counter-based random numbers for the synthetic workloads.

Every value is a pure function of a key tuple and an element index, so any
row can be regenerated on demand and the same arrays feed both the CPU oracle
and the device path.  The generator is SplitMix64 (Steele, Lea and Flood,
"Fast splittable pseudorandom number generators", OOPSLA 2014) used as a hash:
``mix(key + (i + 1) * GOLDEN)`` for element ``i``.  Normals come from the
Box-Muller transform (cosine branch only, one normal per 64-bit word).

This module holds none of the ring method's arithmetic.
"""

from __future__ import annotations

import numpy as np

GOLDEN = np.uint64(0x9E3779B97F4A7C15)
_M1 = np.uint64(0xBF58476D1CE4E5B9)
_M2 = np.uint64(0x94D049BB133111EB)
_MASK64 = (1 << 64) - 1


def _mix(z: np.ndarray) -> np.ndarray:
    """SplitMix64 output function on a uint64 array (wrapping arithmetic)."""
    z = z.astype(np.uint64, copy=True)
    with np.errstate(over="ignore"):
        z ^= z >> np.uint64(30)
        z *= _M1
        z ^= z >> np.uint64(27)
        z *= _M2
        z ^= z >> np.uint64(31)
    return z


def _mix_int(z: int) -> int:
    z &= _MASK64
    z ^= z >> 30
    z = (z * 0xBF58476D1CE4E5B9) & _MASK64
    z ^= z >> 27
    z = (z * 0x94D049BB133111EB) & _MASK64
    z ^= z >> 31
    return z


def key_of(*parts: int) -> int:
    """Fold an ordered tuple of non-negative integers into one 64-bit key."""
    k = 0x243F6A8885A308D3
    for p in parts:
        k = _mix_int((k ^ (int(p) & _MASK64)) + 0x9E3779B97F4A7C15)
    return k


def u64(keys: np.ndarray, n: int) -> np.ndarray:
    """Words ``[len(keys), n]``: element i of row r is mix(keys[r] + (i+1)*GOLDEN)."""
    keys = np.asarray(keys, dtype=np.uint64).reshape(-1, 1)
    idx = np.arange(1, n + 1, dtype=np.uint64).reshape(1, -1)
    with np.errstate(over="ignore"):
        z = keys + idx * GOLDEN
    return _mix(z)


def uniform(keys: np.ndarray, n: int) -> np.ndarray:
    """Uniform doubles in [0, 1) with 53 random bits, shape ``[len(keys), n]``."""
    w = u64(keys, n)
    return (w >> np.uint64(11)).astype(np.float64) * (1.0 / 9007199254740992.0)


def normal(keys: np.ndarray, n: int) -> np.ndarray:
    """Standard normals (float64), shape ``[len(keys), n]``.

    The high 32 bits give u1 in (0, 1], the low 32 bits give u2 in [0, 1);
    z = sqrt(-2 ln u1) * cos(2 pi u2).
    """
    w = u64(keys, n)
    hi = (w >> np.uint64(32)).astype(np.float64)
    lo = (w & np.uint64(0xFFFFFFFF)).astype(np.float64)
    u1 = (hi + 1.0) * (1.0 / 4294967296.0)
    u2 = lo * (1.0 / 4294967296.0)
    return np.sqrt(-2.0 * np.log(u1)) * np.cos(2.0 * np.pi * u2)


def row_keys(base: int, ids: np.ndarray) -> np.ndarray:
    """Per-row keys: mix(base ^ id) for an array of non-negative row ids."""
    ids = np.asarray(ids, dtype=np.int64).astype(np.uint64)
    with np.errstate(over="ignore"):
        return _mix(np.uint64(base) ^ (ids * GOLDEN + np.uint64(0x632BE59BD9B4E019)))
