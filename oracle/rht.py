"""Seeded randomized Hadamard transform (RHT).

Test infrastructure (see ``oracle/__init__.py``).

Source: "vLLM Usage", "TQ Packed Page Contract" builds the rotation with
``build_rotation(dim, RotationMode.RHT, device, seed=42)``; "vLLM Reference
Audit", Feature Checklist row "QR/RHT/block-Hadamard transforms".

Readings taken (the pages give only the name and the seed):

* RHT = a random +-1 diagonal D followed by the orthonormal Sylvester
  Hadamard matrix: ``rht(u) = H (s * u) / sqrt(d)`` with
  ``H[i, j] = (-1)^popcount(i & j)`` (natural order); its inverse is
  ``irht(y) = s * (H y) / sqrt(d)`` because H = H^T and H H = d I.
* The +-1 signs come from SplitMix64 (Steele, Lea & Flood, "Fast splittable
  pseudorandom number generators", OOPSLA 2014) seeded with the rotation
  seed: s_i = -1 when the top bit of the i-th output is set.  The pages do
  not print their generator, so byte parity with their package is
  unpinned; the generator itself is pinned to its published outputs.
* One rotation (one seed) serves K, V, the query and the output, for every
  head.
"""

from __future__ import annotations

import numpy as np

__all__ = ["splitmix64", "rht_signs", "fwht", "rht", "irht"]

_MASK64 = (1 << 64) - 1


def splitmix64(seed: int, n: int):
    """First ``n`` outputs of SplitMix64 from state ``seed`` (Python ints).

    state += 0x9E3779B97F4A7C15; z = state;
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EB;
    out = z ^ (z >> 31)        (all arithmetic mod 2^64)
    """
    state = seed & _MASK64
    out = []
    for _ in range(n):
        state = (state + 0x9E3779B97F4A7C15) & _MASK64
        z = state
        z = ((z ^ (z >> 30)) * 0xBF58476D1CE4E5B9) & _MASK64
        z = ((z ^ (z >> 27)) * 0x94D049BB133111EB) & _MASK64
        z = z ^ (z >> 31)
        out.append(z)
    return out


def rht_signs(seed: int, d: int) -> np.ndarray:
    """The diagonal of D: s_i = -1 if bit 63 of the i-th SplitMix64 output."""
    return np.array([-1 if (z >> 63) else 1 for z in splitmix64(seed, d)], dtype=np.int8)


def fwht(x: np.ndarray) -> np.ndarray:
    """Unnormalised Walsh-Hadamard transform along the last axis (float64).

    Butterflies (a, b) -> (a + b, a - b) on index pairs (i, i + h) with bit h
    of i clear, for h = 1, 2, 4, ..., d/2.  Equals multiplication by the
    Sylvester matrix H[i, j] = (-1)^popcount(i & j).
    """
    y = np.array(x, dtype=np.float64, copy=True)
    d = y.shape[-1]
    if d & (d - 1):
        raise ValueError("length must be a power of two")
    lead = y.shape[:-1]
    h = 1
    while h < d:
        v = y.reshape(lead + (d // (2 * h), 2, h))
        a = v[..., 0, :].copy()
        b = v[..., 1, :]
        v[..., 0, :] = a + b
        v[..., 1, :] = a - b
        h *= 2
    return y


def rht(u: np.ndarray, signs: np.ndarray) -> np.ndarray:
    """rht(u) = H (s * u) / sqrt(d)."""
    d = u.shape[-1]
    return fwht(np.asarray(u, dtype=np.float64) * signs.astype(np.float64)) / np.sqrt(d)


def irht(y: np.ndarray, signs: np.ndarray) -> np.ndarray:
    """irht(y) = s * (H y) / sqrt(d), the inverse (= transpose) of rht."""
    d = y.shape[-1]
    return signs.astype(np.float64) * fwht(np.asarray(y, dtype=np.float64)) / np.sqrt(d)
