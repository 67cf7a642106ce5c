"""TQ row codec and the paged row writer.

Test infrastructure (see ``oracle/__init__.py``).

Sources:

* "vLLM Usage", "TQ Byte Layout": for one component (K or V), one token and
  one KV head, ``index_bytes = ceil(head_dim * bits / 8)`` and
  ``row_bytes = index_bytes + 4``; the last four bytes are the fp32 norm;
  K and V are stored independently (K4/V2 = 68 + 36 = 104 bytes at d=128).
* "vLLM Usage", "Slot Mapping": flat slots, negative slots ignored, a slot
  outside the allocated pages raises.
* "Architecture", "Cache Storage Objects": pages are uint8
  ``[num_blocks, block_size, num_kv_heads, row_bytes]``.
* "vLLM Reference Audit", File Map rows "MSE and QJL codecs" (indices and
  norms) and "bit packing" (1/2/3/4/5-bit).

Readings taken:

* Encode (MSE codec): norm n = ||x||_2; u = x / n (u = 0 when n = 0);
  r = rht(u); index = number of codebook boundaries strictly below r (the
  nearest centroid, ties to the lower index).
* The norm is the correctly rounded float64 sum of the squares (every x_i^2
  of an fp16/fp32 input is exact in float64), its float64 square root, then
  rounded to float32 (round to nearest even).  Stored little-endian.
* Bit packing is one LSB-first bit stream: bit k of the stream is bit
  (k mod b) of index floor(k / b); stream bit 8j + i is bit i of byte j.
  Unused high bits of the last index byte are zero.  No row or page padding.
"""

from __future__ import annotations

import math
import struct

import numpy as np

from .codebook import beta_codebook
from .rht import rht, irht, rht_signs

__all__ = [
    "index_bytes",
    "row_bytes",
    "encode_rows",
    "pack_indices",
    "unpack_indices",
    "rows_to_bytes",
    "bytes_to_rows",
    "dequantize_rows",
    "write_kv",
    "decompress_kv",
    "OracleCodec",
    "NEAR_BOUNDARY",
]

#: distance to a boundary under which an index decision counts as "near"
NEAR_BOUNDARY = 1e-6


def index_bytes(d: int, bits: int) -> int:
    return (d * bits + 7) // 8


def row_bytes(d: int, bits: int) -> int:
    return index_bytes(d, bits) + 4


def _norms(x64: np.ndarray) -> np.ndarray:
    """sqrt(correctly rounded float64 sum of squares) per row."""
    flat = x64.reshape(-1, x64.shape[-1])
    sq = flat * flat  # exact for fp16 / fp32 inputs
    out = np.empty(flat.shape[0], dtype=np.float64)
    for i in range(flat.shape[0]):
        out[i] = math.fsum(sq[i])
    return np.sqrt(out).reshape(x64.shape[:-1])


def encode_rows(x, bits: int, signs: np.ndarray, t64: np.ndarray):
    """Encode rows ``x[..., d]`` (fp16 or fp32 values).

    Returns ``(idx uint8[..., d], norm32 float32[...], r float64[..., d],
    near bool[..., d])`` where ``r`` is the rotated unit vector and ``near``
    marks coordinates within ``NEAR_BOUNDARY`` of a boundary.
    """
    x = np.asarray(x)
    if x.dtype not in (np.float16, np.float32):
        raise TypeError("rows must be float16 or float32")
    x64 = x.astype(np.float64)
    n64 = _norms(x64)
    norm32 = n64.astype(np.float32)
    safe = np.where(n64 > 0, n64, 1.0)
    u = np.where((n64 > 0)[..., None], x64 / safe[..., None], 0.0)
    r = rht(u, signs)
    idx = np.zeros(r.shape, dtype=np.int64)
    near = np.zeros(r.shape, dtype=bool)
    for t in t64:  # count boundaries strictly below r
        idx += t < r
        near |= np.abs(r - t) < NEAR_BOUNDARY
    return idx.astype(np.uint8), norm32, r, near


def pack_indices(idx, bits: int) -> np.ndarray:
    """LSB-first bit stream of b-bit indices ``idx[..., d]`` -> uint8[..., ceil(d b / 8)]."""
    idx = np.asarray(idx, dtype=np.int64)
    if np.any(idx < 0) or np.any(idx >= (1 << bits)):
        raise ValueError("index out of range for bit width")
    lead, d = idx.shape[:-1], idx.shape[-1]
    stream = ((idx[..., :, None] >> np.arange(bits)) & 1).reshape(lead + (d * bits,))
    nbytes = index_bytes(d, bits)
    pad = nbytes * 8 - d * bits
    if pad:
        stream = np.concatenate([stream, np.zeros(lead + (pad,), dtype=stream.dtype)], axis=-1)
    weights = 1 << np.arange(8)
    return (stream.reshape(lead + (nbytes, 8)) * weights).sum(-1).astype(np.uint8)


def unpack_indices(packed, bits: int, d: int) -> np.ndarray:
    """Inverse of ``pack_indices``."""
    packed = np.asarray(packed, dtype=np.uint8)
    lead = packed.shape[:-1]
    stream = ((packed[..., :, None].astype(np.int64) >> np.arange(8)) & 1).reshape(lead + (-1,))
    stream = stream[..., : d * bits].reshape(lead + (d, bits))
    return (stream << np.arange(bits)).sum(-1).astype(np.uint8)


def rows_to_bytes(idx, norm32, bits: int) -> np.ndarray:
    """Row bytes = packed indices followed by the float32 norm, little-endian."""
    packed = pack_indices(idx, bits)
    nb = np.asarray(norm32, dtype="<f4")[..., None].view(np.uint8)
    return np.concatenate([packed, nb], axis=-1)


def bytes_to_rows(rows, bits: int, d: int):
    """Split row bytes into (indices uint8[..., d], norm float32[...])."""
    rows = np.asarray(rows, dtype=np.uint8)
    ib = index_bytes(d, bits)
    if rows.shape[-1] != ib + 4:
        raise ValueError("row length does not match bits")
    idx = unpack_indices(rows[..., :ib], bits, d)
    norm = np.ascontiguousarray(rows[..., ib : ib + 4]).view("<f4")[..., 0].astype(np.float32)
    return idx, norm


def dequantize_rows(rows, bits: int, d: int, signs: np.ndarray, c32: np.ndarray) -> np.ndarray:
    """Reconstruct float64 rows: n * irht(c[idx])."""
    idx, norm = bytes_to_rows(rows, bits, d)
    cent = c32.astype(np.float64)[idx.astype(np.int64)]
    return norm.astype(np.float64)[..., None] * irht(cent, signs)


def write_kv(raw, pages, slots, bits: int, signs, t64):
    """Write rows ``raw[N, Hkv, d]`` into a copy of ``pages[NB, BS, Hkv, RB]``.

    All slots are validated first: any slot >= NB*BS raises ``IndexError``
    and nothing is written.  Token n with slot s >= 0 writes head h's row to
    ``pages[s // BS, s % BS, h]``; negative slots leave the pages untouched.

    Returns ``(pages_out, near)`` where ``near`` (bool ``[NB, BS, Hkv, d]``)
    marks index fields whose coordinate lay within ``NEAR_BOUNDARY`` of a
    codebook boundary when written.
    """
    raw = np.asarray(raw)
    pages = np.asarray(pages, dtype=np.uint8)
    slots = np.asarray(slots, dtype=np.int64)
    N, Hkv, d = raw.shape
    NB, BS, Hp, RB = pages.shape
    if Hp != Hkv or RB != row_bytes(d, bits) or slots.shape != (N,):
        raise ValueError("shape mismatch")
    if np.any(slots >= NB * BS):
        raise IndexError("slot outside the allocated pages")
    out = pages.copy()
    near_all = np.zeros((NB, BS, Hkv, d), dtype=bool)
    keep = slots >= 0
    if np.any(keep):
        idx, norm32, _, near = encode_rows(raw[keep], bits, signs, t64)
        rb = rows_to_bytes(idx, norm32, bits)
        s = slots[keep]
        out[s // BS, s % BS] = rb
        near_all[s // BS, s % BS] = near
    return out, near_all


def decompress_kv(pages, slots, bits: int, signs, c32):
    """Dense rows read back from ``pages[NB, BS, Hkv, RB]`` -> float64 ``[N, Hkv, d]``.

    Sources: "Architecture", "Data Flow" (packed bytes lead to a diagnostic
    dense reconstruction, kept apart from compressed attention) and "vLLM
    Reference Audit", File Map row "TQ4 unpack kernel" (packed index bytes
    and norms in, rows out, a diagnostic readback into a caller's buffer).

    Token n's row for head h is the row stored at flat slot ``slots[n]``
    ("vLLM Usage", "Slot Mapping"), reconstructed as ``n * irht(c[idx])``.
    Readings: a negative slot names no stored row, so its rows are zeros; a
    slot at or past ``NB * BS`` raises ``IndexError``, as the write does.
    """
    pages = np.asarray(pages, dtype=np.uint8)
    slots = np.asarray(slots, dtype=np.int64)
    NB, BS, Hkv, RB = pages.shape
    d = len(signs)
    if RB != row_bytes(d, bits) or slots.ndim != 1:
        raise ValueError("shape mismatch")
    if np.any(slots >= NB * BS):
        raise IndexError("slot outside the allocated pages")
    out = np.zeros((slots.shape[0], Hkv, d), dtype=np.float64)
    keep = slots >= 0
    if np.any(keep):
        s = slots[keep]
        out[keep] = dequantize_rows(pages[s // BS, s % BS], bits, d, signs, c32)
    return out


class OracleCodec:
    """Signs and codebooks for one head_dim and rotation seed."""

    def __init__(self, head_dim: int = 128, seed: int = 42):
        self.d = int(head_dim)
        self.seed = int(seed)
        self.signs = rht_signs(self.seed, self.d)

    def codebook(self, bits):
        return beta_codebook(self.d, bits)

    def centroids32(self, bits):
        return beta_codebook(self.d, bits)[1]

    def boundaries(self, bits):
        return beta_codebook(self.d, bits)[2]

    def encode(self, x, bits):
        return encode_rows(x, bits, self.signs, self.boundaries(bits))

    def encode_bytes(self, x, bits):
        idx, norm32, _, near = self.encode(x, bits)
        return rows_to_bytes(idx, norm32, bits), near

    def dequantize(self, rows, bits):
        return dequantize_rows(rows, bits, self.d, self.signs, self.centroids32(bits))

    def write_kv(self, raw, pages, slots, bits):
        return write_kv(raw, pages, slots, bits, self.signs, self.boundaries(bits))

    def decompress_kv(self, pages, slots, bits):
        return decompress_kv(pages, slots, bits, self.signs, self.centroids32(bits))


def norm_bytes(norm32) -> bytes:
    """Little-endian bytes of a float32 norm (helper for tests)."""
    return struct.pack("<f", float(np.float32(norm32)))
