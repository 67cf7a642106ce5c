"""Inner-product ("prod") key codec: (b-1)-bit MSE indices plus a 1-bit QJL
sketch of the residual.

Test infrastructure (see ``oracle/__init__.py``).

Sources: "vLLM Reference Audit", File Map row "MSE and QJL codecs"
(``TurboQuantMSE``, ``TurboQuantProd``; data: indices, norms, signs) and
Feature Checklist row "QJL residual"; "Architecture", Responsibility Matrix
(core: vector transforms, codebooks, MSE, QJL, packed MSE/QJL payloads).

The pages name the codec and its payload but print none of its arithmetic.
Readings taken (the published TurboQuant inner-product quantiser, which
spends one of the b bits on a quantised Johnson-Lindenstrauss sketch of the
MSE residual, restated here):

* A b-bit prod row encodes the rotated unit vector r = rht(x / n) with the
  (b-1)-bit MSE codec (``codec.encode_rows``: indices of the Lloyd-Max
  codebook for d, b - 1), then sketches the rotated residual
  e = r - c[idx]: with a d x d matrix S of i.i.d. N(0, 1) entries,
  z_i = +1 when (S e)_i >= 0, else -1, and gamma = ||e||_2.
* The inner product of a query y with the row's vector is estimated as
  ``n * (<y~, c[idx]> + gamma * sqrt(pi / 2) / d * <S y~, z>)`` with
  y~ = rht(y); over the draw of S its mean is <y, x>, because
  E[<s, a> sign(<s, e>)] = sqrt(2 / pi) <a, e> / ||e|| for a Gaussian row s.
* S is an input (the random numbers the method draws are passed in).
* Row layout (the pages give none): ceil(d (b-1) / 8) index bytes (LSB-first,
  as the MSE rows), the fp32 norm n, d / 8 sign bytes (stream bit i = 1 when
  z_i = +1, LSB-first), the fp32 gamma; little-endian.  At d = 128, b = 4:
  48 + 4 + 16 + 4 = 72 bytes.
* gamma is ||e|| in float64 rounded once to fp32.  A sign whose projection
  lies within 3e-5 of sum_j |S_ij e_j| of zero is marked near (an fp32 dot
  product of 128 terms can land on either side of zero there).
"""

from __future__ import annotations

import numpy as np

from .codebook import beta_codebook
from .codec import encode_rows, index_bytes, pack_indices, unpack_indices
from .rht import rht

__all__ = [
    "prod_row_bytes",
    "encode_prod",
    "prod_rows_to_bytes",
    "prod_bytes_to_rows",
    "prod_scores",
    "write_prod",
    "paged_prod_scores",
    "NEAR_SIGN",
]

#: relative distance to zero (of sum |S_ij e_j|) under which a sign decision counts as "near"
NEAR_SIGN = 3e-5


def prod_row_bytes(d: int, bits: int) -> int:
    return index_bytes(d, bits - 1) + 4 + d // 8 + 4


def encode_prod(x, bits: int, signs, S):
    """Encode rows ``x[..., d]`` (fp16 / fp32).

    Returns ``(idx uint8[..., d], norm32 float32[...], z bool[..., d] (True = +1),
    gamma32 float32[...], near_idx bool[..., d], near_sign bool[..., d])``.
    """
    x = np.asarray(x)
    d = x.shape[-1]
    _, c32, t64 = beta_codebook(d, bits - 1)
    idx, norm32, r, near_idx = encode_rows(x, bits - 1, signs, t64)
    e = r - c32.astype(np.float64)[idx.astype(np.int64)]
    gamma = np.sqrt(np.sum(e * e, axis=-1))
    S = np.asarray(S, dtype=np.float64)
    proj = e @ S.T
    z = proj >= 0.0
    near_sign = np.abs(proj) <= NEAR_SIGN * (np.abs(e) @ np.abs(S).T)
    return idx, norm32, z, gamma.astype(np.float32), near_idx, near_sign


def prod_rows_to_bytes(idx, norm32, z, gamma32, bits: int) -> np.ndarray:
    """Row bytes: indices, norm, sign bits, gamma."""
    z = np.asarray(z, dtype=bool)
    sign_bytes = np.packbits(z, axis=-1, bitorder="little")
    nb = np.asarray(norm32, dtype="<f4")[..., None].view(np.uint8)
    gb = np.asarray(gamma32, dtype="<f4")[..., None].view(np.uint8)
    return np.concatenate([pack_indices(idx, bits - 1), nb, sign_bytes, gb], axis=-1)


def prod_bytes_to_rows(rows, bits: int, d: int):
    """Split prod row bytes into ``(idx, norm32, z bool, gamma32)``."""
    rows = np.asarray(rows, dtype=np.uint8)
    ib = index_bytes(d, bits - 1)
    if rows.shape[-1] != prod_row_bytes(d, bits):
        raise ValueError("row length does not match bits")
    idx = unpack_indices(rows[..., :ib], bits - 1, d)
    norm = np.ascontiguousarray(rows[..., ib:ib + 4]).view("<f4")[..., 0]
    z = np.unpackbits(rows[..., ib + 4:ib + 4 + d // 8], axis=-1, bitorder="little").astype(bool)
    gamma = np.ascontiguousarray(rows[..., ib + 4 + d // 8:]).view("<f4")[..., 0]
    return idx, norm.astype(np.float32), z, gamma.astype(np.float32)


def prod_scores(y, rows, bits: int, signs, S):
    """Estimated inner products of query ``y[d]`` (or of each query of
    ``y[m, d]``) with each row of ``rows[..., RB]`` (float64; shape
    ``rows.shape[:-1]``, or ``(m,) + rows.shape[:-1]``)."""
    d = len(signs)
    idx, norm, z, gamma = prod_bytes_to_rows(rows, bits, d)
    _, c32, _ = beta_codebook(d, bits - 1)
    y = np.asarray(y, dtype=np.float64)
    yr = rht(np.atleast_2d(y), signs)                 # y~ per query, [m, d]
    sy = yr @ np.asarray(S, dtype=np.float64).T       # S y~ per query
    mse = c32.astype(np.float64)[idx.astype(np.int64)] @ yr.T   # [..., m]
    qjl = np.where(z, 1.0, -1.0) @ sy.T
    est = norm.astype(np.float64)[..., None] * (mse + gamma.astype(np.float64)[..., None] * np.sqrt(np.pi / 2.0) / d * qjl)
    est = np.moveaxis(est, -1, 0)
    return est[0] if y.ndim == 1 else est


def write_prod(raw, pages, slots, bits: int, signs, S):
    """Write prod rows of ``raw[N, Hkv, d]`` into a copy of ``pages[NB, BS, Hkv, RB]``.

    Slot rules as ``codec.write_kv`` (negative skipped, out of range raises).
    Returns ``(pages_out, near_idx, near_sign)`` with the near masks laid out
    ``[NB, BS, Hkv, d]``.
    """
    raw = np.asarray(raw)
    pages = np.asarray(pages, dtype=np.uint8)
    slots = np.asarray(slots, dtype=np.int64)
    N, Hkv, d = raw.shape
    NB, BS, Hp, RB = pages.shape
    if Hp != Hkv or RB != prod_row_bytes(d, bits) or slots.shape != (N,):
        raise ValueError("shape mismatch")
    if np.any(slots >= NB * BS):
        raise IndexError("slot outside the allocated pages")
    out = pages.copy()
    near_i = np.zeros((NB, BS, Hkv, d), dtype=bool)
    near_s = np.zeros((NB, BS, Hkv, d), dtype=bool)
    keep = slots >= 0
    if np.any(keep):
        idx, n32, z, g32, ni, ns = encode_prod(raw[keep], bits, signs, S)
        s = slots[keep]
        out[s // BS, s % BS] = prod_rows_to_bytes(idx, n32, z, g32, bits)
        near_i[s // BS, s % BS] = ni
        near_s[s // BS, s % BS] = ns
    return out, near_i, near_s


def paged_prod_scores(q, pages, block_table, seq_lens, bits: int, signs, S):
    """Estimated <q[b, h], k_t> for every token t < seq_lens[b] of KV head h // G
    -> float64 ``[B, Hq, max(seq_lens)]`` (zeros past a sequence's length)."""
    q = np.asarray(q)
    B, Hq, d = q.shape
    BS, Hkv = pages.shape[1], pages.shape[2]
    G = Hq // Hkv
    Lmax = int(np.max(seq_lens)) if B else 0
    out = np.zeros((B, Hq, Lmax))
    for b in range(B):
        L = int(seq_lens[b])
        if L == 0:
            continue
        t = np.arange(L)
        blk = np.asarray(block_table[b])[t // BS]
        for g in range(Hkv):
            out[b, g * G:(g + 1) * G, :L] = prod_scores(q[b, g * G:(g + 1) * G], pages[blk, t % BS, g], bits, signs, S)
    return out
