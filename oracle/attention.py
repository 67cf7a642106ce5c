"""Single-query paged decode attention over TQ pages (dequantise, then softmax).

Test infrastructure (see ``oracle/__init__.py``).

Sources: "Architecture", "Diagnostic vs Serving Paths" (the TQ paged decode
reference reads packed pages and reconstructs rows inside the loop) and
"Cache Storage Objects" (page shape); "vLLM Usage", "TQ Packed Page
Contract" (``decode_tq4_paged``) and "Live Backend Gap" (decode through
block tables).

This is the plain definition, with no rotated-domain algebra: every key and
value row of the sequence is reconstructed densely in float64
(``k_t = n_k irht(c_K[idx_K])``), scores are ``scale <q, k_t>``, the softmax
subtracts the maximum, and the output is ``sum_t p_t v_t``.

Readings taken: query head h uses KV head ``h // (Hq / Hkv)``; the default
scale is ``1 / sqrt(head_dim)``; token t of sequence b lives in page
``block_table[b, t // block_size]`` at offset ``t % block_size``; a sequence
of length 0 produces zeros; rows that were never written decode to whatever
bytes the page holds (all-zero bytes decode to the zero vector).
"""

from __future__ import annotations

import numpy as np

from .codec import dequantize_rows

__all__ = ["gather_rows", "paged_decode", "paged_decode_heads", "paged_decode_hybrid", "paged_prefill"]


def gather_rows(pages, block_table_row, length, kv_head):
    """Row bytes of tokens 0..length-1 of one sequence for one KV head."""
    BS = pages.shape[1]
    t = np.arange(length)
    blocks = np.asarray(block_table_row)[t // BS]
    return pages[blocks, t % BS, kv_head]


def _attend(q64, K, V, scale):
    s = scale * (K @ q64)
    s = s - s.max()
    p = np.exp(s)
    p /= p.sum()
    return p @ V


def paged_decode_heads(q, k_pages, v_pages, block_table, seq_lens, k_bits, v_bits,
                       signs, ck32, cv32, heads, scale=None):
    """Outputs for the listed ``(b, h)`` pairs only -> float64 [len(heads), d].

    Reconstructs just the rows those heads need (used to check large
    workloads on a sample of heads).
    """
    q = np.asarray(q)
    B, Hq, d = q.shape
    Hkv = k_pages.shape[2]
    G = Hq // Hkv
    scale = 1.0 / np.sqrt(d) if scale is None else float(scale)
    out = np.zeros((len(heads), d), dtype=np.float64)
    cache = {}
    for i, (b, h) in enumerate(heads):
        L = int(seq_lens[b])
        if L == 0:
            continue
        g = h // G
        key = (b, g)
        if key not in cache:
            K = dequantize_rows(gather_rows(k_pages, block_table[b], L, g), k_bits, d, signs, ck32)
            V = dequantize_rows(gather_rows(v_pages, block_table[b], L, g), v_bits, d, signs, cv32)
            cache = {key: (K, V)}
        K, V = cache[key]
        out[i] = _attend(q[b, h].astype(np.float64), K, V, scale)
    return out


def paged_decode(q, k_pages, v_pages, block_table, seq_lens, k_bits, v_bits,
                 signs, ck32, cv32, scale=None):
    """Full decode: float32 ``[B, Hq, d]`` (computed in float64, rounded once)."""
    q = np.asarray(q)
    B, Hq, d = q.shape
    heads = [(b, h) for b in range(B) for h in range(Hq)]
    out = paged_decode_heads(q, k_pages, v_pages, block_table, seq_lens, k_bits, v_bits,
                             signs, ck32, cv32, heads, scale)
    return out.reshape(B, Hq, d).astype(np.float32)


def paged_decode_hybrid(q, k_pages, v_pages, block_table, seq_lens, recent_k, recent_v, recent_lens,
                        k_bits, v_bits, signs, ck32, cv32, scale=None):
    """Decode over packed history plus an exact recent window -> float32 ``[B, Hq, d]``.

    Sources: "Integration API" (vLLM hooks, the hybrid mode: compressed
    history plus the exact recent tokens for decode) and "Architecture",
    "Cache Lifecycle" (decoded tokens are appended to a recent window before
    they are flushed to packed pages).

    Readings: sequence b's context is its ``seq_lens[b]`` packed tokens
    (reconstructed as in ``paged_decode``) together with the first
    ``recent_lens[b]`` rows of ``recent_k[b] / recent_v[b]``
    (``[cap, Hkv, d]``, used exactly as given: fp16 / bf16 / fp32 values
    widened to float64); the window holds tokens the pages do not, and
    attention is over all of them with one softmax; order does not matter.
    A sequence with no token at all gives zeros.
    """
    q = np.asarray(q)
    B, Hq, d = q.shape
    Hkv = k_pages.shape[2]
    G = Hq // Hkv
    scale = 1.0 / np.sqrt(d) if scale is None else float(scale)
    rk = np.asarray(recent_k, dtype=np.float64)
    rv = np.asarray(recent_v, dtype=np.float64)
    if rk.shape[0] != B or rk.shape[2:] != (Hkv, d) or rv.shape != rk.shape:
        raise ValueError("recent window shape mismatch")
    cap = rk.shape[1]
    out = np.zeros((B, Hq, d), dtype=np.float64)
    for b in range(B):
        L, R = int(seq_lens[b]), int(recent_lens[b])
        if not 0 <= R <= cap:
            raise ValueError("recent length outside the window")
        if L + R == 0:
            continue
        for g in range(Hkv):
            K = V = np.zeros((0, d))
            if L > 0:
                K = dequantize_rows(gather_rows(k_pages, block_table[b], L, g), k_bits, d, signs, ck32)
                V = dequantize_rows(gather_rows(v_pages, block_table[b], L, g), v_bits, d, signs, cv32)
            K = np.concatenate([K, rk[b, :R, g]], axis=0)
            V = np.concatenate([V, rv[b, :R, g]], axis=0)
            for h in range(g * G, (g + 1) * G):
                out[b, h] = _attend(q[b, h].astype(np.float64), K, V, scale)
    return out.astype(np.float32)


def paged_prefill(q, q_lens, k_pages, v_pages, block_table, seq_lens, k_bits, v_bits, signs, ck32, cv32,
                  scale=None):
    """Several query tokens per sequence over the packed pages, causal -> float32 ``[B, Lq, Hq, d]``.

    Sources: "vLLM Usage", "Runtime Dispatch" (with a cache present, mixed
    prefill / decode batches attend through the packed cache) and
    "Architecture", "Cache Lifecycle" (prefill, then decode, over the
    compressed store).

    Readings: ``q[b, j]`` for ``j < q_lens[b]`` are the queries of the last
    ``q_lens[b]`` tokens of sequence b, whose K/V rows are already in the
    pages (the cache is updated before attention); query j sits at position
    ``P_b + j`` with ``P_b = seq_lens[b] - q_lens[b]`` and attends tokens
    ``0 .. P_b + j`` (causal within the chunk), rows reconstructed as in
    ``paged_decode``.  Rows ``j >= q_lens[b]`` are zeros.  ``q_lens[b]`` must
    lie in ``0 .. min(Lq, seq_lens[b])``.
    """
    q = np.asarray(q)
    B, Lq, Hq, d = q.shape
    Hkv = k_pages.shape[2]
    G = Hq // Hkv
    scale = 1.0 / np.sqrt(d) if scale is None else float(scale)
    out = np.zeros((B, Lq, Hq, d), dtype=np.float64)
    for b in range(B):
        L, n = int(seq_lens[b]), int(q_lens[b])
        if not 0 <= n <= min(Lq, L):
            raise ValueError("query length outside 0 .. min(Lq, seq_len)")
        if n == 0:
            continue
        P = L - n
        for g in range(Hkv):
            K = dequantize_rows(gather_rows(k_pages, block_table[b], L, g), k_bits, d, signs, ck32)
            V = dequantize_rows(gather_rows(v_pages, block_table[b], L, g), v_bits, d, signs, cv32)
            for j in range(n):
                for h in range(g * G, (g + 1) * G):
                    out[b, j, h] = _attend(q[b, j, h].astype(np.float64), K[: P + j + 1], V[: P + j + 1], scale)
    return out.astype(np.float32)

