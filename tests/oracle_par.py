"""Run the oracle on independent chunks in threads, for the full-size checks.

Only scheduling lives here: every byte and every output still comes from the
oracle's own functions (``OracleCodec.write_kv`` on a run of whole pages,
``oracle.paged_decode_heads`` on one KV head's query group); the results are
put back together in order.  numpy releases the interpreter lock inside its
kernels, so threads give most of the machine's cores without copying inputs
to other processes.
"""

from __future__ import annotations

import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np

import oracle

#: tokens per chunk: a whole number of 16-token pages
CHUNK_TOKENS = 2048


def _threads():
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:
        n = os.cpu_count() or 4
    return max(1, min(16, n))


def sequence_pages(codec, w, b, comp, bits):
    """The oracle's pages of sequence ``b`` for component 'k' or 'v'.

    Token t of the sequence goes to page t // 16, offset t % 16 of a fresh
    zero page tensor (its identity block table); tokens whose flat slot is -1
    in the workload stay zero, as in the workload's own pages.  Returns
    ``(pages [npg, 16, Hkv, RB], near [npg, 16, Hkv, d], kept_tokens)``.
    """
    L = int(w.seq_lens[b])
    bs = w.block_size
    raw = w.seq_rows(comp, b)
    lo = int(w.cu_seqlens[b])
    dropped = w.slots[lo:lo + L] < 0

    def job(c0):
        c1 = min(L, c0 + CHUNK_TOKENS)
        n = c1 - c0
        npg = (n + bs - 1) // bs
        slots = np.where(dropped[c0:c1], -1, np.arange(n)).astype(np.int64)
        zero = np.zeros((npg, bs, w.num_kv_heads, w.row_bytes(bits)), dtype=np.uint8)
        return codec.write_kv(raw[c0:c1], zero, slots, bits)

    with ThreadPoolExecutor(_threads()) as ex:
        parts = list(ex.map(job, range(0, L, CHUNK_TOKENS)))
    pages = np.concatenate([p for p, _ in parts])
    near = np.concatenate([nr for _, nr in parts])
    return pages, near, int((~dropped).sum())


def sequence_outputs(codec, w, b, k_pages, v_pages, queries):
    """Oracle outputs ``[Hq, d]`` of every query head of sequence ``b`` from its
    own pages (identity block table), one KV head's group per thread."""
    L = int(w.seq_lens[b])
    Hq, Hkv = w.num_q_heads, w.num_kv_heads
    G = Hq // Hkv
    if L == 0:
        return np.zeros((Hq, w.head_dim))
    npg = k_pages.shape[0]
    bt = np.arange(npg, dtype=np.int32)[None]
    q = queries[b][None]
    ck, cv = codec.centroids32(w.k_bits), codec.centroids32(w.v_bits)

    def job(g):
        heads = [(0, h) for h in range(g * G, (g + 1) * G)]
        return oracle.paged_decode_heads(q, k_pages, v_pages, bt, np.array([L]), w.k_bits, w.v_bits,
                                         codec.signs, ck, cv, heads)

    with ThreadPoolExecutor(min(_threads(), Hkv)) as ex:
        parts = list(ex.map(job, range(Hkv)))
    return np.concatenate(parts)


def sequence_hybrid_outputs(codec, w, b, k_pages, v_pages, queries, recent_k, recent_v, recent_len):
    """``oracle.paged_decode_hybrid`` outputs ``[Hq, d]`` of sequence ``b`` from
    its own pages (identity block table) and its window rows ``[cap, Hkv, d]``,
    one KV head (its pages' and window's head slice, its query group) per
    thread."""
    L = int(w.seq_lens[b])
    Hq, Hkv = w.num_q_heads, w.num_kv_heads
    G = Hq // Hkv
    npg = k_pages.shape[0]
    bt = np.arange(max(npg, 1), dtype=np.int32)[None]
    ck, cv = codec.centroids32(w.k_bits), codec.centroids32(w.v_bits)

    def job(g):
        kp = np.ascontiguousarray(k_pages[:, :, g:g + 1])
        vp = np.ascontiguousarray(v_pages[:, :, g:g + 1])
        q = queries[b][None, g * G:(g + 1) * G]
        return oracle.paged_decode_hybrid(q, kp, vp, bt, np.array([L]), recent_k[None, :, g:g + 1],
                                          recent_v[None, :, g:g + 1], np.array([recent_len]), w.k_bits, w.v_bits,
                                          codec.signs, ck, cv)[0]

    with ThreadPoolExecutor(min(_threads(), Hkv)) as ex:
        parts = list(ex.map(job, range(Hkv)))
    return np.concatenate(parts).astype(np.float64)


def sequence_prefill_outputs(codec, w, b, k_pages, v_pages, q, q_len):
    """``oracle.paged_prefill`` outputs ``[Lq, Hq, d]`` of sequence ``b`` from
    its own pages (identity block table), one KV head (its pages' head slice,
    its query group) per thread; ``q`` is the sequence's ``[Lq, Hq, d]``."""
    L = int(w.seq_lens[b])
    Hq, Hkv = w.num_q_heads, w.num_kv_heads
    G = Hq // Hkv
    npg = k_pages.shape[0]
    bt = np.arange(max(npg, 1), dtype=np.int32)[None]
    ck, cv = codec.centroids32(w.k_bits), codec.centroids32(w.v_bits)

    def job(g):
        kp = np.ascontiguousarray(k_pages[:, :, g:g + 1])
        vp = np.ascontiguousarray(v_pages[:, :, g:g + 1])
        return oracle.paged_prefill(q[None, :, g * G:(g + 1) * G], np.array([q_len]), kp, vp, bt, np.array([L]),
                                    w.k_bits, w.v_bits, codec.signs, ck, cv)[0]

    with ThreadPoolExecutor(min(_threads(), Hkv)) as ex:
        parts = list(ex.map(job, range(Hkv)))
    return np.concatenate(parts, axis=1).astype(np.float64)


def sequence_prod_pages(w, b, bits, signs, S):
    """The oracle's prod key pages of sequence ``b`` (identity block table), as
    ``sequence_pages``: ``(pages, near_idx, near_sign, kept_tokens)``."""
    L = int(w.seq_lens[b])
    bs = w.block_size
    raw = w.seq_rows("k", b)
    lo = int(w.cu_seqlens[b])
    dropped = w.slots[lo:lo + L] < 0

    def job(c0):
        c1 = min(L, c0 + CHUNK_TOKENS)
        n = c1 - c0
        npg = (n + bs - 1) // bs
        slots = np.where(dropped[c0:c1], -1, np.arange(n)).astype(np.int64)
        zero = np.zeros((npg, bs, w.num_kv_heads, oracle.prod_row_bytes(w.head_dim, bits)), dtype=np.uint8)
        return oracle.write_prod(raw[c0:c1], zero, slots, bits, signs, S)

    with ThreadPoolExecutor(_threads()) as ex:
        parts = list(ex.map(job, range(0, L, CHUNK_TOKENS)))
    return (np.concatenate([p[0] for p in parts]), np.concatenate([p[1] for p in parts]),
            np.concatenate([p[2] for p in parts]), int((~dropped).sum()))

