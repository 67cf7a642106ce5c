"""Pins for the oracle's hybrid decode (packed history + exact recent window), CPU only.

References: torch's scaled_dot_product_attention on the CPU in float64 over
the concatenated rows (history reconstructed densely, window rows as given),
the special cases that reduce to one part, and invariants of one softmax
over a union of tokens.
"""

import numpy as np
import pytest
import torch

import oracle
from paged_decode_attention_tq_amd import workloads


def _setup(w):
    codec = oracle.OracleCodec(w.head_dim, w.rht_seed)
    kp, _ = codec.write_kv(w.rows("k"), w.zero_pages(w.k_bits), w.slots, w.k_bits)
    vp, _ = codec.write_kv(w.rows("v"), w.zero_pages(w.v_bits), w.slots, w.v_bits)
    return codec, kp, vp


def _hybrid(w, codec, kp, vp, rk, rv, rl, q=None, lens=None, scale=None):
    return oracle.paged_decode_hybrid(
        w.queries() if q is None else q, kp, vp, w.block_table, w.seq_lens if lens is None else lens,
        rk, rv, rl, w.k_bits, w.v_bits, codec.signs, codec.centroids32(w.k_bits), codec.centroids32(w.v_bits),
        scale)


def _small(**kw):
    base = dict(head_dim=128, k_bits=4, v_bits=2, num_q_heads=8, num_kv_heads=2,
                block_size=16, seq_lens=[37, 1, 64, 0, 20], seed=11, extra_blocks=2)
    base.update(kw)
    return workloads.make_workload("hyb", **base)


def _sdpa(q, K, V, G):
    """q [Hq, d], K/V [L, Hkv, d] float64 -> [Hq, d] by torch SDPA."""
    Kt = torch.from_numpy(K).permute(1, 0, 2).repeat_interleave(G, 0)
    Vt = torch.from_numpy(V).permute(1, 0, 2).repeat_interleave(G, 0)
    return torch.nn.functional.scaled_dot_product_attention(torch.from_numpy(q)[:, None, :], Kt, Vt)[:, 0].numpy()


def test_matches_sdpa_over_history_and_window():
    w = _small()
    codec, kp, vp = _setup(w)
    rl = np.array([5, 0, 16, 7, 1])
    rk, rv = w.recent_window(16, rl, seed=1)
    out = _hybrid(w, codec, kp, vp, rk, rv, rl).astype(np.float64)
    q = w.queries().astype(np.float64)
    G = w.num_q_heads // w.num_kv_heads
    for b in range(w.batch):
        L, R = int(w.seq_lens[b]), int(rl[b])
        if L + R == 0:
            assert not out[b].any()
            continue
        t = np.arange(L)
        blk = w.block_table[b, t // 16]
        Kh = codec.dequantize(kp[blk, t % 16], w.k_bits) if L else np.zeros((0, w.num_kv_heads, 128))
        Vh = codec.dequantize(vp[blk, t % 16], w.v_bits) if L else np.zeros((0, w.num_kv_heads, 128))
        K = np.concatenate([Kh, rk[b, :R].astype(np.float64)])
        V = np.concatenate([Vh, rv[b, :R].astype(np.float64)])
        np.testing.assert_allclose(out[b], _sdpa(q[b], K, V, G), rtol=1e-6, atol=1e-6)


def test_window_only_and_empty():
    w = _small(seq_lens=[0, 0, 0])
    codec, kp, vp = _setup(w)
    rl = np.array([9, 0, 1])
    rk, rv = w.recent_window(12, rl, seed=2)
    out = _hybrid(w, codec, kp, vp, rk, rv, rl).astype(np.float64)
    q = w.queries().astype(np.float64)
    G = w.num_q_heads // w.num_kv_heads
    np.testing.assert_allclose(out[0], _sdpa(q[0], rk[0, :9].astype(np.float64), rv[0, :9].astype(np.float64), G),
                               rtol=1e-6, atol=1e-6)
    assert not out[1].any()  # no token at all
    # a single token: its value, for every query head of its KV head
    np.testing.assert_allclose(out[2], np.repeat(rv[2, 0].astype(np.float64), G, axis=0), rtol=1e-6)


def test_empty_window_is_the_packed_decode():
    w = _small()
    codec, kp, vp = _setup(w)
    rl = np.zeros(w.batch, dtype=np.int64)
    rk, rv = w.recent_window(4, rl, seed=3)
    out = _hybrid(w, codec, kp, vp, rk, rv, rl)
    ref = oracle.paged_decode(w.queries(), kp, vp, w.block_table, w.seq_lens, w.k_bits, w.v_bits, codec.signs,
                              codec.centroids32(w.k_bits), codec.centroids32(w.v_bits))
    np.testing.assert_allclose(out, ref, rtol=1e-6, atol=1e-7)


def test_moving_the_last_tokens_into_the_window_changes_nothing():
    # the last R tokens of each sequence, reconstructed, as an exact window:
    # same context, same output (the split point between the parts is free)
    w = _small(seq_lens=[40, 17, 33])
    codec, kp, vp = _setup(w)
    R = np.array([8, 17, 1])
    short = w.seq_lens - R
    cap = int(R.max())
    rk = np.zeros((w.batch, cap, w.num_kv_heads, 128))
    rv = np.zeros_like(rk)
    for b in range(w.batch):
        t = np.arange(short[b], w.seq_lens[b])
        blk = w.block_table[b, t // 16]
        rk[b, :R[b]] = codec.dequantize(kp[blk, t % 16], w.k_bits)
        rv[b, :R[b]] = codec.dequantize(vp[blk, t % 16], w.v_bits)
    a = _hybrid(w, codec, kp, vp, rk, rv, R, lens=short)
    ref = oracle.paged_decode(w.queries(), kp, vp, w.block_table, w.seq_lens, w.k_bits, w.v_bits, codec.signs,
                              codec.centroids32(w.k_bits), codec.centroids32(w.v_bits))
    np.testing.assert_allclose(a, ref, rtol=1e-6, atol=1e-7)


def test_rows_past_the_window_length_are_ignored_and_a_dominant_token_wins():
    w = _small(seq_lens=[30, 5])
    codec, kp, vp = _setup(w)
    rl = np.array([3, 2])
    rk, rv = w.recent_window(6, rl, seed=4)
    base = _hybrid(w, codec, kp, vp, rk, rv, rl)
    rk2, rv2 = rk.copy(), rv.copy()
    rk2[:, 3:] = 100
    rv2[:, 3:] = -100
    assert np.array_equal(base, _hybrid(w, codec, kp, vp, rk2, rv2, rl))
    # a window key equal to 40x the query dominates the softmax: the output is its value
    q = w.queries().astype(np.float32)
    rk3 = rk.astype(np.float32).copy()
    rk3[0, 1, 0] = 40 * q[0, 0]  # KV head 0, query head 0
    out = _hybrid(w, codec, kp, vp, rk3, rv.astype(np.float32), rl, q=q)
    np.testing.assert_allclose(out[0, 0], rv[0, 1, 0].astype(np.float32), rtol=1e-6, atol=1e-6)
