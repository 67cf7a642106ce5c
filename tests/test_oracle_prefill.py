"""Pins for the oracle's multi-query (prefill / verify chunk) attention, CPU only.

References: torch's scaled_dot_product_attention on the CPU in float64 with
an explicit causal mask over the densely reconstructed rows; the reduction
of each query to a single-query decode over the tokens it may see; the
one-query case.
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


def _small(**kw):
    base = dict(head_dim=128, k_bits=4, v_bits=3, num_q_heads=8, num_kv_heads=2,
                block_size=16, seq_lens=[37, 5, 64, 20], seed=21, extra_blocks=2)
    base.update(kw)
    return workloads.make_workload("pre", **base)


def _queries(w, Lq, seed):
    return np.random.default_rng(seed).standard_normal((w.batch, Lq, w.num_q_heads, 128)).astype(np.float16)


def _run(w, codec, kp, vp, q, ql, lens=None):
    return oracle.paged_prefill(q, ql, kp, vp, w.block_table, w.seq_lens if lens is None else lens, w.k_bits,
                                w.v_bits, codec.signs, codec.centroids32(w.k_bits), codec.centroids32(w.v_bits))


def test_matches_causal_sdpa():
    w = _small()
    codec, kp, vp = _setup(w)
    Lq = 6
    ql = np.array([6, 5, 1, 4])
    q = _queries(w, Lq, 1)
    out = _run(w, codec, kp, vp, q, ql).astype(np.float64)
    G = w.num_q_heads // w.num_kv_heads
    for b in range(w.batch):
        L, n = int(w.seq_lens[b]), int(ql[b])
        t = np.arange(L)
        blk = w.block_table[b, t // 16]
        K = torch.from_numpy(codec.dequantize(kp[blk, t % 16], w.k_bits)).permute(1, 0, 2).repeat_interleave(G, 0)
        V = torch.from_numpy(codec.dequantize(vp[blk, t % 16], w.v_bits)).permute(1, 0, 2).repeat_interleave(G, 0)
        qq = torch.from_numpy(q[b, :n].astype(np.float64)).permute(1, 0, 2)  # [Hq, n, d]
        pos = L - n + np.arange(n)
        mask = torch.from_numpy(np.arange(L)[None, :] <= pos[:, None])  # [n, L], True = may attend
        ref = torch.nn.functional.scaled_dot_product_attention(qq, K, V, attn_mask=mask)  # [Hq, n, d]
        np.testing.assert_allclose(out[b, :n], ref.permute(1, 0, 2).numpy(), rtol=1e-6, atol=1e-6)
        assert not out[b, n:].any()


def test_each_query_is_a_decode_over_the_tokens_it_sees():
    w = _small(seq_lens=[40, 17])
    codec, kp, vp = _setup(w)
    Lq = 3
    ql = np.array([3, 2])
    q = _queries(w, Lq, 2)
    out = _run(w, codec, kp, vp, q, ql)
    for j in range(Lq):
        lens = np.maximum(w.seq_lens - ql + j + 1, 0).astype(np.int32)
        ref = oracle.paged_decode(np.ascontiguousarray(q[:, j]), kp, vp, w.block_table, lens, w.k_bits, w.v_bits,
                                  codec.signs, codec.centroids32(w.k_bits), codec.centroids32(w.v_bits))
        for b in range(w.batch):
            if j < ql[b]:
                np.testing.assert_allclose(out[b, j], ref[b], rtol=1e-6, atol=1e-7)


def test_one_query_is_the_decode_and_bad_lengths_raise():
    w = _small()
    codec, kp, vp = _setup(w)
    q = _queries(w, 1, 3)
    out = _run(w, codec, kp, vp, q, np.ones(w.batch, dtype=np.int64))
    ref = oracle.paged_decode(np.ascontiguousarray(q[:, 0]), kp, vp, w.block_table, w.seq_lens, w.k_bits, w.v_bits,
                              codec.signs, codec.centroids32(w.k_bits), codec.centroids32(w.v_bits))
    np.testing.assert_allclose(out[:, 0], ref, rtol=1e-6, atol=1e-7)
    with pytest.raises(ValueError):
        _run(w, codec, kp, vp, _queries(w, 6, 4), np.array([6, 6, 1, 1]))  # 6 queries on a 5-token sequence
