"""Seeded workload generators: shapes, slot maps and determinism (CPU only)."""

import numpy as np
import pytest

from paged_decode_attention_tq_amd import workloads


@pytest.mark.parametrize(
    "name,B,L,Hq,Hkv,kb,vb,NB",
    [
        ("tiny", 1, 64, 2, 1, 4, 4, 4),
        ("pages_geometry", 32, 2048, 16, 2, 4, 4, 4096),
        ("mixed_bits", 64, 8192, 32, 8, 4, 2, 32768),
        ("long_context", 8, 131072, 64, 8, 4, 4, 65536),
    ],
)
def test_fixed_length_presets(name, B, L, Hq, Hkv, kb, vb, NB):
    w = workloads.preset(name)
    assert (w.batch, w.num_q_heads, w.num_kv_heads, w.k_bits, w.v_bits, w.num_blocks) == (B, Hq, Hkv, kb, vb, NB)
    assert np.all(w.seq_lens == L) and w.block_table.shape == (B, L // 16)
    # every page used exactly once
    assert np.array_equal(np.sort(w.block_table.ravel()), np.arange(NB))
    assert np.all(w.slots >= 0) and len(np.unique(w.slots)) == w.num_tokens


def test_long_context_packed_bytes():
    w = workloads.preset("long_context")
    assert w.packed_kv_bytes() == 1_140_850_688


def test_ragged_preset():
    w = workloads.preset("ragged_write")
    assert w.batch == 256 and w.seed == 7 and (w.k_bits, w.v_bits) == (3, 3)
    assert w.seq_lens.min() >= 1 and w.seq_lens.max() <= 32768
    npages = (w.seq_lens + 15) // 16
    assert w.num_blocks == npages.sum()
    assert w.block_table.shape == (256, npages.max())
    used = np.concatenate([w.block_table[b, : npages[b]] for b in range(256)])
    assert np.array_equal(np.sort(used), np.arange(w.num_blocks))
    dropped = (w.slots < 0).sum()
    assert dropped == round(0.1 * w.num_tokens)
    valid = w.slots[w.slots >= 0]
    assert len(np.unique(valid)) == len(valid) and valid.max() < w.num_blocks * 16


def test_slots_follow_the_block_table():
    w = workloads.make_workload("t", num_q_heads=4, num_kv_heads=2, seq_lens=[3, 33, 17], seed=1)
    cu = w.cu_seqlens
    for b in range(w.batch):
        for t in range(int(w.seq_lens[b])):
            assert w.slots[cu[b] + t] == w.block_table[b, t // 16] * 16 + t % 16


def test_rows_are_deterministic_and_per_sequence():
    w = workloads.make_workload("t", num_q_heads=4, num_kv_heads=2, seq_lens=[5, 9], seed=1,
                                lognormal_sigma=0.5, outlier_frac=0.02)
    a = w.rows("k")
    assert np.array_equal(a, w.rows("k"))
    assert np.array_equal(a[5:], w.seq_rows("k", 1))
    assert not np.array_equal(w.seq_rows("k", 0), w.seq_rows("v", 0)[:5])
    assert a.dtype == np.float16 and w.queries().shape == (2, 4, 128)
    assert w.outliers.shape == (round(0.02 * 2 * 128), 2)


def test_mixed_bits_outlier_count():
    w = workloads.preset("mixed_bits", batch=2, seq_len=32)
    assert w.outliers.shape == (10, 2)
    x = w.seq_rows("k", 0).astype(np.float32)
    ch = np.abs(x).mean(axis=0)  # [Hkv, d]
    big = ch[w.outliers[:, 0], w.outliers[:, 1]]
    assert big.min() > 3 * np.median(ch)


def test_chunked_oracle_helpers_equal_whole_sequence_oracle():
    # the full-size checks run the oracle on 2048-token chunks in threads; the
    # pieces put back together must be the oracle's whole-sequence result
    import oracle
    from tests import oracle_par

    w = workloads.make_workload("chunks", k_bits=3, v_bits=4, num_q_heads=8, num_kv_heads=2,
                                seq_lens=[5000, 37], seed=3, drop_frac=0.1)
    codec = oracle.OracleCodec(128, 42)
    q = w.queries()
    for b in range(w.batch):
        L = int(w.seq_lens[b])
        npg = (L + 15) // 16
        lo = int(w.cu_seqlens[b])
        slots = np.where(w.slots[lo:lo + L] < 0, -1, np.arange(L)).astype(np.int64)
        outs = {}
        for comp, bits in (("k", w.k_bits), ("v", w.v_bits)):
            whole, near = codec.write_kv(w.seq_rows(comp, b), np.zeros((npg, 16, 2, w.row_bytes(bits)), np.uint8),
                                         slots, bits)
            pages, near_c, kept = oracle_par.sequence_pages(codec, w, b, comp, bits)
            assert np.array_equal(pages, whole) and np.array_equal(near_c, near)
            assert kept == int((slots >= 0).sum())
            outs[comp] = whole
        ref = oracle.paged_decode_heads(q[b][None], outs["k"], outs["v"], np.arange(npg, dtype=np.int32)[None],
                                        np.array([L]), w.k_bits, w.v_bits, codec.signs, codec.centroids32(w.k_bits),
                                        codec.centroids32(w.v_bits), [(0, h) for h in range(8)])
        got = oracle_par.sequence_outputs(codec, w, b, outs["k"], outs["v"], q)
        assert np.array_equal(got, ref)
