"""Pins for the oracle's dense readback of pages (``oracle.decompress_kv``), CPU only.

The expected rows come from closed forms, not from the oracle's own
transform: when the indices of a row follow the sign pattern of Hadamard
row k over a symmetric pair of centroids (c_j and c_{2^b-1-j} = -c_j), the
reconstruction n * s * H c / sqrt(d) is a single spike n * s_k * c_j * sqrt(d)
at coordinate k, because H H = d I.
"""

import struct

import numpy as np
import pytest

import oracle


def _hadamard_pattern(d, k, j, bits):
    top = (1 << bits) - 1
    par = np.array([bin(i & k).count("1") & 1 for i in range(d)])
    return np.where(par == 0, j, top - j).astype(np.uint8)


def _row(idx, norm, bits):
    return np.concatenate([oracle.pack_indices(idx, bits), np.frombuffer(struct.pack("<f", norm), np.uint8)])


@pytest.mark.parametrize("bits,k,j", [(2, 0, 3), (2, 127, 0), (3, 5, 6), (4, 64, 1), (4, 1, 9), (5, 77, 30)])
def test_hadamard_row_pattern_reconstructs_a_single_spike(bits, k, j):
    d = 128
    codec = oracle.OracleCodec(d, 42)
    c32 = codec.centroids32(bits)
    top = (1 << bits) - 1
    assert c32[top - j] == -c32[j]  # the symmetric codebook this pin relies on
    norm = 2.5
    pages = np.zeros((2, 16, 1, oracle.row_bytes(d, bits)), dtype=np.uint8)
    pages[1, 3, 0] = _row(_hadamard_pattern(d, k, j, bits), norm, bits)
    out = codec.decompress_kv(pages, np.array([19], dtype=np.int64), bits)
    want = np.zeros(d)
    want[k] = norm * float(codec.signs[k]) * float(c32[j]) * np.sqrt(d)
    np.testing.assert_allclose(out[0, 0], want, atol=1e-13)


def test_slots_select_page_offset_and_head():
    d, bits, NB, BS, Hkv = 128, 4, 3, 16, 2
    codec = oracle.OracleCodec(d, 42)
    c32 = codec.centroids32(bits)
    RB = oracle.row_bytes(d, bits)
    pages = np.zeros((NB, BS, Hkv, RB), dtype=np.uint8)
    pat = _hadamard_pattern(d, 0, 15, bits)  # spike at coordinate 0
    for p in range(NB):
        for t in range(BS):
            for h in range(Hkv):
                pages[p, t, h] = _row(pat, float(1 + p * 100 + t * 2 + h), bits)
    slots = np.array([5, -1, 47, 16, -7, 0], dtype=np.int64)
    out = codec.decompress_kv(pages, slots, bits)
    assert out.shape == (6, Hkv, d)
    amp = float(codec.signs[0]) * float(c32[15]) * np.sqrt(d)
    for n, s in enumerate(slots):
        for h in range(Hkv):
            want = np.zeros(d)
            if s >= 0:
                p, t = divmod(int(s), BS)
                want[0] = (1 + p * 100 + t * 2 + h) * amp
            np.testing.assert_allclose(out[n, h], want, rtol=1e-14, atol=0)


def test_out_of_range_slot_raises_and_empty_read():
    d, bits = 128, 3
    codec = oracle.OracleCodec(d, 42)
    pages = np.zeros((2, 16, 1, oracle.row_bytes(d, bits)), dtype=np.uint8)
    with pytest.raises(IndexError):
        codec.decompress_kv(pages, np.array([0, 32], dtype=np.int64), bits)
    assert codec.decompress_kv(pages, np.zeros(0, dtype=np.int64), bits).shape == (0, 1, d)
    # all-zero bytes: norm 0, so the row reconstructs to zeros
    assert not np.any(codec.decompress_kv(pages, np.array([31], dtype=np.int64), bits))


def test_written_rows_read_back_within_the_codebook_distortion():
    # end to end through the oracle writer: ||x - xhat||^2 / ||x||^2 stays near
    # d * MSE of the 4-bit codebook (about 0.0095) and far below 1
    d, bits = 128, 4
    codec = oracle.OracleCodec(d, 42)
    x = np.random.default_rng(9).standard_normal((64, 2, d)).astype(np.float16)
    slots = np.random.default_rng(10).permutation(64).astype(np.int64)
    pages, _ = codec.write_kv(x, np.zeros((4, 16, 2, oracle.row_bytes(d, bits)), np.uint8), slots, bits)
    xh = codec.decompress_kv(pages, slots, bits)
    x64 = x.astype(np.float64)
    rel = np.sum((xh - x64) ** 2, axis=-1) / np.sum(x64 ** 2, axis=-1)
    assert 0.005 < rel.mean() < 0.015 and rel.max() < 0.05
