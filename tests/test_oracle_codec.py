"""Pins for the oracle's row codec and paged row writer (CPU only)."""

import json
import math
import struct
from fractions import Fraction

import numpy as np
import pytest
from scipy import integrate

import oracle
from oracle.codebook import beta_pdf
from paged_decode_attention_tq_amd import workloads
from tests.conftest import golden_path


def _sylvester(d):
    H = np.array([[1.0]])
    while H.shape[0] < d:
        H = np.kron(np.array([[1.0, 1.0], [1.0, -1.0]]), H)
    return H


def test_row_bytes_match_the_layout_table():
    with open(golden_path("row_bytes_layout.json")) as fh:
        g = json.load(fh)
    d = g["head_dim"]
    for row in g["table"]:
        assert oracle.index_bytes(d, row["bits"]) == row["index_bytes"]
        assert oracle.row_bytes(d, row["bits"]) == row["row_bytes"]
    assert oracle.row_bytes(d, 4) + oracle.row_bytes(d, 2) == g["k4_v2_token_head_bytes"]
    ex = g["page_shape_example"]
    codec = oracle.OracleCodec(128, 42)
    raw = np.random.default_rng(1).standard_normal((ex["tokens"], ex["num_kv_heads"], 128)).astype(np.float32)
    pages = np.zeros((ex["num_blocks"], ex["block_size"], ex["num_kv_heads"], ex["row_bytes"]), np.uint8)
    out, _ = codec.write_kv(raw, pages, np.arange(ex["tokens"]), 4)
    assert out.shape == pages.shape


def test_pack_worked_examples():
    with open(golden_path("pack_worked_examples.json")) as fh:
        g = json.load(fh)
    for ex in g["examples"]:
        idx = np.array(ex["indices"])
        got = oracle.pack_indices(idx[None, :], ex["bits"])[0]
        assert got.tobytes().hex() == ex["bytes"], ex
        back = oracle.unpack_indices(got[None, :], ex["bits"], len(idx))[0]
        assert np.array_equal(back, idx)


@pytest.mark.parametrize("bits", [1, 2, 3, 4, 5])
@pytest.mark.parametrize("d", [5, 8, 64, 128, 256])
def test_pack_round_trip_and_zero_padding(bits, d):
    rng = np.random.default_rng(bits * 1000 + d)
    idx = rng.integers(0, 1 << bits, size=(17, d))
    packed = oracle.pack_indices(idx, bits)
    assert packed.shape == (17, (d * bits + 7) // 8)
    assert np.array_equal(oracle.unpack_indices(packed, bits, d), idx)
    # the bit stream in order equals the concatenated LSB-first index bits
    stream = np.unpackbits(packed, axis=1, bitorder="little")
    want = ((idx[:, :, None] >> np.arange(bits)) & 1).reshape(17, -1)
    assert np.array_equal(stream[:, : d * bits], want)
    assert not stream[:, d * bits :].any()


def _exact_norm32(row):
    # float32( sqrt( float64( exact sum of squares ) ) ) with Fraction arithmetic
    s = sum(Fraction(float(v)) ** 2 for v in row)
    return np.float32(math.sqrt(float(s)))


@pytest.mark.parametrize("dtype", [np.float16, np.float32])
def test_norm_bytes(dtype):
    codec = oracle.OracleCodec(128, 42)
    rng = np.random.default_rng(5)
    x = (rng.standard_normal((40, 128)) * np.exp(rng.standard_normal((40, 1)))).astype(dtype)
    x[3, :] = 0
    x[4, :7] = dtype(1e-4)  # tiny values
    rows, _ = codec.encode_bytes(x, 4)
    for i in range(len(x)):
        assert rows[i, -4:].tobytes() == struct.pack("<f", float(_exact_norm32(x[i]))), i


@pytest.mark.parametrize("bits", [1, 2, 3, 4, 5])
def test_zero_row(bits):
    codec = oracle.OracleCodec(128, 42)
    idx, norm32, r, _ = codec.encode(np.zeros((1, 128), np.float32), bits)
    assert norm32[0] == 0 and not r.any()
    # r = 0 sits on the middle boundary 0; a tie goes to the lower index
    assert np.all(idx == (1 << (bits - 1)) - 1)


@pytest.mark.parametrize("bits", [2, 3, 4, 5])
def test_indices_are_nearest_centroids_of_the_rotated_unit_vector(bits):
    d = 128
    codec = oracle.OracleCodec(d, 42)
    rng = np.random.default_rng(bits)
    x = rng.standard_normal((64, d)).astype(np.float16)
    idx, norm32, r, near = codec.encode(x, bits)
    # independent rotation: dense Sylvester matrix times the signed unit vector
    x64 = x.astype(np.float64)
    u = x64 / np.linalg.norm(x64, axis=1, keepdims=True)
    r_ref = (u * codec.signs) @ _sylvester(d).T / np.sqrt(d)
    np.testing.assert_allclose(r, r_ref, atol=1e-14)
    c32 = codec.centroids32(bits).astype(np.float64)
    nearest = np.argmin(np.abs(r_ref[..., None] - c32), axis=-1)
    assert np.array_equal(idx[~near], nearest[~near])


@pytest.mark.parametrize("bits", [2, 3, 4])
def test_sign_symmetry_and_scale_invariance(bits):
    codec = oracle.OracleCodec(128, 42)
    x = np.random.default_rng(11).standard_normal((50, 128)).astype(np.float32)
    idx, n, _, near = codec.encode(x, bits)
    idx_neg, n_neg, _, _ = codec.encode(-x, bits)
    assert np.array_equal(n, n_neg)
    top = (1 << bits) - 1
    assert np.array_equal(idx_neg[~near], top - idx[~near])
    idx2, n2, _, _ = codec.encode(x * np.float32(4), bits)
    assert np.array_equal(idx2, idx) and np.array_equal(n2, n * np.float32(4))


@pytest.mark.parametrize("bits", [2, 3, 4])
def test_distortion_matches_the_codebook(bits):
    # The rotated unit vector's coordinates follow the Beta law, so the mean
    # squared reconstruction error of the unit vector equals d * MSE(codebook).
    d = 128
    codec = oracle.OracleCodec(d, 42)
    x = np.random.default_rng(100 + bits).standard_normal((4000, d)).astype(np.float32)
    rows, _ = codec.encode_bytes(x, bits)
    xhat = codec.dequantize(rows, bits)
    x64 = x.astype(np.float64)
    n = np.linalg.norm(x64, axis=1, keepdims=True)
    err = np.sum((xhat / n - x64 / n) ** 2, axis=1)
    c64, c32, t64 = codec.codebook(bits)
    e = np.concatenate([[-1.0], t64, [1.0]])
    mse = sum(
        integrate.quad(lambda v: (v - float(c32[j])) ** 2 * float(beta_pdf(np.array(v), d)), e[j], e[j + 1])[0]
        for j in range(len(c32))
    )
    se = err.std() / math.sqrt(len(err))
    assert abs(err.mean() - d * mse) < 4 * se, (err.mean(), d * mse, se)


def test_dequantize_is_norm_times_inverse_rotation():
    d = 128
    codec = oracle.OracleCodec(d, 42)
    x = np.random.default_rng(3).standard_normal((8, d)).astype(np.float16)
    rows, _ = codec.encode_bytes(x, 4)
    idx, norm = oracle.bytes_to_rows(rows, 4, d)
    c = codec.centroids32(4).astype(np.float64)[idx]
    R = _sylvester(d) * codec.signs[None, :] / np.sqrt(d)
    np.testing.assert_allclose(codec.dequantize(rows, 4), norm[:, None].astype(np.float64) * (c @ R), atol=1e-13)


def test_write_kv_slot_semantics():
    d, BS, Hkv, NB, bits = 128, 4, 2, 3, 3
    codec = oracle.OracleCodec(d, 42)
    RB = oracle.row_bytes(d, bits)
    rng = np.random.default_rng(9)
    raw = rng.standard_normal((6, Hkv, d)).astype(np.float16)
    pages = rng.integers(0, 256, size=(NB, BS, Hkv, RB), dtype=np.uint8)
    slots = np.array([0, 5, -1, 11, -7, 6])
    out, near = codec.write_kv(raw, pages, slots, bits)
    rows, _ = codec.encode_bytes(raw, bits)
    written = np.zeros((NB, BS), bool)
    for n, s in enumerate(slots):
        if s >= 0:
            assert np.array_equal(out[s // BS, s % BS], rows[n])
            written[s // BS, s % BS] = True
    assert np.array_equal(out[~written], pages[~written])  # negative slots touch nothing
    with pytest.raises(IndexError):
        codec.write_kv(raw, pages, np.array([0, 1, 2, NB * BS, 3, 4]), bits)


def test_identity_block_table_placement_on_the_tiny_workload():
    w = workloads.preset("tiny")
    assert w.block_table.tolist() == [[0, 1, 2, 3]] and w.num_blocks == 4
    codec = oracle.OracleCodec(w.head_dim, w.rht_seed)
    raw = w.rows("k")
    out, _ = codec.write_kv(raw, w.zero_pages(4), w.slots, 4)
    rows, _ = codec.encode_bytes(raw, 4)
    for t in range(64):
        assert np.array_equal(out[t // 16, t % 16], rows[t])
