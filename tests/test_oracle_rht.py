"""Pins for the oracle's seeded randomized Hadamard transform (CPU only)."""

import json

import numpy as np
import pytest

import oracle
from tests.conftest import golden_path


def test_splitmix64_published_outputs():
    with open(golden_path("splitmix64_vectors.json")) as fh:
        g = json.load(fh)
    for v in g["vectors"]:
        want = [int(o, 0) for o in v["outputs"]]
        assert oracle.splitmix64(v["seed"], len(want)) == want


def test_signs_are_bit_63_of_the_published_outputs():
    # the sign rule is pinned to the published generator outputs themselves
    # (not to the oracle's own SplitMix64): s_i = -1 exactly when bit 63 of
    # the i-th output is set; the vectors hold both signs
    with open(golden_path("splitmix64_vectors.json")) as fh:
        g = json.load(fh)
    seen = set()
    for v in g["vectors"]:
        outs = [int(o, 0) for o in v["outputs"]]
        want = np.array([-1 if (o >> 63) & 1 else 1 for o in outs], dtype=np.int8)
        assert np.array_equal(oracle.rht_signs(v["seed"], len(outs)), want)
        seen.update(want.tolist())
    assert seen == {-1, 1}


def test_signs_are_top_bits_and_balanced():
    s = oracle.rht_signs(42, 4096)
    assert set(np.unique(s)) == {-1, 1}
    # top bit of a well-mixed 64-bit output is a fair coin
    assert abs(int(s.sum())) < 4 * np.sqrt(4096)
    assert not np.array_equal(oracle.rht_signs(42, 128), oracle.rht_signs(43, 128))


def _sylvester_kron(d):
    H = np.array([[1.0]])
    H2 = np.array([[1.0, 1.0], [1.0, -1.0]])
    while H.shape[0] < d:
        H = np.kron(H2, H)
    return H


def test_two_point_butterfly_by_hand():
    np.testing.assert_array_equal(oracle.fwht(np.array([3.0, 5.0])), [8.0, -2.0])


@pytest.mark.parametrize("d", [1, 2, 4, 8, 16, 32, 64, 128, 256])
def test_fwht_is_the_sylvester_matrix(d):
    H = _sylvester_kron(d)
    np.testing.assert_array_equal(oracle.fwht(np.eye(d)), H.T)
    i = np.arange(d)
    pop = np.vectorize(lambda v: bin(v).count("1"))(i[:, None] & i[None, :])
    np.testing.assert_array_equal(H, (-1.0) ** pop)


@pytest.mark.parametrize("d", [64, 128, 256])
def test_rht_is_orthonormal_and_inverted_by_irht(d):
    s = oracle.rht_signs(42, d)
    R = oracle.rht(np.eye(d), s).T  # column j = rht(e_j)
    np.testing.assert_allclose(R @ R.T, np.eye(d), atol=1e-13)
    np.testing.assert_allclose(np.abs(R), 1.0 / np.sqrt(d), rtol=1e-14)
    # R = H D / sqrt(d), D = diag(s)
    np.testing.assert_allclose(R, _sylvester_kron(d) * s[None, :] / np.sqrt(d), atol=1e-15)
    x = np.random.default_rng(0).standard_normal((5, d))
    y = oracle.rht(x, s)
    np.testing.assert_allclose(oracle.irht(y, s), x, atol=1e-13)
    np.testing.assert_allclose(np.linalg.norm(y, axis=1), np.linalg.norm(x, axis=1), rtol=1e-14)
    Ri = oracle.irht(np.eye(d), s).T
    np.testing.assert_allclose(Ri, R.T, atol=1e-15)
