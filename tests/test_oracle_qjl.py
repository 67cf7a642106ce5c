"""Pins for the oracle's prod key codec (MSE indices + QJL residual sketch), CPU only.

References: closed forms for hand-built rows (a zero residual; an identity
sketch matrix), the layout, and the statistics the published estimator
guarantees: over independent Gaussian sketch matrices its mean is the exact
inner product and its variance stays under pi / (2 d) n^2 gamma^2 ||y||^2.
"""

import math
import struct

import numpy as np
import pytest

import oracle
from oracle.rht import rht
from paged_decode_attention_tq_amd import workloads


def _row(idx, norm, z, gamma, bits):
    return oracle.prod_rows_to_bytes(np.asarray(idx, np.uint8), np.float32(norm), np.asarray(z, bool),
                                     np.float32(gamma), bits)


def test_layout_and_round_trip():
    d = 128
    assert [oracle.prod_row_bytes(d, b) for b in (2, 3, 4, 5)] == [40, 56, 72, 88]
    rng = np.random.default_rng(1)
    idx = rng.integers(0, 8, size=d).astype(np.uint8)
    z = rng.integers(0, 2, size=d).astype(bool)
    row = _row(idx, 2.5, z, 0.125, 4)
    assert row.shape == (72,)
    assert row[48:52].tobytes() == struct.pack("<f", 2.5)
    assert row[68:72].tobytes() == struct.pack("<f", 0.125)
    assert row[52] & 1 == z[0] and (row[52] >> 1) & 1 == z[1] and (row[67] >> 7) & 1 == z[127]
    i2, n2, z2, g2 = oracle.prod_bytes_to_rows(row, 4, d)
    assert np.array_equal(i2, idx) and n2 == np.float32(2.5) and np.array_equal(z2, z) and g2 == np.float32(0.125)


def test_closed_forms_zero_residual_and_identity_sketch():
    d, bits = 128, 4
    signs = oracle.rht_signs(42, d)
    c = oracle.beta_codebook(d, bits - 1)[1].astype(np.float64)
    rng = np.random.default_rng(2)
    y = rng.standard_normal(d)
    yr = rht(y, signs)
    idx = rng.integers(0, 8, size=d).astype(np.uint8)
    z = rng.integers(0, 2, size=d).astype(bool)
    S = rng.standard_normal((d, d))
    # gamma 0: the QJL term vanishes, the estimate is the MSE inner product
    est = oracle.prod_scores(y, _row(idx, 3.0, z, 0.0, bits)[None], bits, signs, S)[0]
    assert math.isclose(est, 3.0 * float(c[idx] @ yr), rel_tol=1e-12, abs_tol=1e-12)
    # S = I, every sign +1: the QJL term is gamma sqrt(pi / 2) / d * sum(y~)
    est = oracle.prod_scores(y, _row(idx, 3.0, np.ones(d, bool), 0.5, bits)[None], bits, signs, np.eye(d))[0]
    want = 3.0 * (float(c[idx] @ yr) + 0.5 * math.sqrt(math.pi / 2) / d * float(yr.sum()))
    assert math.isclose(est, want, rel_tol=1e-12)


def test_encoding_signs_follow_the_sketch_of_the_residual():
    d, bits = 128, 3
    signs = oracle.rht_signs(42, d)
    S = workloads.qjl_matrix(d, seed=3)
    x = np.random.default_rng(4).standard_normal((16, d)).astype(np.float16)
    idx, n32, z, g32, _, _ = oracle.encode_prod(x, bits, signs, S)
    x64 = x.astype(np.float64)
    n = np.sqrt(np.sum(x64 * x64, axis=1))
    r = rht(x64 / n[:, None], signs)
    e = r - oracle.beta_codebook(d, bits - 1)[1].astype(np.float64)[idx.astype(np.int64)]
    np.testing.assert_allclose(g32, np.linalg.norm(e, axis=1), rtol=1e-6)
    assert np.array_equal(z, (e @ S.T.astype(np.float64)) >= 0)
    # the MSE part is the (b-1)-bit codec's
    assert np.array_equal(idx, oracle.OracleCodec(d, 42).encode(x, bits - 1)[0])


@pytest.mark.parametrize("bits", [2, 4])
def test_estimator_is_unbiased_with_the_stated_variance(bits):
    d, trials = 128, 3000
    signs = oracle.rht_signs(42, d)
    rng = np.random.default_rng(10 + bits)
    x = rng.standard_normal((1, d)).astype(np.float32)
    y = rng.standard_normal(d)
    true = float(x[0].astype(np.float64) @ y)
    est = np.empty(trials)
    gamma = n = None
    for k in range(trials):
        S = rng.standard_normal((d, d))
        idx, n32, z, g32, _, _ = oracle.encode_prod(x, bits, signs, S)
        est[k] = oracle.prod_scores(y, oracle.prod_rows_to_bytes(idx, n32, z, g32, bits), bits, signs, S)[0]
        gamma, n = float(g32[0]), float(n32[0])
    se = est.std() / math.sqrt(trials)
    assert abs(est.mean() - true) < 5 * se + 1e-6 * abs(true), (est.mean(), true, se)
    bound = math.pi / (2 * d) * n * n * gamma * gamma * float(y @ y)
    assert est.var() <= 1.15 * bound, (est.var(), bound)
