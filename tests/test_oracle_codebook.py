"""Pins for the oracle's Lloyd-Max codebook (CPU only).

Each check is independent of the code it tests: closed forms of the law,
an independent quadrature (scipy.integrate.quad) of the Lloyd-Max
conditions, the Beta law from scipy.stats, and Max's 1960 table for the
generic iteration.
"""

import json
import math

import mpmath
import numpy as np
import pytest
from scipy import integrate, special, stats

import oracle
from oracle.codebook import beta_pdf, beta_cell_mass, gaussian_lloyd_max
from tests.conftest import golden_path


@pytest.mark.parametrize("bits", [1, 2, 3, 4, 5])
def test_uniform_law_closed_form(bits):
    # d = 3: the coordinate of a uniform point on S^2 is uniform on [-1, 1]
    # (Archimedes), whose Lloyd-Max quantiser is the uniform one.
    c64, c32, t64 = oracle.beta_codebook(3, bits)
    n = 1 << bits
    want = -1.0 + (2 * np.arange(n) + 1) / n
    np.testing.assert_allclose(c64, want, atol=1e-14, rtol=0)
    assert np.array_equal(c32, want.astype(np.float32))
    np.testing.assert_allclose(t64, -1.0 + 2 * np.arange(1, n) / n, atol=1e-14, rtol=0)


@pytest.mark.parametrize("d", [4, 16, 64, 128, 256])
def test_one_bit_closed_form(d):
    # 1 bit: cells are the two half-lines, centroids +-E|X|,
    # E|X| = Gamma(d/2) / (sqrt(pi) Gamma((d+1)/2)).
    c64, _, t64 = oracle.beta_codebook(d, 1)
    with mpmath.workdps(30):
        e_abs = float(mpmath.gamma(mpmath.mpf(d) / 2) / (mpmath.sqrt(mpmath.pi) * mpmath.gamma(mpmath.mpf(d + 1) / 2)))
    np.testing.assert_allclose(c64, [-e_abs, e_abs], rtol=2e-16)
    assert t64[0] == 0.0


@pytest.mark.parametrize("d", [16, 128])
def test_density_is_the_beta_law(d):
    x = np.linspace(-0.999, 0.999, 101)
    a = (d - 1) / 2
    ref = stats.beta.pdf((x + 1) / 2, a, a) / 2
    np.testing.assert_allclose(beta_pdf(x, d), ref, rtol=1e-11, atol=1e-13 * ref.max())
    total, _ = integrate.quad(lambda v: beta_pdf(np.array(v), d), -1, 1, epsabs=1e-14, epsrel=1e-13)
    assert abs(total - 1.0) < 1e-12


@pytest.mark.parametrize("bits", [2, 3, 4, 5])
def test_lloyd_max_conditions_by_quadrature(bits):
    d = 128
    c64, c32, t64 = oracle.beta_codebook(d, bits)
    n = 1 << bits
    mid = 0.5 * (c64[1:] + c64[:-1])
    edges = np.concatenate([[-1.0], mid, [1.0]])
    f = lambda v: float(beta_pdf(np.array(v), d))
    for j in range(n):
        a, b = edges[j], edges[j + 1]
        mass, _ = integrate.quad(f, a, b, epsabs=0, epsrel=1e-13, limit=200)
        mom, _ = integrate.quad(lambda v: v * f(v), a, b, epsabs=0, epsrel=1e-13, limit=200)
        assert abs(mom / mass - c64[j]) < 1e-12, (j, mom / mass, c64[j])
    # boundaries are midpoints of the float32 centroids, exactly
    assert np.array_equal(t64, (c32[1:].astype(np.float64) + c32[:-1].astype(np.float64)) / 2)


@pytest.mark.parametrize("bits", [1, 2, 3, 4, 5])
def test_symmetry_order_and_rounding(bits):
    c64, c32, t64 = oracle.beta_codebook(128, bits)
    assert np.all(np.diff(c64) > 0) and np.all(np.diff(c32) > 0)
    assert np.array_equal(c32, -c32[::-1])
    assert t64[len(t64) // 2] == 0.0
    # float32 centroids are the nearest float32 values of the float64 ones
    for v64, v32 in zip(c64, c32):
        lo = np.nextafter(v32, np.float32(-1))
        hi = np.nextafter(v32, np.float32(1))
        assert abs(float(v32) - v64) <= min(abs(float(lo) - v64), abs(float(hi) - v64))


def test_cell_masses_sum_to_one():
    for bits in (2, 4, 5):
        c64, _, _ = oracle.beta_codebook(128, bits)
        mid = 0.5 * (c64[1:] + c64[:-1])
        e = np.concatenate([[-1.0], mid, [1.0]])
        assert abs(beta_cell_mass(e[:-1], e[1:], 128).sum() - 1.0) < 1e-14


def test_generic_iteration_reproduces_max_1960():
    with open(golden_path("max1960_gaussian.json")) as fh:
        g = json.load(fh)
    tol = g["tolerance"]
    for n_str, levels in g["levels"].items():
        bits = int(math.log2(int(n_str)))
        c = gaussian_lloyd_max(bits)
        pos = c[len(c) // 2 :]
        np.testing.assert_allclose(pos, levels, atol=tol, rtol=0)
        # its distortion, by quadrature over the cells
        edges = np.concatenate([[-np.inf], 0.5 * (c[1:] + c[:-1]), [np.inf]])
        mse = sum(
            integrate.quad(lambda x: (x - c[j]) ** 2 * stats.norm.pdf(x), edges[j], edges[j + 1])[0]
            for j in range(len(c))
        )
        assert abs(mse - g["mse"][n_str]) / g["mse"][n_str] < 2e-3


@pytest.mark.parametrize("bits", [2, 3, 4])
def test_high_dimension_limit_is_gaussian(bits):
    # sqrt(d) X converges in law to N(0, 1); the codebooks follow at rate O(1/d).
    g = gaussian_lloyd_max(bits)
    prev = None
    for d in (256, 1024, 4096):
        c64, _, _ = oracle.beta_codebook(d, bits)
        err = np.max(np.abs(math.sqrt(d) * c64 - g))
        if prev is not None:
            assert err < prev / 3  # shrinks ~4x per 4x in d
        prev = err
    assert prev < 2e-3


def test_distortion_falls_with_bits_and_sits_below_gaussian():
    d = 128
    prev = np.inf
    for bits in (1, 2, 3, 4, 5):
        c64, _, _ = oracle.beta_codebook(d, bits)
        e = np.concatenate([[-1.0], 0.5 * (c64[1:] + c64[:-1]), [1.0]])
        mse = sum(
            integrate.quad(lambda x: (x - c64[j]) ** 2 * float(beta_pdf(np.array(x), d)), e[j], e[j + 1])[0]
            for j in range(len(c64))
        )
        assert mse < prev
        prev = mse
        gauss = gaussian_lloyd_max(bits)
        ge = np.concatenate([[-np.inf], 0.5 * (gauss[1:] + gauss[:-1]), [np.inf]])
        gmse = sum(
            integrate.quad(lambda x: (x - gauss[j]) ** 2 * stats.norm.pdf(x), ge[j], ge[j + 1])[0]
            for j in range(len(gauss))
        )
        # the sphere's law has lighter tails than the Gaussian limit
        assert d * mse < gmse
