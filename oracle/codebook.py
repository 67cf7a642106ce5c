"""Lloyd-Max scalar codebook for one coordinate of a rotated unit vector.

Test infrastructure (see ``oracle/__init__.py``).

Source: "vLLM Reference Audit", File Map row "Lloyd-Max codebooks"
(``solve_lloyd_max``, ``LloydMaxCodebook``: centroids and boundaries) and the
Feature Checklist entry "keep exact Beta tests"; "vLLM Usage", "TQ Packed
Page Contract" (``get_codebook_tensors(dim, bits)`` returns the centroids).

Reading taken (the pages give only the names):

* The quantised quantity is one coordinate ``x`` of a unit vector after a
  random rotation, which is modelled as a uniformly distributed point on the
  sphere S^{d-1}.  Its exact law ("exact Beta") is

      f_d(x) = Gamma(d/2) / (sqrt(pi) Gamma((d-1)/2)) * (1 - x^2)^((d-3)/2),

  on |x| <= 1, i.e. (x + 1)/2 ~ Beta((d-1)/2, (d-1)/2).
* The codebook is the 2^b-level Lloyd-Max quantiser of that law: every
  centroid is the conditional mean of its cell, every boundary is the
  midpoint of its two neighbouring centroids.  Lloyd's iteration
  (alternate the two conditions) is run to convergence from the law's
  quantiles; the fixed point is then refined to 40 significant digits by
  Newton's method on the same two conditions (only so that rounding to
  float32 is exact), symmetrised, and rounded to float32.
* Boundaries are the midpoints of the float32 centroids, held in float64
  (exact: the sum of two float32 values and a halving are exact in float64).
"""

from __future__ import annotations

import functools
import math

import mpmath
import numpy as np
from scipy import special

__all__ = [
    "lloyd_max_iterate",
    "beta_pdf",
    "beta_cell_mass",
    "beta_cell_moment",
    "beta_codebook",
    "gaussian_lloyd_max",
]


def lloyd_max_iterate(cell_mass, cell_moment, c0, lo, hi, tol=1e-14, max_iter=100_000):
    """Lloyd's iteration for a 1-D law supported on [lo, hi].

    ``cell_mass(a, b)`` and ``cell_moment(a, b)`` return the probability and
    the first moment of the law over the cells [a_j, b_j] (vectorised).
    Step 1: boundaries = midpoints of the current centroids.  Step 2:
    centroids = moment / mass of each cell.  Stops when no centroid moves by
    more than ``tol``.
    """
    c = np.asarray(c0, dtype=np.float64).copy()
    for _ in range(max_iter):
        t = 0.5 * (c[1:] + c[:-1])
        edges = np.concatenate([[lo], t, [hi]])
        c_new = cell_moment(edges[:-1], edges[1:]) / cell_mass(edges[:-1], edges[1:])
        step = np.max(np.abs(c_new - c))
        c = c_new
        if step <= tol:
            break
    return c


# --- the exact coordinate law of a uniform unit vector in R^d ---------------


def _log_norm_const(d):
    return special.gammaln(d / 2.0) - 0.5 * math.log(math.pi) - special.gammaln((d - 1) / 2.0)


def beta_pdf(x, d):
    """f_d(x) = K (1 - x^2)^((d-3)/2) on |x| <= 1 (0 outside)."""
    x = np.asarray(x, dtype=np.float64)
    m = (d - 3) / 2.0
    inside = np.abs(x) < 1.0
    out = np.zeros_like(x)
    xi = x[inside]
    out[inside] = np.exp(_log_norm_const(d) + m * np.log1p(-xi * xi))
    if m == 0:
        out[np.abs(x) == 1.0] = np.exp(_log_norm_const(d))
    return out


def beta_cell_mass(a, b, d):
    """P(a <= X <= b) via the regularised incomplete beta function.

    (X+1)/2 ~ Beta(alpha, alpha) with alpha = (d-1)/2; each cell is evaluated
    on the tail side closest to it to avoid cancellation.
    """
    alpha = (d - 1) / 2.0
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)

    def upper(x):  # P(X > x)
        return np.where(
            x >= 0,
            special.betainc(alpha, alpha, (1.0 - x) / 2.0),
            1.0 - special.betainc(alpha, alpha, (1.0 + x) / 2.0),
        )

    return upper(a) - upper(b)


def beta_cell_moment(a, b, d):
    """Integral of x f_d(x) over [a, b], closed form.

    d/dx (1-x^2)^(m+1) = -2(m+1) x (1-x^2)^m, so the integral is
    K [(1-a^2)^(m+1) - (1-b^2)^(m+1)] / (2(m+1)) with m = (d-3)/2.
    """
    m = (d - 3) / 2.0
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    w = lambda x: np.exp((m + 1.0) * np.log1p(-x * x))
    with np.errstate(divide="ignore"):
        return np.exp(_log_norm_const(d)) * (w(a) - w(b)) / (2.0 * (m + 1.0))


def _polish_mp(c, d, dps=40, iters=8):
    """Newton refinement of the Lloyd-Max conditions in mpmath.

    Unknowns: the n centroids.  Residual: c_j - E[X | t_{j-1} < X < t_j] with
    t_j = (c_j + c_{j+1})/2, t_{-1} = -1, t_{n-1} = 1.  The Jacobian of the
    conditional mean M_j with respect to the cell ends a < b is
    dM/db = f(b)(b - M)/D and dM/da = f(a)(M - a)/D (D = cell mass), and each
    end moves by 1/2 per neighbouring centroid; it is tridiagonal.
    """
    with mpmath.workdps(dps):
        alpha = mpmath.mpf(d - 1) / 2
        m = mpmath.mpf(d - 3) / 2
        K = mpmath.gamma(mpmath.mpf(d) / 2) / (mpmath.sqrt(mpmath.pi) * mpmath.gamma(alpha))
        one = mpmath.mpf(1)

        def f(x):
            return K * (one - x * x) ** m if abs(x) < 1 else (K if m == 0 else mpmath.mpf(0))

        def moment(a, b):
            return K * ((one - a * a) ** (m + 1) - (one - b * b) ** (m + 1)) / (2 * (m + 1))

        def mass(a, b):
            return mpmath.betainc(alpha, alpha, (a + 1) / 2, (b + 1) / 2, regularized=True)

        n = len(c)
        cm = [mpmath.mpf(float(v)) for v in c]
        for _ in range(iters):
            edges = [-one] + [(cm[j] + cm[j + 1]) / 2 for j in range(n - 1)] + [one]
            D = [mass(edges[j], edges[j + 1]) for j in range(n)]
            M = [moment(edges[j], edges[j + 1]) / D[j] for j in range(n)]
            J = mpmath.zeros(n, n)
            for j in range(n):
                a, b = edges[j], edges[j + 1]
                dMa = f(a) * (M[j] - a) / D[j] if j > 0 else mpmath.mpf(0)
                dMb = f(b) * (b - M[j]) / D[j] if j < n - 1 else mpmath.mpf(0)
                # residual r_j = c_j - M_j ; a depends on c_{j-1}, c_j ; b on c_j, c_{j+1}
                J[j, j] = 1 - (dMa + dMb) / 2
                if j > 0:
                    J[j, j - 1] = -dMa / 2
                if j < n - 1:
                    J[j, j + 1] = -dMb / 2
            r = mpmath.matrix([cm[j] - M[j] for j in range(n)])
            delta = mpmath.lu_solve(J, r)
            cm = [cm[j] - delta[j] for j in range(n)]
            if max(abs(delta[j]) for j in range(n)) < mpmath.mpf(10) ** (-(dps - 5)):
                break
        # symmetrise: the law is even, so c_j = -c_{n-1-j}
        cm = [(cm[j] - cm[n - 1 - j]) / 2 for j in range(n)]
        c64 = np.array([float(v) for v in cm], dtype=np.float64)
        c32 = np.array([_nearest_f32(v) for v in cm], dtype=np.float32)
        return c64, c32


def _nearest_f32(v):
    """float32 nearest to the mpmath value ``v`` (rounded once, not via float64)."""
    f = np.float32(float(v))
    cands = [np.nextafter(f, np.float32(-np.inf)), f, np.nextafter(f, np.float32(np.inf))]
    return min(cands, key=lambda x: abs(mpmath.mpf(float(x)) - v))


@functools.lru_cache(maxsize=None)
def _beta_codebook_cached(d, bits):
    n = 1 << bits
    alpha = (d - 1) / 2.0
    # start from the law's own quantiles at (j + 1/2)/n
    c0 = 2.0 * special.betaincinv(alpha, alpha, (np.arange(n) + 0.5) / n) - 1.0
    c = lloyd_max_iterate(
        lambda a, b: beta_cell_mass(a, b, d),
        lambda a, b: beta_cell_moment(a, b, d),
        c0,
        -1.0,
        1.0,
        tol=1e-13,
    )
    c64, c32 = _polish_mp(c, d)
    t64 = 0.5 * (c32[1:].astype(np.float64) + c32[:-1].astype(np.float64))
    c64.setflags(write=False)
    c32.setflags(write=False)
    t64.setflags(write=False)
    return c64, c32, t64


def beta_codebook(d: int, bits: int):
    """Codebook for head_dim ``d`` and ``bits`` bits per index.

    Returns ``(c64, c32, t64)``: the centroids rounded to float64 and to
    float32 (each rounded once from a 40-digit solution; the float32 ones
    are what the stored format decodes to), and the 2^b - 1
    float64 boundaries (midpoints of consecutive float32 centroids).  Index
    ``j`` decodes to ``c32[j]``; centroids are increasing.
    """
    if d < 3:
        raise ValueError("head_dim must be >= 3")
    if not 1 <= bits <= 8:
        raise ValueError("bits must be in 1..8")
    return _beta_codebook_cached(int(d), int(bits))


def gaussian_lloyd_max(bits: int, tol=1e-13):
    """Lloyd-Max quantiser of N(0, 1) with the same iteration.

    Used only to pin ``lloyd_max_iterate`` against Max's published table.
    Cell mass = Phi(b) - Phi(a); first moment = phi(a) - phi(b).
    """
    n = 1 << bits
    phi = lambda x: np.exp(-0.5 * x * x) / math.sqrt(2.0 * math.pi)
    mass = lambda a, b: special.ndtr(b) - special.ndtr(a)
    moment = lambda a, b: phi(a) - phi(b)
    c0 = special.ndtri((np.arange(n) + 0.5) / n)
    return lloyd_max_iterate(mass, moment, c0, -np.inf, np.inf, tol=tol)
