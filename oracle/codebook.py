"""Lloyd-Max codebook for one rotated coordinate of a unit vector.

Page "TurboQuant 설명", section "1단계: 무작위 회전 + PolarQuant 압축": after
the rotation each coordinate of a unit vector in R^d follows
Beta((d-1)/2, (d-1)/2) on [-1, 1]; that law is known in advance, so the
optimal centroids can be computed once per (dimension, bit width) and a
Lloyd-Max quantiser optimal in MSE for it maps each coordinate to a few bits.
Section "TurboQuant 구현 방법" repeats that the codebook is precomputed for the
model's hidden size and the target bit width.

The density on (-1, 1) is f_d(x) = C_d (1 - x^2)^((d-3)/2) with
C_d = Gamma(d/2) / (sqrt(pi) Gamma((d-1)/2)), i.e. the Beta((d-1)/2,(d-1)/2)
law mapped from [0, 1] to [-1, 1].  Cell integrals have closed forms:

  P([a, b])  = I_{(1+b)/2}(alpha, alpha) - I_{(1+a)/2}(alpha, alpha),
               alpha = (d-1)/2, I the regularised incomplete beta;
  mu([a, b]) = int_a^b x f_d(x) dx
             = C_d [(1-a^2)^((d-1)/2) - (1-b^2)^((d-1)/2)] / (d-1).

Lloyd's iteration (S. Lloyd 1957/1982; J. Max 1960): boundaries are the
midpoints of adjacent centroids, centroids are the conditional means of their
cells.  Start at the (k + 1/2)/K quantiles; stop when no centroid moves by more
than ``tol``.  Distortion per coordinate: E[X^2] - sum_k P_k c_k^2 with
E[X^2] = 1/d.  The library solves the same fixed point by numerical
quadrature; this closed-form route is independent of it.
"""

import functools
import math

import numpy as np
from scipy import special


def _alpha(d):
    return 0.5 * (d - 1)


def log_norm_const(d):
    """log C_d."""
    return math.lgamma(d / 2.0) - 0.5 * math.log(math.pi) - math.lgamma((d - 1) / 2.0)


def density(x, d):
    """f_d(x) on (-1, 1)."""
    x = np.asarray(x, dtype=np.float64)
    return np.exp(log_norm_const(d)) * np.power(1.0 - x * x, 0.5 * (d - 3))


def cdf(x, d):
    """F(x) = P(X <= x)."""
    a = _alpha(d)
    return special.betainc(a, a, 0.5 * (1.0 + np.asarray(x, dtype=np.float64)))


def cell_mass(lo, hi, d):
    """P(lo < X < hi), evaluated on the tail that avoids cancellation."""
    a = _alpha(d)
    lo = np.asarray(lo, dtype=np.float64)
    hi = np.asarray(hi, dtype=np.float64)
    lower = special.betainc(a, a, 0.5 * (1.0 + hi)) - special.betainc(a, a, 0.5 * (1.0 + lo))
    upper = special.betainc(a, a, 0.5 * (1.0 - lo)) - special.betainc(a, a, 0.5 * (1.0 - hi))
    return np.where(lo >= 0.0, upper, lower)


def cell_first_moment(lo, hi, d):
    """int_lo^hi x f_d(x) dx in closed form."""
    e = 0.5 * (d - 1)
    lo = np.asarray(lo, dtype=np.float64)
    hi = np.asarray(hi, dtype=np.float64)
    c = math.exp(log_norm_const(d))
    return c * (np.power(1.0 - lo * lo, e) - np.power(1.0 - hi * hi, e)) / (d - 1)


def quantile_init(d, levels):
    """Centroids at the (k + 1/2)/K quantiles of f_d."""
    a = _alpha(d)
    p = (np.arange(levels) + 0.5) / levels
    return 2.0 * special.betaincinv(a, a, p) - 1.0


def lloyd_max(d, bits, init=None, tol=1e-15, max_iter=1_000_000):
    """Lloyd-Max fixed point for f_d with 2**bits levels.

    Returns (centroids, boundaries, iterations); raises RuntimeError when the
    iteration does not settle within ``max_iter`` steps.
    """
    if d < 3:
        raise ValueError("d must be >= 3")
    if not 1 <= bits <= 8:
        raise ValueError("bits must be in 1..8")
    levels = 1 << bits
    c = quantile_init(d, levels) if init is None else np.array(init, dtype=np.float64)
    for it in range(1, max_iter + 1):
        t = 0.5 * (c[:-1] + c[1:])
        edges = np.concatenate(([-1.0], t, [1.0]))
        mass = cell_mass(edges[:-1], edges[1:], d)
        mom = cell_first_moment(edges[:-1], edges[1:], d)
        c_new = mom / mass
        step = np.max(np.abs(c_new - c))
        c = c_new
        if step < tol:
            return c, 0.5 * (c[:-1] + c[1:]), it
    raise RuntimeError("Lloyd-Max iteration did not converge")


def distortion_per_coord(d, centroids):
    """E[(X - Q(X))^2] for the nearest-centroid quantiser of ``centroids``.

    Sum over cells of E[X^2; cell] - 2 c mu + c^2 P, with the cell second
    moments summed in closed form to E[X^2] = 1/d:
    D = 1/d - sum_k c_k (2 mu_k - c_k P_k).  (At the fixed point mu = c P and
    this is 1/d - sum P c^2.)  Summing 1/d once avoids the cancellation of
    per-cell second moments near x = 0.
    """
    c = np.asarray(centroids, dtype=np.float64)
    t = 0.5 * (c[:-1] + c[1:])
    edges = np.concatenate(([-1.0], t, [1.0]))
    mass = cell_mass(edges[:-1], edges[1:], d)
    mom = cell_first_moment(edges[:-1], edges[1:], d)
    return float(1.0 / d - np.sum(c * (2.0 * mom - c * mass)))


@functools.lru_cache(maxsize=None)
def _codebook_cached(d, bits):
    c, _, _ = lloyd_max(d, bits)
    # The law is symmetric and log-concave, so the Lloyd-Max fixed point is
    # unique (P. Fleischer 1964) and therefore symmetric; averaging c_k with
    # -c_{K-1-k} only removes rounding noise (<1e-14, pinned by the tests on
    # the raw iteration) and makes the middle boundary exactly 0.
    c = 0.5 * (c - c[::-1])
    t = 0.5 * (c[:-1] + c[1:])
    return c, t, distortion_per_coord(d, c)


def codebook(d, bits):
    """(centroids, boundaries, distortion per coordinate) for (d, bits)."""
    c, t, dist = _codebook_cached(int(d), int(bits))
    return c.copy(), t.copy(), dist
