"""Pins for the Lloyd-Max codebook of the Beta coordinate law (page section "1단계")."""

import math

import numpy as np
import pytest
from scipy import special, stats

from oracle import codebook as cb

CASES = [(16, 1), (16, 3), (64, 2), (128, 1), (128, 2), (128, 3), (128, 4), (256, 2), (256, 4)]


@pytest.mark.parametrize("d,bits", CASES)
def test_raw_iteration_symmetric(d, bits):
    c, t, _ = cb.lloyd_max(d, bits)
    assert np.max(np.abs(c + c[::-1])) < 1e-12
    assert np.all(np.diff(c) > 0)
    assert np.allclose(t, 0.5 * (c[:-1] + c[1:]), rtol=0, atol=0)


@pytest.mark.parametrize("d,bits", CASES)
def test_converged_fixed_point(d, bits):
    c, t, _ = cb.codebook(d, bits)
    edges = np.concatenate(([-1.0], t, [1.0]))
    cond_mean = cb.cell_first_moment(edges[:-1], edges[1:], d) / cb.cell_mass(edges[:-1], edges[1:], d)
    assert np.max(np.abs(cond_mean - c)) < 1e-12


def test_unique_fixed_point_from_other_start():
    d, bits = 128, 3
    c_q, _, _ = cb.lloyd_max(d, bits)
    init = np.linspace(-0.5, 0.3, 8)           # asymmetric, far from the optimum
    c_o, _, _ = cb.lloyd_max(d, bits, init=init)
    assert np.max(np.abs(c_q - c_o)) < 1e-12


@pytest.mark.parametrize("bits", [1, 2, 3])
def test_d3_is_uniform(bits):
    # d = 3: Beta(1, 1) on [-1, 1] is uniform, so the optimum is the uniform
    # quantiser: c_k = -1 + (2k + 1) / K and D = 1 / (3 K^2).
    k = 1 << bits
    c, t, dist = cb.codebook(3, bits)
    assert np.allclose(c, -1 + (2 * np.arange(k) + 1) / k, rtol=0, atol=1e-14)
    assert dist == pytest.approx(1 / (3 * k * k), rel=1e-12)


@pytest.mark.parametrize("d", [5, 16, 128, 256])
def test_one_bit_closed_form(d):
    # b' = 1: centroids are +-E|X| = +-Gamma(d/2) / (sqrt(pi) Gamma((d+1)/2)).
    c, t, dist = cb.codebook(d, 1)
    e_abs = math.exp(math.lgamma(d / 2) - 0.5 * math.log(math.pi) - math.lgamma((d + 1) / 2))
    assert c[1] == pytest.approx(e_abs, rel=1e-13)
    assert t[0] == 0.0
    assert dist == pytest.approx(1 / d - e_abs ** 2, rel=1e-11)


# J. Max (1960), "Quantizing for minimum distortion", optimum levels for a unit
# Gaussian (positive half) and their mean squared errors.
MAX_LEVELS = {1: [0.7979], 2: [0.4528, 1.510], 3: [0.2451, 0.7560, 1.344, 2.152],
              4: [0.1284, 0.3881, 0.6568, 0.9424, 1.256, 1.618, 2.069, 2.733]}
MAX_MSE = {1: 0.3634, 2: 0.1175, 3: 0.03455, 4: 0.009497}


@pytest.mark.parametrize("bits", [1, 2, 3, 4])
def test_gaussian_limit(bits):
    # sqrt(d) X -> N(0, 1) as d grows, so sqrt(d) c tends to Max's levels.
    d = 65536
    c, _, _ = cb.lloyd_max(d, bits, tol=1e-13)
    pos = math.sqrt(d) * c[len(c) // 2:]
    assert np.max(np.abs(pos - MAX_LEVELS[bits])) < 1.2e-3
    assert d * cb.distortion_per_coord(d, c) == pytest.approx(MAX_MSE[bits], rel=2e-3)


def test_density_and_cdf_match_scipy_beta():
    d = 40
    law = stats.beta((d - 1) / 2, (d - 1) / 2, loc=-1, scale=2)
    x = np.linspace(-0.9, 0.9, 19)
    assert np.allclose(cb.density(x, d), law.pdf(x), rtol=1e-12)
    assert np.allclose(cb.cdf(x, d), law.cdf(x), rtol=1e-12)
    lo, hi = np.array([-0.3, 0.1, -1.0]), np.array([0.2, 0.7, 1.0])
    assert np.allclose(cb.cell_mass(lo, hi, d), law.cdf(hi) - law.cdf(lo), rtol=1e-12)
    num = [law.expect(lambda v: v, lb=a, ub=b) for a, b in zip(lo, hi)]
    assert np.allclose(cb.cell_first_moment(lo, hi, d), num, rtol=1e-8, atol=1e-14)


@pytest.mark.parametrize("d,bits", [(128, 2), (128, 3), (128, 4), (256, 4)])
def test_empirical_mse_matches_integrated_distortion(d, bits):
    # Random unit vectors have exactly the Beta coordinate law; quantising
    # every coordinate must reproduce the distortion within 2%.
    rng = np.random.default_rng(d * 10 + bits)
    v = rng.standard_normal((10_000, d))
    v /= np.linalg.norm(v, axis=1, keepdims=True)
    c, t, dist = cb.codebook(d, bits)
    idx = np.searchsorted(t, v, side="right")
    mse = np.mean((v - c[idx]) ** 2)
    assert mse == pytest.approx(dist, rel=0.02)


def test_boundary_count_equals_nearest_centroid():
    c, t, _ = cb.codebook(128, 3)
    v = np.random.default_rng(1).uniform(-0.4, 0.4, 100_000)
    by_count = np.sum(v[:, None] >= t[None, :], axis=1)
    brute = np.argmin(np.abs(v[:, None] - c[None, :]), axis=1)
    assert np.array_equal(by_count, brute)


def test_rejects_bad_arguments():
    with pytest.raises(ValueError):
        cb.lloyd_max(2, 3)
    with pytest.raises(ValueError):
        cb.lloyd_max(128, 0)
    with pytest.raises(RuntimeError):
        cb.lloyd_max(256, 4, max_iter=3)


def test_mass_sums_to_one():
    for d, bits in [(7, 2), (128, 4), (256, 4)]:
        c, t, _ = cb.codebook(d, bits)
        edges = np.concatenate(([-1.0], t, [1.0]))
        assert np.sum(cb.cell_mass(edges[:-1], edges[1:], d)) == pytest.approx(1.0, abs=1e-13)
        assert special.betainc((d - 1) / 2, (d - 1) / 2, 0.5) == pytest.approx(0.5, abs=1e-15)
