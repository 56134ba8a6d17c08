"""Pins for the oracle's SplitMix64 / Box-Muller streams (the generator is the reading stated in oracle/splitmix.py)."""

import numpy as np
import pytest
from scipy import stats

from oracle import splitmix as sm


def test_splitmix64_published_vector():
    # First outputs of SplitMix64 from state 0, as published with the
    # generator's reference implementation (Vigna, splitmix64.c).
    assert sm.splitmix64_stream(0, 1)[0] == 0xE220A8397B1DCDAF
    assert sm.splitmix64_stream(0, 2)[1] == 0x6E789E6AA1B965F4


def test_splitmix64_is_counter_based():
    # Output i depends only on state + (i+1) * gamma: restarting from the
    # advanced state continues the same stream.
    full = sm.splitmix64_stream(12345, 10)
    tail = sm.splitmix64_stream((12345 + 4 * sm.GOLDEN_GAMMA) & sm.MASK64, 6)
    assert full[4:] == tail


def test_stream_state_mapping():
    assert sm.stream_state(0, 0) == 0
    assert sm.stream_state(0, 1) == 1
    assert sm.stream_state(5, 1) == 11
    assert sm.stream_state(2 ** 63, 0) == 0  # wraps mod 2^64


def test_uniforms_open_closed_unit_interval():
    u = np.array(sm.uniforms(7, 20000))
    assert u.min() > 0.0 and u.max() <= 1.0
    assert abs(u.mean() - 0.5) < 4 * np.sqrt(1 / 12 / u.size)


def test_normals_moments_and_law():
    z = np.array(sm.normals(3, 100_000))
    se = 1 / np.sqrt(z.size)
    assert abs(z.mean()) < 4 * se
    assert abs(z.var() - 1.0) < 4 * np.sqrt(2.0) * se
    assert stats.kstest(z, "norm").pvalue > 1e-3


def test_box_muller_pair_by_hand():
    w = sm.splitmix64_stream(9, 2)
    v1 = ((w[0] >> 11) + 0.5) * 2.0 ** -53
    v2 = ((w[1] >> 11) + 0.5) * 2.0 ** -53
    r = np.sqrt(-2 * np.log(v1))
    z = sm.normals(9, 2)
    assert z[0] == pytest.approx(r * np.cos(2 * np.pi * v2), rel=1e-15, abs=1e-15)
    assert z[1] == pytest.approx(r * np.sin(2 * np.pi * v2), rel=1e-15, abs=1e-15)


def test_gaussian_matrix_row_major_and_kinds_independent():
    g = sm.gaussian_matrix(3, 4, 11, 0)
    flat = sm.normals(sm.stream_state(11, 0), 12)
    assert np.array_equal(g.reshape(-1), np.array(flat))
    g1 = sm.gaussian_matrix(3, 4, 11, 1)
    assert not np.allclose(g, g1)
