"""Pins for Pi, S and M = S Pi^T (page section "1단계"; the sign fix and y = Pi x are the readings stated in oracle/rotation.py)."""

import numpy as np
import pytest
from scipy import stats

from oracle import rotation as rot


@pytest.mark.parametrize("d", [16, 128, 256])
def test_pi_orthogonal(d):
    p = rot.haar_rotation(d, 0)
    assert np.max(np.abs(p.T @ p - np.eye(d))) < 1e-10
    assert np.max(np.abs(p @ p.T - np.eye(d))) < 1e-10


def test_pi_is_qr_of_gaussian_with_positive_r_diagonal():
    # Pi^T G must be upper triangular with a positive diagonal (the unique QR
    # of G with R_ii > 0).
    from oracle.splitmix import gaussian_matrix
    d = 32
    g = gaussian_matrix(d, d, 4, rot.KIND_PI)
    p = rot.haar_rotation(d, 4)
    r = p.T @ g
    assert np.max(np.abs(np.tril(r, -1))) < 1e-12
    assert np.all(np.diag(r) > 0)


def test_haar_sign_fix():
    # Haar: Pi[0, 0] is symmetric about 0.  LAPACK's Householder QR alone
    # always returns Q[0, 0] <= 0, so a missing sign fix fails this test.
    d = 8
    vals = np.array([rot.haar_rotation(d, s)[0, 0] for s in range(1000)])
    se = vals.std() / np.sqrt(vals.size)
    assert abs(vals.mean()) < 3 * se


def test_rotated_coordinate_follows_beta_law():
    # Page section "1단계": after the rotation each coordinate of a unit vector
    # follows Beta((d-1)/2, (d-1)/2) on [-1, 1].
    d = 12
    v = np.zeros(d)
    v[0] = 0.6
    v[3] = 0.8
    ys = np.array([(rot.haar_rotation(d, s) @ v)[2] for s in range(3000)])
    law = stats.beta((d - 1) / 2, (d - 1) / 2, loc=-1, scale=2)
    assert stats.kstest(ys, law.cdf).pvalue > 1e-3


def test_qjl_matrix_is_kind1_stream_and_m_relation():
    d = 16
    s = rot.qjl_matrix(d, 3)
    p = rot.haar_rotation(d, 3)
    m = rot.qjl_rotated(d, 3)
    r = np.random.default_rng(0).standard_normal(d)
    # S r == M (Pi r): the QJL projection in the rotated domain.
    assert np.allclose(s @ r, m @ (p @ r), rtol=0, atol=1e-12)
    assert np.array_equal(rot.make_rotation(d, 3, 1), s)
    assert abs(s.mean()) < 4 / d and abs(s.var() - 1) < 0.2
