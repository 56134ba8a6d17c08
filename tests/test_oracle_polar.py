"""Pins for the PolarQuant variant of the oracle (oracle/polar.py).

The transform is pinned by a hand-worked example and by its inverse; the
angle laws by closed forms (k = 1, 2) and by Monte Carlo on the sphere; the
codebooks by the Lloyd conditions with closed-form cell integrals (k = 2) and
brute-force quadrature; the quantiser by brute-force nearest centroids,
exact reconstruction of vectors sitting on centroids, zero vectors and the
distortion the page reports for 3 bits.
"""

import math

import numpy as np
import pytest
from scipy import stats

from oracle import polar as pq
from oracle import quantizer as qz
from oracle import rotation as rot


def test_hand_worked_d4():
    y = np.array([[1.0, 1.0, 0.0, 2.0]])
    phi, psis, r = pq.polar_angles(y)
    np.testing.assert_allclose(phi[0], [math.pi / 4, math.pi / 2], rtol=0, atol=1e-15)
    np.testing.assert_allclose(psis[0][0], [math.atan(2.0 / math.sqrt(2.0))], rtol=0, atol=1e-15)
    assert abs(r[0] - math.sqrt(6.0)) < 1e-15
    # third quadrant and a negative-zero-free fourth quadrant angle
    phi2, _, _ = pq.polar_angles(np.array([[-1.0, -1.0, 1.0, -1.0]]))
    np.testing.assert_allclose(phi2[0], [1.25 * math.pi, 1.75 * math.pi], rtol=0, atol=1e-15)


def test_round_trip():
    y = np.random.default_rng(1).standard_normal((50, 64))
    phi, psis, r = pq.polar_angles(y)
    np.testing.assert_allclose(pq.from_angles(phi, psis, r), y, rtol=0, atol=1e-13)
    np.testing.assert_allclose(r, np.linalg.norm(y, axis=1), rtol=1e-15, atol=0)
    assert np.all((phi >= 0) & (phi < 2 * math.pi))
    assert all(np.all((p >= 0) & (p <= math.pi / 2)) for p in psis)


def test_law_closed_forms():
    t = np.linspace(0.01, math.pi / 2 - 0.01, 50)
    np.testing.assert_allclose(pq.angle_cdf(t, 1), 2 * t / math.pi, rtol=1e-13, atol=1e-15)
    np.testing.assert_allclose(pq.angle_cdf(t, 2), np.sin(t) ** 2, rtol=1e-13, atol=1e-15)
    np.testing.assert_allclose(pq.angle_pdf(t, 2), np.sin(2 * t), rtol=1e-13, atol=1e-15)
    for k in (1, 2, 4, 16, 64):
        from scipy import integrate
        tot, _ = integrate.quad(lambda s: float(pq.angle_pdf(s, k)), 0, math.pi / 2, limit=200)
        assert abs(tot - 1.0) < 1e-9
        h = 1e-6
        mid = np.array([0.3, 0.7, 1.1])
        num = (pq.angle_cdf(mid + h, k) - pq.angle_cdf(mid - h, k)) / (2 * h)
        np.testing.assert_allclose(num, pq.angle_pdf(mid, k), rtol=1e-6)


def test_laws_on_the_sphere():
    rng = np.random.default_rng(7)
    g = rng.standard_normal((20000, 128))
    y = g / np.linalg.norm(g, axis=1, keepdims=True)
    phi, psis, _ = pq.polar_angles(y)
    assert stats.kstest(phi[:, 0], "uniform", args=(0, 2 * math.pi)).pvalue > 1e-3
    for lv, psi in enumerate(psis, start=2):
        k = 1 << (lv - 1)
        p = stats.kstest(psi[:, 0], lambda s: pq.angle_cdf(s, k)).pvalue
        assert p > 1e-3, (lv, p)


def _closed_k2(lo, hi):
    # density sin 2t: mass [-cos 2t / 2], first moment [sin 2t / 4 - t cos 2t / 2]
    f = lambda t: math.sin(2 * t) / 4 - t * math.cos(2 * t) / 2
    m = (math.cos(2 * lo) - math.cos(2 * hi)) / 2
    return m, f(hi) - f(lo)


def test_codebook_k2_closed_form_fixed_point():
    c, t = pq.angle_codebook(2, 2)
    np.testing.assert_allclose(t, 0.5 * (c[1:] + c[:-1]), rtol=0, atol=1e-15)
    edges = [0.0, *t, math.pi / 2]
    for i in range(4):
        m, f = _closed_k2(edges[i], edges[i + 1])
        assert abs(f / m - c[i]) < 1e-12
    np.testing.assert_allclose(c + c[::-1], math.pi / 2, rtol=0, atol=1e-14)


@pytest.mark.parametrize("k", [4, 32, 64])
def test_codebook_lloyd_conditions_brute_force(k):
    c, t = pq.angle_codebook(k, 2)
    edges = [0.0, *t, math.pi / 2]
    for i in range(4):
        g = np.linspace(edges[i], edges[i + 1], 200001)      # trapezoid rule on each cell
        w = pq.angle_pdf(g, k)
        assert abs(np.trapezoid(g * w, g) / np.trapezoid(w, g) - c[i]) < 1e-9
    np.testing.assert_allclose(c + c[::-1], math.pi / 2, rtol=0, atol=1e-14)


def test_level1_sectors():
    c, t = pq.level1_codebook()
    assert len(c) == 16 and len(t) == 15
    ang = np.random.default_rng(3).uniform(0, 2 * math.pi, 5000)
    idx = np.minimum(np.floor(ang * 16 / (2 * math.pi)).astype(int), 15)
    circ = np.abs((ang[:, None] - c[None, :] + math.pi) % (2 * math.pi) - math.pi)
    np.testing.assert_array_equal(idx, np.argmin(circ, axis=1))


def test_quantize_is_nearest_centroid_and_packs():
    d = 64
    pi = rot.haar_rotation(d, 0)
    x = np.random.default_rng(4).standard_normal((300, d)) * 3.0
    ref = pq.quantize(x, pi)
    books = pq.codebooks(d)
    off = 0
    for lv, psi in enumerate(ref["psis"], start=2):
        c = books[lv - 1][0]
        want = np.argmin(np.abs(psi[:, :, None] - c[None, None, :]), axis=2)
        got = ref["idx_up"][:, off:off + psi.shape[1]]
        np.testing.assert_array_equal(got, want)
        off += psi.shape[1]
    sector = np.sum(ref["phi"][:, :, None] >= books[0][1][None, None, :], axis=2)
    np.testing.assert_array_equal(ref["idx1"], sector)
    i1, iu = pq.unpack(ref["codes"], d)
    np.testing.assert_array_equal(i1, ref["idx1"])
    np.testing.assert_array_equal(iu, ref["idx_up"])
    assert ref["codes"].shape == (300, pq.row_bytes(d))
    with pytest.raises(ValueError):
        pq.pack(ref["idx1"][:, :16], ref["idx_up"][:, :15], 32)


def test_vectors_on_centroids_reconstruct_exactly():
    d = 64
    pi = rot.haar_rotation(d, 2)
    rng = np.random.default_rng(5)
    books = pq.codebooks(d)
    phi = books[0][0][rng.integers(0, 16, (20, d // 2))]
    psis = [books[lv - 1][0][rng.integers(0, 4, (20, d >> lv))] for lv in range(2, pq.n_levels(d) + 1)]
    y = pq.from_angles(phi, psis)
    n = np.float64(np.float16(2.5))                     # an fp16-exact norm
    x = n * (y @ pi)
    ref = pq.quantize(x, pi)
    xh = pq.dequantize(ref["codes"], ref["norm"], pi)
    np.testing.assert_allclose(xh, x, rtol=0, atol=1e-12)


def test_zero_vector_and_distortion():
    d = 128
    pi = rot.haar_rotation(d, 0)
    x = np.random.default_rng(6).standard_normal((2000, d)) * np.exp(np.random.default_rng(9).standard_normal(d))
    x[0] = 0.0
    ref = pq.quantize(x, pi)
    assert np.all(ref["idx1"][0] == 0) and np.all(ref["idx_up"][0] == 0) and ref["norm"][0] == 0
    xh = pq.dequantize(ref["codes"], ref["norm"], pi)
    assert np.all(xh[0] == 0.0)
    cos = np.sum(x[1:] * xh[1:], 1) / np.linalg.norm(x[1:], axis=1) / np.linalg.norm(xh[1:], axis=1)
    assert 0.98 < cos.mean() < 0.99                     # the page: about 0.983 at 3 bits
    yh = xh[1:] @ pi.T / qz.from_fp16_bits(ref["norm"][1:])[:, None]
    np.testing.assert_allclose(np.linalg.norm(yh, axis=1), 1.0, rtol=1e-13)


@pytest.mark.parametrize("d", [64, 128])
def test_logits_rotated_form_equals_dequantize_then_dot(d):
    """The bottom-up pass over the angle tree with the rotated query equals
    the plain definition (reconstruct x_hat, then dot): a dropped level, a
    swapped cos/sin or a wrong slot in either fails."""
    pi = rot.haar_rotation(d, 3)
    rng = np.random.default_rng(d)
    x = rng.standard_normal((300, d)) * np.exp(rng.standard_normal(d))
    x[7] = 0.0
    ref = pq.quantize(x, pi)
    q = rng.standard_normal((5, d))
    want = pq.logits(q, ref["codes"], ref["norm"], pi, 0.3)
    got = pq.logits_rotated(q, ref["codes"], ref["norm"], pi, 0.3)
    np.testing.assert_allclose(got, want, rtol=1e-12, atol=1e-12 * np.abs(want).max())
    assert np.all(got[:, 7] == 0.0)


def test_logits_closed_case():
    """Pi = I, x = 3 e_0 and x = e_1 + e_2 at d = 64: every angle is known by hand.
    e_0: every level-1 angle is 0 (sector 0, midpoint pi/16), every higher
    angle 0 (lowest cell), so y_hat_0 = cos(pi/16) prod_l cos(c_l[0]),
    y_hat_1 = sin(pi/16) prod_l cos(c_l[0]) and y_hat_2 = cos(pi/16)
    sin(c_2[0]) prod_{l>2} cos(c_l[0]).  e_1 + e_2: pair 0 has angle
    pi/2 (sector 4), pair 1 angle 0 (sector 0), the level-2 angle of pairs 0
    and 1 is pi/4 (cell 2 of its 4: the law is symmetric about pi/4 and ties
    go up), every higher angle 0."""
    d = 64
    pi = np.eye(d)
    books = pq.codebooks(d)
    up0 = np.prod([math.cos(books[lv - 1][0][0]) for lv in range(2, pq.n_levels(d) + 1)])
    x = np.zeros((2, d))
    x[0, 0] = 3.0
    x[1, 1] = x[1, 2] = 1.0
    ref = pq.quantize(x, pi)
    n16 = qz.from_fp16_bits(ref["norm"])
    assert n16[0] == 3.0
    q = np.zeros((3, d))
    q[0, 0] = 1.0
    q[1, 1] = 1.0
    q[2, 2] = 1.0
    got = pq.logits_rotated(q, ref["codes"], ref["norm"], pi, 0.5)
    c16, s16 = math.cos(math.pi / 16), math.sin(math.pi / 16)
    assert abs(got[0, 0] - 0.5 * 3.0 * c16 * up0) < 1e-14
    assert abs(got[1, 0] - 0.5 * 3.0 * s16 * up0) < 1e-14
    # coordinate 2 is pair 1 (angle 0, sector 0): its radius takes sin of the
    # level-2 centroid, not cos, and the reconstruction does not vanish there
    rest = np.prod([math.cos(books[lv - 1][0][0]) for lv in range(3, pq.n_levels(d) + 1)])
    assert abs(got[2, 0] - 0.5 * 3.0 * math.sin(books[1][0][0]) * rest * c16) < 1e-14
    # e_1 + e_2: y_hat_1 = cos(psi_2) * rest * sin(9 pi/16), y_hat_2 = sin(psi_2) * rest * cos(pi/16)
    assert ref["idx1"][1, 0] == 4 and ref["idx1"][1, 1] == 0 and ref["idx_up"][1, 0] == 2
    c2 = books[1][0][2]
    sq2 = n16[1]
    assert abs(got[1, 1] - 0.5 * sq2 * math.cos(c2) * rest * math.sin(9 * math.pi / 16)) < 1e-14
    assert abs(got[2, 1] - 0.5 * sq2 * math.sin(c2) * rest * math.cos(math.pi / 16)) < 1e-14
