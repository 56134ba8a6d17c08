"""PolarQuant variant of stage 1 (fp64).

Test infrastructure: only the tests, the smoke check and the benchmark's CPU
baseline use this module; the GPU path never calls it.

Page "TurboQuant 설명: 무엇인지와 LLM 메모리 6배 절약 구현 방법", section
"1단계: 무작위 회전 + PolarQuant 압축": after the random rotation the vector is
normalised and turned from Cartesian into polar coordinates by pairing the
dimensions recursively; the radius carries the magnitude, the angles the
direction; the angle laws are concentrated and known in advance, so no
per-block normalisation constants are stored; Lloyd-Max quantisers map the
values to a few bits (about 3 bits per coordinate in all).

Readings (the page gives the idea only):
* d = 2^L.  Level 1 pairs the rotated unit coordinates (y_2i, y_2i+1) into a
  radius and an angle phi_i = atan2(y_2i+1, y_2i) taken in [0, 2 pi); level
  l >= 2 pairs the radii (rho_2i, rho_2i+1) of level l - 1 into a radius and
  an angle psi_i = atan2(rho_2i+1, rho_2i) in [0, pi/2].  After L levels one
  radius is left, ||y|| = 1; the norm n = ||x|| is stored as fp16 as in the
  per-coordinate variant.
* Laws, for y uniform on the sphere (which the Haar rotation gives for any
  fixed x): phi is uniform on [0, 2 pi); at level l the two radii are norms
  of independent k = 2^(l-1)-dimensional Gaussian blocks up to one common
  scale, so sin^2 psi ~ Beta(k/2, k/2): density 2 (sin psi cos psi)^(k-1) /
  B(k/2, k/2) on [0, pi/2].
* Bits (the page gives none): 4 bits for every level-1 angle, 2 bits for
  every higher angle: 4 d/2 + 2 (d/2 - 1) = 3 d - 2 bits, the page's 3 bits
  per coordinate.  Codebooks are the Lloyd-Max quantisers of each law in the
  angle (squared-error) metric; the uniform circular law is served by 16
  equal sectors [2 pi j/16, 2 pi (j+1)/16) with their midpoints as centroids
  (every rotation of that partition is optimal; this one is fixed).  Ties
  go to the upper cell, as in the per-coordinate variant.
* Packing, 3 d / 8 bytes per vector (d >= 64, so the planes fill whole
  32-slot groups): the d/2 level-1 indices as 4 bit planes
  over groups of 32 slots (group g at words 4 g + p), then the higher indices
  in level order (level 2 first; one zero slot pads them to d/2) as 2 bit
  planes at words 2 d / 32 + 2 g + p.
* A zero vector (and a pair or block whose coordinates are all zero) has
  angle 0 (atan2(0, 0) = 0); it reconstructs to 0 through n = 0.
* Reconstruction: y_hat from the centroid angles from the top down (radius
  1), x_hat = n16 Pi^T y_hat; y_hat is a unit vector by construction.
* Logits: scale * <q, x_hat> (``logits``, the definition); ``logits_rotated``
  reaches the same value from the rotated query without forming x_hat.
"""

import functools
import math

import numpy as np
from scipy import integrate, special

from . import quantizer as qz

LEVEL1_BITS = 4
UPPER_BITS = 2


def n_levels(d):
    L = int(round(math.log2(d)))
    if d < 4 or (1 << L) != d:
        raise ValueError("d must be a power of two >= 4")
    return L


def check_packable(d):
    """The packed layout needs whole 32-slot groups: d >= 64."""
    if n_levels(d) < 6:
        raise ValueError("packed polar codes need d >= 64")


def polar_angles(y):
    """Angles of rows y [n, d]: (phi [n, d/2] in [0, 2 pi), [psi_2, ..., psi_L], radius [n])."""
    y = np.asarray(y, dtype=np.float64)
    L = n_levels(y.shape[1])
    even, odd = y[:, 0::2], y[:, 1::2]
    phi = np.arctan2(odd, even)
    phi = np.where(phi < 0.0, phi + 2.0 * math.pi, phi)
    rho = np.hypot(even, odd)
    psis = []
    for _ in range(2, L + 1):
        a, b = rho[:, 0::2], rho[:, 1::2]
        psis.append(np.arctan2(b, a))
        rho = np.hypot(a, b)
    return phi, psis, rho[:, 0]


def from_angles(phi, psis, radius=None):
    """Inverse of ``polar_angles``: rows y from the angles (radius 1 unless given)."""
    phi = np.asarray(phi, dtype=np.float64)
    n = phi.shape[0]
    rho = np.ones((n, 1)) if radius is None else np.asarray(radius, dtype=np.float64).reshape(n, 1)
    for psi in reversed(psis):
        psi = np.asarray(psi, dtype=np.float64)
        nxt = np.empty((n, 2 * rho.shape[1]))
        nxt[:, 0::2] = rho * np.cos(psi)
        nxt[:, 1::2] = rho * np.sin(psi)
        rho = nxt
    y = np.empty((n, 2 * rho.shape[1]))
    y[:, 0::2] = rho * np.cos(phi)
    y[:, 1::2] = rho * np.sin(phi)
    return y


def angle_pdf(psi, k):
    """Density of a level angle whose two radii span k dimensions each."""
    psi = np.asarray(psi, dtype=np.float64)
    lb = special.betaln(k / 2.0, k / 2.0)
    s = np.sin(psi) * np.cos(psi)
    with np.errstate(divide="ignore"):
        return np.where(s > 0.0, 2.0 * np.exp((k - 1) * np.log(np.where(s > 0.0, s, 1.0)) - lb),
                        2.0 / math.exp(lb) if k == 1 else 0.0)


def angle_cdf(psi, k):
    """P(Psi <= psi) = I_{sin^2 psi}(k/2, k/2)."""
    return special.betainc(k / 2.0, k / 2.0, np.sin(np.asarray(psi, dtype=np.float64)) ** 2)


def _cell_moments(lo, hi, k):
    mass = float(angle_cdf(hi, k) - angle_cdf(lo, k))
    first, _ = integrate.quad(lambda t: t * float(angle_pdf(t, k)), lo, hi, epsabs=0.0, epsrel=1e-13, limit=200)
    return mass, first


@functools.lru_cache(maxsize=None)
def _angle_codebook(k, bits):
    K = 1 << bits
    q = (np.arange(K) + 0.5) / K
    # start at the quantiles (inverse of the Beta cdf through sin^2)
    c = np.arcsin(np.sqrt(special.betaincinv(k / 2.0, k / 2.0, q)))
    for _ in range(10000):
        t = 0.5 * (c[1:] + c[:-1])
        edges = np.concatenate([[0.0], t, [0.5 * math.pi]])
        new = np.empty(K)
        for i in range(K):
            mass, first = _cell_moments(edges[i], edges[i + 1], k)
            new[i] = first / mass
        step = np.max(np.abs(new - c))
        c = new
        if step < 1e-14:
            break
    # the law is symmetric about pi/4
    c = 0.5 * (c + (0.5 * math.pi - c[::-1]))
    return c, 0.5 * (c[1:] + c[:-1])


def angle_codebook(k, bits=UPPER_BITS):
    """Lloyd-Max centroids and boundaries (angles) for the level law with k."""
    c, t = _angle_codebook(k, bits)
    return c.copy(), t.copy()


def level1_codebook(bits=LEVEL1_BITS):
    """Uniform circular law: sector boundaries 2 pi j / K, midpoints as centroids."""
    K = 1 << bits
    c = 2.0 * math.pi * (np.arange(K) + 0.5) / K
    t = 2.0 * math.pi * np.arange(1, K) / K
    return c, t


def codebooks(d):
    """[(centroids, boundaries)] for levels 1..L."""
    L = n_levels(d)
    books = [level1_codebook()]
    for level in range(2, L + 1):
        books.append(angle_codebook(1 << (level - 1)))
    return books


def row_bytes(d):
    return 3 * d // 8


def pack(idx1, idx_up, d):
    """Codes [n, 3 d / 8] from level-1 indices [n, d/2] and the higher ones [n, d/2 - 1]."""
    check_packable(d)
    n = idx1.shape[0]
    up = np.concatenate([idx_up, np.zeros((n, 1), dtype=np.int64)], axis=1)
    a = qz.pack_planes(idx1, LEVEL1_BITS)
    b = qz.pack_planes(up, UPPER_BITS)
    return np.concatenate([a, b], axis=1)


def unpack(codes, d):
    check_packable(d)
    codes = np.asarray(codes, dtype=np.uint8)
    na = LEVEL1_BITS * (d // 2) // 8
    idx1 = qz.unpack_planes(codes[:, :na], LEVEL1_BITS, d // 2)
    up = qz.unpack_planes(codes[:, na:], UPPER_BITS, d // 2)
    return idx1, up[:, :d // 2 - 1]


def quantize(x, pi):
    """Rows of x -> dict(codes, norm, and the fp64 intermediates the parity rules need)."""
    x = np.asarray(x, dtype=np.float64)
    n_vec, d = x.shape
    L = n_levels(d)
    norm = np.sqrt(np.einsum("ij,ij->i", x, x))
    safe = np.where(norm > 0.0, norm, 1.0)
    u = np.where(norm[:, None] > 0.0, x / safe[:, None], 0.0)
    y = u @ pi.T
    phi, psis, _ = polar_angles(y)
    books = codebooks(d)
    idx1 = np.minimum(np.floor(phi * ((1 << LEVEL1_BITS) / (2.0 * math.pi))).astype(np.int64),
                      (1 << LEVEL1_BITS) - 1)
    ups = [np.sum(p[:, :, None] >= books[lv + 1][1][None, None, :], axis=2) for lv, p in enumerate(psis)]
    idx_up = np.concatenate(ups, axis=1) if ups else np.zeros((n_vec, 0), dtype=np.int64)
    return {"codes": pack(idx1, idx_up, d), "norm": qz.to_fp16_bits(norm), "norm64": norm,
            "y": y, "phi": phi, "psis": psis, "idx1": idx1, "idx_up": idx_up}


def dequantize(codes, norm, pi):
    """x_hat = n16 Pi^T y_hat for packed rows."""
    d = pi.shape[0]
    L = n_levels(d)
    books = codebooks(d)
    idx1, idx_up = unpack(codes, d)
    phi = books[0][0][idx1]
    psis, off = [], 0
    for level in range(2, L + 1):
        cnt = d >> level
        psis.append(books[level - 1][0][idx_up[:, off:off + cnt]])
        off += cnt
    y = from_angles(phi, psis)
    return qz.from_fp16_bits(norm)[:, None] * (y @ pi)


def logits(q, codes, norm, pi, scale):
    """scale * <q, x_hat> for every query row of q [m, d] and packed key row:
    the plain definition, through the reconstruction (logits [m, n])."""
    q = np.asarray(q, dtype=np.float64)
    return scale * (q @ dequantize(codes, norm, pi).T)


def logits_rotated(q, codes, norm, pi, scale):
    """The same logits through the query rotated once (page: the query is
    rotated once, section "2단계" closing paragraph) and a bottom-up pass over
    the angle tree, without forming y_hat: a level-1 pair i contributes
    a_i = q'_2i cos(phi_i) + q'_2i+1 sin(phi_i); an angle psi of level l joins
    the partial sums of the two nodes it splits as cos(psi) a_2i + sin(psi)
    a_2i+1; the last one left is <q', y_hat>, and the logit is
    scale * n16 * <q', y_hat> with q' = Pi q."""
    q = np.asarray(q, dtype=np.float64)
    d = pi.shape[0]
    L = n_levels(d)
    books = codebooks(d)
    idx1, idx_up = unpack(codes, d)
    qr = q @ pi.T                                        # rows of Pi q
    phi = books[0][0][idx1]                              # [n, d/2]
    # [m, n, d/2]: level-1 partial sums of every query and key
    a = qr[:, None, 0::2] * np.cos(phi)[None] + qr[:, None, 1::2] * np.sin(phi)[None]
    off = 0
    for level in range(2, L + 1):
        cnt = d >> level
        psi = books[level - 1][0][idx_up[:, off:off + cnt]][None]    # [1, n, cnt]
        a = np.cos(psi) * a[:, :, 0::2] + np.sin(psi) * a[:, :, 1::2]
        off += cnt
    return scale * qz.from_fp16_bits(norm)[None, :] * a[:, :, 0]
