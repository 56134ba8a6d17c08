"""Random rotation Pi, QJL matrix S and the rotated-domain QJL matrix M.

Page "TurboQuant 설명", section "1단계: 무작위 회전 + PolarQuant 압축": every
vector goes through one data-independent random orthogonal transform obtained
from the QR factorisation of a Gaussian matrix.  Section "2단계: QJL 잔차
보정": the residual is sketched with a Gaussian (Johnson-Lindenstrauss)
projection and only the sign of each projected coordinate is kept.

Readings:
* Pi = Q diag(sign R_ii) with sign(0) = +1, where G = QR and G is the seeded
  Gaussian matrix of kind 0.  The sign fix makes Pi Haar distributed
  (F. Mezzadri, "How to generate random matrices from the classical compact
  groups", Notices AMS 54, 2007); without it the Beta law of the rotated
  coordinates would not hold exactly.  The rotation is applied as y = Pi x.
* S is the m x d Gaussian matrix of kind 1 with m = d rows (no QR).
* M = S Pi^T, so that S r = M (Pi r) for any residual r.
"""

import numpy as np

from .splitmix import gaussian_matrix

KIND_PI = 0
KIND_S = 1
KIND_M = 2


def haar_rotation(d, seed):
    """d x d Haar-orthogonal Pi from the seeded Gaussian matrix (fp64)."""
    g = gaussian_matrix(d, d, seed, KIND_PI)
    q, r = np.linalg.qr(g)
    sgn = np.where(np.diag(r) < 0.0, -1.0, 1.0)
    return q * sgn[None, :]


def qjl_matrix(d, seed):
    """m x d (m = d) i.i.d. N(0,1) QJL projection S (fp64)."""
    return gaussian_matrix(d, d, seed, KIND_S)


def qjl_rotated(d, seed):
    """M = S Pi^T: the QJL projection expressed in the rotated domain."""
    return qjl_matrix(d, seed) @ haar_rotation(d, seed).T


def make_rotation(d, seed, kind):
    """Dispatch on kind: 0 -> Pi, 1 -> S, 2 -> M."""
    if kind == KIND_PI:
        return haar_rotation(d, seed)
    if kind == KIND_S:
        return qjl_matrix(d, seed)
    if kind == KIND_M:
        return qjl_rotated(d, seed)
    raise ValueError("kind must be 0, 1 or 2")
