"""SplitMix64 and the Gaussian streams that feed the rotation and QJL matrices.

The page ("TurboQuant 설명", section "1단계: 무작위 회전 + PolarQuant 압축")
only says the rotation comes from the QR factorisation of a Gaussian matrix,
and section "2단계: QJL 잔차 보정" uses a Gaussian projection.  It fixes no
generator.  The reading adopted:

* generator: SplitMix64 (G. Steele, D. Lea, C. Flood, "Fast splittable
  pseudorandom number generators", OOPSLA 2014): the state advances by the
  odd constant 0x9E3779B97F4A7C15 and each output is the state passed through
  two xor-shift-multiply rounds and a final xor-shift;
* initial state for matrix kind k (0 = rotation, 1 = QJL) and user seed s:
  2*s + k (mod 2**64), so one seed gives independent Pi and S;
* uniform in (0, 1]: ((w >> 11) + 0.5) * 2**-53;
* normals: Box-Muller pairs sqrt(-2 ln v1) * (cos 2 pi v2, sin 2 pi v2),
  consumed in order, filling the matrix row-major.

Pure Python integers: slow but obviously correct.
"""

import math

import numpy as np

MASK64 = (1 << 64) - 1
GOLDEN_GAMMA = 0x9E3779B97F4A7C15
MIX1 = 0xBF58476D1CE4E5B9
MIX2 = 0x94D049BB133111EB


def splitmix64_stream(state, count):
    """Return ``count`` successive SplitMix64 outputs starting from ``state``."""
    out = []
    s = state & MASK64
    for _ in range(count):
        s = (s + GOLDEN_GAMMA) & MASK64
        z = s
        z = ((z ^ (z >> 30)) * MIX1) & MASK64
        z = ((z ^ (z >> 27)) * MIX2) & MASK64
        out.append(z ^ (z >> 31))
    return out


def uniforms(state, count):
    """Uniform doubles in (0, 1] from the top 53 bits of each output."""
    return [((w >> 11) + 0.5) * 2.0 ** -53 for w in splitmix64_stream(state, count)]


def normals(state, count):
    """Standard normals by Box-Muller, two per pair of uniforms, in order."""
    npairs = (count + 1) // 2
    v = uniforms(state, 2 * npairs)
    out = []
    for p in range(npairs):
        v1, v2 = v[2 * p], v[2 * p + 1]
        rad = math.sqrt(-2.0 * math.log(v1))
        ang = 2.0 * math.pi * v2
        out.append(rad * math.cos(ang))
        out.append(rad * math.sin(ang))
    return out[:count]


def stream_state(seed, kind):
    """Initial SplitMix64 state of matrix ``kind`` for user ``seed``."""
    return (2 * seed + kind) & MASK64


def gaussian_matrix(rows, cols, seed, kind):
    """rows x cols matrix of i.i.d. N(0,1), filled row-major (fp64)."""
    z = normals(stream_state(seed, kind), rows * cols)
    return np.array(z, dtype=np.float64).reshape(rows, cols)
