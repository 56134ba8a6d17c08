"""Shared helpers of the GPU parity tests: oracle tables, tolerance rules.

Tolerance rules:
* codes (the per-coordinate records): Lloyd-Max indices bit-exact, except
  coordinates whose oracle value u = y/n lies within
  1e-5 of a decision boundary; those are counted and must stay under 0.01%
  of all coordinates.  QJL sign bits the same with value z/gamma and
  boundary 0, on the rows whose Lloyd-Max indices equal the oracle's: the
  signs sketch the residual of the chosen index, so a row where a
  near-boundary index legitimately went the other way has a different
  residual and its signs are not comparable (such rows are counted).
* norm: bit-exact fp16.
* rnorm (fp16 of gamma), on the rows whose Lloyd-Max indices equal the
  oracle's: bit-exact, except rows whose oracle gamma lies within a relative
  window RNORM_WINDOW = 2^-20 of the rounding midpoint between the oracle's
  fp16 value and the GPU's (the GPU rounded to the other neighbour of that
  midpoint); such flips are counted and number at most MAX_RNORM_FLIP_FRAC =
  0.05% of the compared rows (at least one allowed).  Derivation: the device
  forms gamma from the fp32 rotation (fp32 accumulation of 22-bit products),
  the correctly rounded fp32 1/||x|| (a common factor of the vector) and
  fp32 sums of the staged residual; emulating those roundings gives a
  relative error of gamma of std 5e-8 (b' = 2) to 8e-8 (b' = 3), largest
  4e-7 in 2e4 vectors, so the window is over twice the largest error.  A
  flip needs the error to reach past the midpoint: with fp16 midpoints
  2^-11..2^-10 apart (relative) the expected flip rate is about
  2 E|err| / 2^-10.5 = 0.013% to 0.017%, and the bound allows three times
  that.
* a row whose packed record (codes and rnorm) differs from the oracle's
  carries at least one of the counted mismatches above; ``check_records``
  asserts that and returns the mask of identical rows, on which logits and
  reconstructions are then compared.
* logits from identical (oracle-packed) codes: |l_gpu - l_orc| <= 1e-4 *
  max(|l_orc|, 1e-2 * |scale| * n16 * ||q||).
* dequantize: ||x_gpu - x_orc|| <= 1e-4 ||x_orc|| per vector (fp32 output).
* polar format: angle indices bit-exact except angles within 1e-5 rad of a
  cell boundary (level-1 angles also within 1e-6 / rho of it, rho the pair's
  radius: the angle of a small pair moves by the coordinates' error over
  rho), each off by one cell; fewer than 0.01% of the angles.
"""

import numpy as np
import torch

from oracle import codebook as ocb
from oracle import quantizer as oqz
from oracle import rotation as orot

CODE_WINDOW = 1e-5
MAX_MISMATCH_FRAC = 1e-4
RNORM_WINDOW = 2.0 ** -20
MAX_RNORM_FLIP_FRAC = 5e-4
LOGIT_RTOL = 1e-4
LOGIT_FLOOR = 1e-2
DEQUANT_RTOL = 1e-4


class OracleTables:
    def __init__(self, d, bits, mode, seed=0):
        self.d, self.bits, self.mode = d, bits, mode
        self.lb = oqz.lloyd_bits(bits, mode)
        self.c, self.t, self.dist = ocb.codebook(d, self.lb)
        self.pi = orot.haar_rotation(d, seed)
        self.s = orot.qjl_matrix(d, seed) if mode == oqz.MODE_PROD else None

    def quantize(self, x64):
        return oqz.quantize(x64, self.pi, self.c, self.t, self.mode, s_mat=self.s)


def dev_u16(arr, device):
    return torch.from_numpy(np.ascontiguousarray(arr).view(np.int16)).to(device)


def dev_bf16(bits, device):
    return dev_u16(bits, device).view(torch.bfloat16)


def cache_from_oracle(tq, ref, d, bits, mode, device):
    return tq.PackedKV.from_tensors(
        d, bits, mode, torch.from_numpy(ref["codes"]).to(device), dev_u16(ref["norm"], device),
        dev_u16(ref["rnorm"], device) if ref["rnorm"] is not None else None)


def check_codes(gpu_codes, ref, lb, d, t, mode=oqz.MODE_MSE):
    """Codes rule; returns (mismatched coordinates, total coordinates)."""
    g, _ = oqz.unpack_records(gpu_codes, lb, mode, d)
    o = ref["idx"]
    bad = g != o
    n_bad = int(bad.sum())
    if n_bad:
        u = ref["u_rot"][bad]
        dist = np.min(np.abs(u[:, None] - t[None, :]), axis=1)
        assert np.all(dist < CODE_WINDOW), "mismatch far from a boundary: %g" % dist.max()
        assert np.all(np.abs(g[bad] - o[bad]) == 1)
    assert n_bad <= MAX_MISMATCH_FRAC * o.size, "%d of %d codes differ" % (n_bad, o.size)
    return n_bad, o.size


def check_signs(gpu_codes, ref, lb, d):
    """Sign rule on rows with identical Lloyd-Max indices; returns (mismatched
    signs, rows skipped because an index differs)."""
    gi, gs = oqz.unpack_records(gpu_codes, lb, oqz.MODE_PROD, d)
    rows = np.all(gi == ref["idx"], axis=1)
    g = gs.astype(bool)[rows]
    o = ref["sign_bits"][rows]
    bad = g != o
    n_bad = int(bad.sum())
    if n_bad:
        gam = np.where(ref["gamma"][rows] > 0, ref["gamma"][rows], 1.0)
        zr = np.abs(ref["z"][rows] / gam[:, None])[bad]
        assert np.all(zr < CODE_WINDOW), "sign mismatch far from 0: %g" % zr.max()
    assert n_bad <= MAX_MISMATCH_FRAC * max(o.size, 1), "%d of %d signs differ" % (n_bad, o.size)
    return n_bad, int(np.sum(~rows))


def check_norms(gpu_norm, ref):
    g = np.asarray(gpu_norm).view(np.uint16)
    assert np.array_equal(g, ref["norm"]), "norm differs in %d rows" % int(np.sum(g != ref["norm"]))


def allowed_mismatches(total, frac=MAX_MISMATCH_FRAC):
    return max(1, int(np.ceil(frac * total)))


def rnorm_flip_distance(gamma, oracle_bits, gpu_bits):
    """Relative distance of the oracle's fp64 gamma to the midpoint between
    the oracle's fp16 value and the GPU's (the rounding point the two sides
    fell on either side of); infinite where that is not a rounding flip."""
    o = oqz.from_fp16_bits(oracle_bits)
    g = oqz.from_fp16_bits(gpu_bits)
    adjacent = np.abs(np.asarray(oracle_bits, np.int64) - np.asarray(gpu_bits, np.int64)) == 1
    mid = 0.5 * (o + g)
    with np.errstate(divide="ignore", invalid="ignore"):
        dist = np.abs(gamma - mid) / gamma
    return np.where(adjacent & (gamma > 0) & np.isfinite(dist), dist, np.inf)


def check_rnorm(gpu_rnorm, ref, rows=None):
    """rnorm rule on the rows selected by ``rows`` (default: all); returns the
    number of counted flips."""
    g = np.asarray(gpu_rnorm).view(np.uint16)
    o = ref["rnorm"]
    gam = ref["gamma"]
    if rows is not None:
        g, o, gam = g[rows], o[rows], gam[rows]
    bad = g != o
    n_bad = int(bad.sum())
    if n_bad:
        dist = rnorm_flip_distance(gam[bad], o[bad], g[bad])
        assert np.all(dist < RNORM_WINDOW), "rnorm differs beyond a rounding flip: %.3g" % dist.max()
    assert n_bad <= allowed_mismatches(g.size, MAX_RNORM_FLIP_FRAC), "%d of %d rnorm values differ" % (n_bad, g.size)
    return n_bad


def check_records(gpu_codes, gpu_norm, gpu_rnorm, ref, ot, report=None):
    """Every per-vector rule (codes, signs, norm, rnorm) on a block of rows.

    Returns the mask of rows whose packed record (code row and rnorm) equals
    the oracle's.  Every other row must carry a counted mismatch that its rule
    accepted: a Lloyd-Max index within the boundary window, a sign within the
    window of 0, or an rnorm flip next to a rounding midpoint.  ``report``
    (a dict) receives the counts.
    """
    gpu_codes = np.asarray(gpu_codes)
    n_code, _ = check_codes(gpu_codes, ref, ot.lb, ot.d, ot.t, ot.mode)
    check_norms(gpu_norm, ref)
    gi, gs = oqz.unpack_records(gpu_codes, ot.lb, ot.mode, ot.d)
    idx_ok = np.all(gi == ref["idx"], axis=1)
    same = np.all(gpu_codes == ref["codes"], axis=1)
    counts = {"rows": int(len(gpu_codes)), "code_mismatches": n_code, "rows_index_mismatch": int(np.sum(~idx_ok))}
    explained = ~idx_ok
    if ot.mode == oqz.MODE_PROD:
        n_sign, _ = check_signs(gpu_codes, ref, ot.lb, ot.d)
        n_rn = check_rnorm(gpu_rnorm, ref, rows=idx_ok)
        rn_diff = np.asarray(gpu_rnorm).view(np.uint16) != ref["rnorm"]
        same &= ~rn_diff
        sign_diff = np.any(gs.astype(bool) != ref["sign_bits"], axis=1)
        explained = explained | (idx_ok & (sign_diff | rn_diff))
        counts.update(sign_mismatches=n_sign, rnorm_flips=n_rn)
    unexplained = ~same & ~explained
    assert not unexplained.any(), "%d rows differ without a counted mismatch" % int(unexplained.sum())
    counts["rows_differing"] = int(np.sum(~same))
    if report is not None:
        report.update(counts)
    print("record parity:", counts)
    return same


def logit_floor(scale, norm16, q):
    qn = np.linalg.norm(np.asarray(q, dtype=np.float64), axis=-1)
    return LOGIT_FLOOR * abs(scale) * oqz.from_fp16_bits(norm16)[None, :] * qn[:, None]


def check_logits(gpu, want, scale, norm16, q):
    """gpu/want: [H, T] for queries q [H, d] over keys with fp16 norms norm16 [T]."""
    den = np.maximum(np.abs(want), logit_floor(scale, norm16, q))
    err = np.abs(np.asarray(gpu, dtype=np.float64) - want) / den
    assert err.max() <= LOGIT_RTOL, "logit error %.3g" % err.max()
    return float(err.max())


def check_dequant(gpu, want):
    num = np.linalg.norm(np.asarray(gpu, dtype=np.float64) - want, axis=1)
    den = np.maximum(np.linalg.norm(want, axis=1), 1e-30)
    rel = np.where(np.linalg.norm(want, axis=1) > 0, num / den, num)
    assert rel.max() <= DEQUANT_RTOL, "dequant error %.3g" % rel.max()
    return float(rel.max())


# polar format: angle windows
POLAR_ANGLE_WINDOW = 1e-5      # radians, plus the conditioning of a small pair
POLAR_PAIR_EPS = 1e-6          # absolute error of a rotated unit coordinate


def check_polar_codes(gpu_codes, ref, d):
    """Angle indices bit-exact except angles within the window of a cell
    boundary (level 1 also at 0 = 2 pi), off by one cell; fewer than 0.01%."""
    from oracle import polar as opq
    g1, gu = opq.unpack(gpu_codes, d)
    y = ref["y"]
    rho = np.hypot(y[:, 0::2], y[:, 1::2])
    bad1 = g1 != ref["idx1"]
    if bad1.any():
        phi = ref["phi"][bad1]
        bnd = 2 * np.pi * np.arange(17) / 16                 # includes 0 and 2 pi
        dist = np.min(np.abs(phi[:, None] - bnd[None, :]), axis=1)
        win = POLAR_ANGLE_WINDOW + POLAR_PAIR_EPS / np.maximum(rho[bad1], 1e-30)
        assert np.all(dist < win), "level-1 mismatch far from a boundary: %g" % (dist / win).max()
        step = (g1[bad1] - ref["idx1"][bad1]) % 16
        assert np.all((step == 1) | (step == 15))
    badu = gu != ref["idx_up"]
    if badu.any():
        books = opq.codebooks(d)
        psi_all = np.concatenate(ref["psis"], axis=1)
        lv_of = np.concatenate([np.full(p.shape[1], lv) for lv, p in enumerate(ref["psis"], start=2)])
        rows, cols = np.nonzero(badu)
        for r, c in zip(rows, cols):
            t = books[lv_of[c] - 1][1]
            assert np.min(np.abs(psi_all[r, c] - t)) < POLAR_ANGLE_WINDOW, "upper-level mismatch far from a boundary"
            assert abs(int(gu[r, c]) - int(ref["idx_up"][r, c])) == 1
    n_bad = int(bad1.sum() + badu.sum())
    total = g1.size + gu.size
    assert n_bad <= 1e-4 * total, "%d of %d angle indices differ" % (n_bad, total)
    return n_bad
