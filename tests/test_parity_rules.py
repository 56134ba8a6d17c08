"""The GPU parity rules themselves (tests/parity.py), exercised on the CPU.

Each rule must accept the deviations it is meant to allow (a rounding flip
next to an fp16 midpoint, an index next to a boundary) and reject every other
one; the mistakes are planted in copies of the oracle's own outputs.
"""

import numpy as np
import pytest

from oracle import quantizer as oqz
from parity import (MAX_RNORM_FLIP_FRAC, RNORM_WINDOW, OracleTables, allowed_mismatches, check_records,
                    check_rnorm, rnorm_flip_distance)


@pytest.fixture(scope="module")
def prod_case():
    ot = OracleTables(64, 3, oqz.MODE_PROD)
    x = np.random.default_rng(9).standard_normal((400, 64)) * 2.0
    x[5] = 0.0
    return ot, ot.quantize(x)


def _flip_toward_midpoint(ref, row, rel):
    """Move the oracle's gamma of ``row`` to a relative distance ``rel`` above
    the midpoint below its fp16 value; returns the fp16 bits one ulp down."""
    h = oqz.from_fp16_bits(ref["rnorm"][row])
    lo = np.nextafter(np.float16(h), np.float16(0)).astype(np.float64)
    mid = 0.5 * (h + lo)
    ref["gamma"][row] = mid * (1.0 + rel)
    ref["rnorm"][row] = oqz.to_fp16_bits(ref["gamma"][row])
    return ref["rnorm"][row] - 1


def test_rnorm_flip_inside_window_is_counted(prod_case):
    ot, ref0 = prod_case
    ref = {k: (v.copy() if isinstance(v, np.ndarray) else v) for k, v in ref0.items()}
    gpu = ref["rnorm"].copy()
    gpu[17] = _flip_toward_midpoint(ref, 17, 0.25 * RNORM_WINDOW)
    assert check_rnorm(gpu.view(np.int16), ref) == 1


@pytest.mark.parametrize("plant", ["far_from_midpoint", "two_ulp", "zero_gamma", "wrong_side"])
def test_rnorm_rule_rejects(prod_case, plant):
    ot, ref0 = prod_case
    ref = {k: (v.copy() if isinstance(v, np.ndarray) else v) for k, v in ref0.items()}
    gpu = ref["rnorm"].copy()
    if plant == "far_from_midpoint":
        gpu[17] = _flip_toward_midpoint(ref, 17, 4.0 * RNORM_WINDOW)
    elif plant == "two_ulp":
        gpu[17] = ref["rnorm"][17] + 2
    elif plant == "zero_gamma":
        gpu[5] = 1
    else:      # gamma just above the lower midpoint, GPU one ulp up (crossing nothing)
        _flip_toward_midpoint(ref, 17, 0.25 * RNORM_WINDOW)
        gpu[17] = ref["rnorm"][17] + 1
    with pytest.raises(AssertionError):
        check_rnorm(gpu.view(np.int16), ref)


def test_rnorm_count_bound(prod_case):
    ot, ref0 = prod_case
    ref = {k: (v.copy() if isinstance(v, np.ndarray) else v) for k, v in ref0.items()}
    gpu = ref["rnorm"].copy()
    rows = [r for r in range(20, 400) if ref["gamma"][r] > 0][:allowed_mismatches(400, MAX_RNORM_FLIP_FRAC) + 1]
    for r in rows:
        gpu[r] = _flip_toward_midpoint(ref, r, 0.1 * RNORM_WINDOW)
    with pytest.raises(AssertionError):
        check_rnorm(gpu.view(np.int16), ref)


def test_flip_distance_of_exact_midpoint():
    g = np.array([0.3])
    b = oqz.to_fp16_bits(g)
    d_up = rnorm_flip_distance(g, b, b + 1)
    assert np.isfinite(d_up[0]) and d_up[0] > RNORM_WINDOW
    assert np.isinf(rnorm_flip_distance(g, b, b + 3)[0])


def test_records_identical_and_planted(prod_case):
    ot, ref = prod_case
    same = check_records(ref["codes"], ref["norm"].view(np.int16), ref["rnorm"].view(np.int16), ref, ot)
    assert same.all()
    # an index far from any boundary flipped: rejected
    codes = ref["codes"].copy()
    u = ref["u_rot"][3]
    j = int(np.argmax(np.min(np.abs(u[:, None] - ot.t[None, :]), axis=1)))
    codes[3, 4 * (ot.bits * (j // 32)) + (j % 32) // 8] ^= np.uint8(1 << (j % 8))    # bit 0 of idx_j
    with pytest.raises(AssertionError):
        check_records(codes, ref["norm"].view(np.int16), ref["rnorm"].view(np.int16), ref, ot)
    # a norm that differs: rejected
    norm = ref["norm"].copy()
    norm[9] += 1
    with pytest.raises(AssertionError):
        check_records(ref["codes"], norm.view(np.int16), ref["rnorm"].view(np.int16), ref, ot)
