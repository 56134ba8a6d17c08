"""CPU checks of the C-ABI library: exports, host-side tables, argument errors.

No GPU compute is called: only host functions (codebook, rotation) and the
argument validation that runs before any launch.
"""

import ctypes
import os
import re

import numpy as np
import pytest

from oracle import codebook as ocb
from oracle import rotation as orot

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def tq():
    from online_vector_quantization_amd import build as b
    if not os.path.exists(b.LIB):
        b.build_library()
    import online_vector_quantization_amd as pkg
    return pkg


def test_exports_every_declared_symbol(tq):
    header = open(os.path.join(ROOT, "include", "tq.h")).read()
    declared = set(re.findall(r"^\s*(?:tq_status|const char \*)\s*(tq_\w+)\s*\(", header, re.M))
    assert {"tq_make_codebook", "tq_make_rotation", "tq_quantize_kv", "tq_attn_logits",
            "tq_dequantize"} <= declared
    for name in declared:
        assert hasattr(tq.LIB, name), name


@pytest.mark.parametrize("d", [16, 64, 128, 256])
def test_rotation_matches_oracle(tq, d):
    for kind, tol in ((0, 1e-13), (1, 1e-15), (2, 1e-12)):
        lib = tq.make_rotation(d, 0, kind)
        ref = orot.make_rotation(d, 0, kind)
        assert np.max(np.abs(lib - ref)) < tol * max(1.0, np.max(np.abs(ref)))
    p = tq.make_rotation(d, 7, 0)
    assert np.max(np.abs(p.T @ p - np.eye(d))) < 1e-10


def test_seed_streams_are_independent(tq):
    a = tq.make_rotation(32, 1, 1)
    b = tq.make_rotation(32, 2, 1)
    assert not np.allclose(a, b)
    # kind 1 of seed s and kind 0 of seed s share no stream: 2s+1 vs 2s
    assert not np.allclose(tq.make_rotation(32, 1, 1), orot.qjl_matrix(32, 0))


@pytest.mark.parametrize("d,bits", [(3, 1), (3, 2), (3, 3), (4, 2), (5, 3), (16, 3), (64, 2),
                                    (128, 1), (128, 2), (128, 3), (128, 4), (256, 2), (256, 4)])
def test_codebook_matches_oracle(tq, d, bits):
    c, t, mse = tq.make_codebook(d, bits)
    co, to, do = ocb.codebook(d, bits)
    assert np.max(np.abs(c - co)) < 1e-12
    assert np.max(np.abs(t - to)) < 1e-12
    assert mse == pytest.approx(do, rel=1e-10)
    assert np.all(c == -c[::-1])                  # exactly antisymmetric
    assert t[len(t) // 2] == 0.0


def test_host_argument_errors(tq):
    buf = np.zeros(300)
    lib = tq.LIB
    assert lib.tq_make_codebook(2, 3, buf.ctypes.data, buf.ctypes.data, None) == tq.TQ_ERR_INVALID
    assert lib.tq_make_codebook(128, 0, buf.ctypes.data, buf.ctypes.data, None) == tq.TQ_ERR_INVALID
    assert lib.tq_make_codebook(128, 9, buf.ctypes.data, buf.ctypes.data, None) == tq.TQ_ERR_INVALID
    assert lib.tq_make_codebook(128, 3, None, buf.ctypes.data, None) == tq.TQ_ERR_INVALID
    assert lib.tq_make_rotation(16, 0, 3, buf.ctypes.data) == tq.TQ_ERR_INVALID
    assert lib.tq_make_rotation(1, 0, 0, buf.ctypes.data) == tq.TQ_ERR_INVALID
    assert lib.tq_make_rotation(16, 0, 0, None) == tq.TQ_ERR_INVALID
    assert tq.status_string(tq.TQ_ERR_UNSUPPORTED) == "unsupported configuration"


def test_device_calls_validate_before_launch(tq):
    lib = tq.LIB
    dummy = ctypes.c_void_p(16)
    p = tq.Params(128, 3, tq.MODE_MSE, 0, dummy, None, None, dummy, dummy)
    pk = tq.Packed(dummy, dummy, None)
    # NULL params / bad bits / bad mode / reserved
    assert lib.tq_quantize_kv(None, dummy, 0, 1, 128, ctypes.byref(pk), 0, None) == tq.TQ_ERR_INVALID
    bad = tq.Params(128, 9, tq.MODE_MSE, 0, dummy, None, None, dummy, dummy)
    assert lib.tq_quantize_kv(ctypes.byref(bad), dummy, 0, 1, 128, ctypes.byref(pk), 0, None) == tq.TQ_ERR_INVALID
    bad = tq.Params(128, 1, tq.MODE_PROD, 0, dummy, dummy, dummy, dummy, dummy)
    assert lib.tq_quantize_kv(ctypes.byref(bad), dummy, 0, 1, 128, ctypes.byref(pk), 0, None) == tq.TQ_ERR_INVALID
    bad = tq.Params(128, 3, 7, 0, dummy, None, None, dummy, dummy)
    assert lib.tq_dequantize(ctypes.byref(bad), ctypes.byref(pk), 1, dummy, 0, None) == tq.TQ_ERR_INVALID
    bad = tq.Params(128, 3, tq.MODE_MSE, 1, dummy, None, None, dummy, dummy)
    assert lib.tq_dequantize(ctypes.byref(bad), ctypes.byref(pk), 1, dummy, 0, None) == tq.TQ_ERR_INVALID
    # bad dtype, negative sizes, stride < d, prod without QJL tables
    assert lib.tq_quantize_kv(ctypes.byref(p), dummy, 5, 1, 128, ctypes.byref(pk), 0, None) == tq.TQ_ERR_INVALID
    assert lib.tq_quantize_kv(ctypes.byref(p), dummy, 0, -1, 128, ctypes.byref(pk), 0, None) == tq.TQ_ERR_INVALID
    assert lib.tq_quantize_kv(ctypes.byref(p), dummy, 0, 4, 100, ctypes.byref(pk), 0, None) == tq.TQ_ERR_INVALID
    pp = tq.Params(128, 3, tq.MODE_PROD, 0, dummy, None, None, dummy, dummy)
    assert lib.tq_quantize_kv(ctypes.byref(pp), dummy, 0, 4, 128, ctypes.byref(pk), 0, None) == tq.TQ_ERR_INVALID
    # empty work is a no-op that touches nothing
    assert lib.tq_quantize_kv(ctypes.byref(p), None, 0, 0, 128, ctypes.byref(pk), 0, None) == tq.TQ_OK
    assert lib.tq_dequantize(ctypes.byref(p), ctypes.byref(pk), 0, None, 0, None) == tq.TQ_OK
    # logits: GQA divisibility, seq_len > row_tokens, top-k larger than seq_len
    f = ctypes.c_float(1.0)
    assert lib.tq_attn_logits(ctypes.byref(p), dummy, 0, 1, 6, 4, ctypes.byref(pk), 10, 10, f, dummy,
                              0, None, None) == tq.TQ_ERR_INVALID
    assert lib.tq_attn_logits(ctypes.byref(p), dummy, 0, 1, 4, 4, ctypes.byref(pk), 5, 10, f, dummy,
                              0, None, None) == tq.TQ_ERR_INVALID
    assert lib.tq_attn_logits(ctypes.byref(p), dummy, 0, 1, 4, 4, ctypes.byref(pk), 10, 5, f, dummy,
                              10, dummy, None) == tq.TQ_ERR_INVALID
    assert lib.tq_attn_logits(ctypes.byref(p), dummy, 0, 1, 4, 4, ctypes.byref(pk), 10, 0, f, dummy,
                              0, None, None) == tq.TQ_OK
    # misaligned input rows are refused, not read
    assert lib.tq_quantize_kv(ctypes.byref(p), ctypes.c_void_p(18), 1, 4, 128, ctypes.byref(pk), 0,
                              None) == tq.TQ_ERR_UNSUPPORTED
    # d without a kernel (prod at d = 256) is reported before any launch
    p256 = tq.Params(256, 3, tq.MODE_PROD, 0, dummy, dummy, dummy, dummy, dummy)
    pk2 = tq.Packed(dummy, dummy, dummy)
    assert lib.tq_quantize_kv(ctypes.byref(p256), dummy, 0, 1, 256, ctypes.byref(pk2), 0,
                              None) == tq.TQ_ERR_UNSUPPORTED


def test_polar_codebooks_match_oracle():
    """Angle codebooks of the polar format: the library (composite Gauss-Legendre
    and Lloyd iteration) against the oracle (incomplete beta and adaptive
    quadrature), levels 2..7 at d = 128."""
    import online_vector_quantization_amd as tq
    from oracle import polar as opq
    c, t = tq.make_polar_codebook(128)
    assert c.shape == (6, 4) and t.shape == (6, 3)
    for lv in range(2, 8):
        oc, ot = opq.angle_codebook(1 << (lv - 1))
        np.testing.assert_allclose(c[lv - 2], oc, rtol=0, atol=1e-12)
        np.testing.assert_allclose(t[lv - 2], ot, rtol=0, atol=1e-12)
    with pytest.raises(tq.TQError):
        tq.make_polar_codebook(96)
