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
            "tq_dequantize", "tq_attn_logits_workspace_size", "tq_attn_output_workspace_size"} <= declared
    assert declared == set(tq.EXPORTED)
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
    ws = ctypes.c_void_p(1 << 20)          # 256-byte aligned stand-in, never dereferenced here
    big = 1 << 30
    assert lib.tq_attn_logits(ctypes.byref(p), dummy, 0, 1, 6, 4, ctypes.byref(pk), 10, 10, f, dummy,
                              0, None, ws, big, None) == tq.TQ_ERR_INVALID
    assert lib.tq_attn_logits(ctypes.byref(p), dummy, 0, 1, 4, 4, ctypes.byref(pk), 5, 10, f, dummy,
                              0, None, ws, big, None) == tq.TQ_ERR_INVALID
    assert lib.tq_attn_logits(ctypes.byref(p), dummy, 0, 1, 4, 4, ctypes.byref(pk), 10, 5, f, dummy,
                              10, dummy, ws, big, None) == tq.TQ_ERR_INVALID
    assert lib.tq_attn_logits(ctypes.byref(p), dummy, 0, 1, 4, 4, ctypes.byref(pk), 10, 0, f, dummy,
                              0, None, None, 0, None) == tq.TQ_OK
    # misaligned input rows are refused, not read
    assert lib.tq_quantize_kv(ctypes.byref(p), ctypes.c_void_p(18), 1, 4, 128, ctypes.byref(pk), 0,
                              None) == tq.TQ_ERR_UNSUPPORTED
    # a d without kernels (96: neither 64, 128 nor 256) is reported before any launch
    pk2 = tq.Packed(dummy, dummy, dummy)
    for mode in (tq.MODE_MSE, tq.MODE_PROD):
        p96 = tq.Params(96, 3, mode, 0, dummy, dummy, dummy, dummy, dummy)
        assert lib.tq_quantize_kv(ctypes.byref(p96), dummy, 0, 1, 96, ctypes.byref(pk2), 0,
                                  None) == tq.TQ_ERR_UNSUPPORTED
        assert lib.tq_dequantize(ctypes.byref(p96), ctypes.byref(pk2), 1, dummy, 0,
                                 None) == tq.TQ_ERR_UNSUPPORTED
        assert lib.tq_attn_logits(ctypes.byref(p96), dummy, 0, 1, 4, 1, ctypes.byref(pk2), 64, 64, f, dummy,
                                  0, None, ws, big, None) == tq.TQ_ERR_UNSUPPORTED


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
    # d = 256 adds level 8 (k = 128); d = 64 stops at level 6
    c256, t256 = tq.make_polar_codebook(256)
    assert c256.shape == (7, 4) and np.array_equal(c256[:6], c)
    oc, ot = opq.angle_codebook(128)
    np.testing.assert_allclose(c256[6], oc, rtol=0, atol=1e-12)
    np.testing.assert_allclose(t256[6], ot, rtol=0, atol=1e-12)
    c64, _ = tq.make_polar_codebook(64)
    assert c64.shape == (5, 4) and np.array_equal(c64, c[:5])
    with pytest.raises(tq.TQError):
        tq.make_polar_codebook(96)


def _size(fn, *args):
    n = ctypes.c_size_t(7)
    st = fn(*args, ctypes.byref(n))
    return st, n.value


def test_workspace_queries_and_checks(tq):
    """Caller-owned scratch: the size queries, and the calls refuse a missing,
    short or misaligned workspace before any launch."""
    lib = tq.LIB
    dummy = ctypes.c_void_p(16)
    f = ctypes.c_float(1.0)
    pp = tq.Params(128, 3, tq.MODE_PROD, 0, dummy, dummy, dummy, dummy, dummy)
    pm = tq.Params(128, 3, tq.MODE_MSE, 0, dummy, None, None, dummy, dummy)
    pk = tq.Packed(dummy, dummy, dummy)
    # dense logits: query tables of every (batch, kv head) stream, independent of seq_len
    st, n8 = _size(lib.tq_attn_logits_workspace_size, ctypes.byref(pp), 1, 32, 8, 32768, 0)
    assert st == tq.TQ_OK and n8 > 0 and n8 % 256 == 0
    st, n64 = _size(lib.tq_attn_logits_workspace_size, ctypes.byref(pp), 8, 32, 8, 131072, 0)
    assert st == tq.TQ_OK and n64 >= 8 * n8 - 8 * 256
    assert _size(lib.tq_attn_logits_workspace_size, ctypes.byref(pp), 1, 32, 8, 5, 0) == (tq.TQ_OK, n8)
    assert _size(lib.tq_attn_logits_workspace_size, ctypes.byref(pp), 0, 32, 8, 5, 0) == (tq.TQ_OK, 0)
    assert _size(lib.tq_attn_logits_workspace_size, ctypes.byref(pp), 1, 32, 8, 0, 0) == (tq.TQ_OK, 0)
    assert _size(lib.tq_attn_logits_workspace_size, ctypes.byref(pp), 1, 30, 8, 5, 0)[0] == tq.TQ_ERR_INVALID
    assert lib.tq_attn_logits_workspace_size(ctypes.byref(pp), 1, 32, 8, 5, 0, None) == tq.TQ_ERR_INVALID
    # top-k search (MSE only): partial lists grow with the query count
    st, s1 = _size(lib.tq_attn_logits_workspace_size, ctypes.byref(pm), 1, 1000, 1, 100000, 10)
    st2, s2 = _size(lib.tq_attn_logits_workspace_size, ctypes.byref(pm), 1, 2000, 1, 100000, 10)
    assert st == st2 == tq.TQ_OK and 0 < s1 < s2
    assert _size(lib.tq_attn_logits_workspace_size, ctypes.byref(pp), 1, 4, 1, 100, 10)[0] == tq.TQ_ERR_UNSUPPORTED
    assert _size(lib.tq_attn_logits_workspace_size, ctypes.byref(pm), 1, 4, 1, 100, 17)[0] == tq.TQ_ERR_UNSUPPORTED
    # attention output: MSE only
    st, na = _size(lib.tq_attn_output_workspace_size, ctypes.byref(pm), 1, 32, 8, 32768)
    assert st == tq.TQ_OK and na > 0
    assert _size(lib.tq_attn_output_workspace_size, ctypes.byref(pm), 1, 32, 8, 0) == (tq.TQ_OK, 0)
    assert _size(lib.tq_attn_output_workspace_size, ctypes.byref(pp), 1, 32, 8, 100)[0] == tq.TQ_ERR_UNSUPPORTED
    # the calls: NULL / short workspace -> invalid, misaligned -> unsupported
    args = (ctypes.byref(pp), dummy, 0, 1, 32, 8, ctypes.byref(pk), 64, 64, f, dummy, 0, None)
    assert lib.tq_attn_logits(*args, None, 0, None) == tq.TQ_ERR_INVALID
    assert lib.tq_attn_logits(*args, ctypes.c_void_p(1 << 20), n8 - 1, None) == tq.TQ_ERR_INVALID
    assert lib.tq_attn_logits(*args, ctypes.c_void_p((1 << 20) + 16), n8, None) == tq.TQ_ERR_UNSUPPORTED
    app = (ctypes.byref(pp), dummy, 0, dummy, 0, 1, 32, 8, ctypes.byref(pk), 64, 10, f, dummy)
    assert lib.tq_append_attn_logits(*app, None, 0, None) == tq.TQ_ERR_INVALID
    sargs = (ctypes.byref(pm), dummy, 0, 1, 1000, 1, ctypes.byref(pk), 100000, 100000, f, dummy, 10, dummy)
    assert lib.tq_attn_logits(*sargs, None, 0, None) == tq.TQ_ERR_INVALID
    assert lib.tq_attn_logits(*sargs, ctypes.c_void_p(1 << 20), s1 - 1, None) == tq.TQ_ERR_INVALID
    assert lib.tq_attn_logits(*sargs, ctypes.c_void_p((1 << 20) + 16), s1, None) == tq.TQ_ERR_UNSUPPORTED
    pv = tq.Packed(ctypes.c_void_p(1 << 20), dummy, None)
    att = (ctypes.byref(pm), dummy, 1, 32, 8, ctypes.byref(pv), 32768, 32768, dummy, 0)
    assert lib.tq_attn_output(*att, None, 0, None) == tq.TQ_ERR_INVALID
    assert lib.tq_attn_output(*att, ctypes.c_void_p(1 << 20), na - 1, None) == tq.TQ_ERR_INVALID


def test_logit_ranges_stay_below_2_31(tq):
    """The streaming kernel drops lanes' stores through the byte offset 2^31,
    so one stream's logits (group x seq_len fp32) must stay below 2^31 bytes:
    larger calls are refused before any launch (no buffers needed)."""
    lib = tq.LIB
    dummy = ctypes.c_void_p(16)
    f = ctypes.c_float(1.0)
    for bits, mode, group in ((3, tq.MODE_PROD, 16), (1, tq.MODE_MSE, 8)):
        p = tq.Params(128, bits, mode, 0, dummy, dummy, dummy, dummy, dummy)
        pk = tq.Packed(dummy, dummy, dummy)
        limit = (1 << 31) // (4 * group)                  # tokens at which the logits reach 2^31 bytes
        assert _size(lib.tq_attn_logits_workspace_size, ctypes.byref(p), 1, group, 1, limit - 1, 0)[0] == tq.TQ_OK
        assert _size(lib.tq_attn_logits_workspace_size, ctypes.byref(p), 1, group, 1, limit, 0)[0] == \
            tq.TQ_ERR_UNSUPPORTED
        assert lib.tq_attn_logits(ctypes.byref(p), dummy, 0, 1, group, 1, ctypes.byref(pk), limit, limit, f,
                                  dummy, 0, None, ctypes.c_void_p(1 << 20), 1 << 30, None) == tq.TQ_ERR_UNSUPPORTED
        assert lib.tq_append_attn_logits(ctypes.byref(p), dummy, 0, dummy, 0, 1, group, 1, ctypes.byref(pk),
                                         limit, limit - 1, f, dummy, ctypes.c_void_p(1 << 20), 1 << 30,
                                         None) == tq.TQ_ERR_UNSUPPORTED


def test_noalloc_entry_validates_before_launch(tq):
    """tq_attn_output_noalloc: the same argument checks as tq_attn_output, and
    shapes whose partials exceed its fixed array are refused before any HIP
    call (the array's address is only looked up once a call is accepted)."""
    lib = tq.LIB
    dummy = ctypes.c_void_p(16)
    pm = tq.Params(256, 3, tq.MODE_MSE, 0, dummy, None, None, dummy, dummy)
    pv = tq.Packed(ctypes.c_void_p(1 << 20), dummy, None)
    st, need = _size(lib.tq_attn_output_workspace_size, ctypes.byref(pm), 64, 1024, 64, 256)
    assert st == tq.TQ_OK and need > tq.NOALLOC_SCRATCH_BYTES
    assert lib.tq_attn_output_noalloc(ctypes.byref(pm), dummy, 64, 1024, 64, ctypes.byref(pv), 256, 256, dummy, 0,
                                      None) == tq.TQ_ERR_UNSUPPORTED
    assert lib.tq_attn_output_noalloc(ctypes.byref(pm), dummy, 1, 6, 4, ctypes.byref(pv), 256, 256, dummy, 0,
                                      None) == tq.TQ_ERR_INVALID
    assert lib.tq_attn_output_noalloc(None, dummy, 1, 4, 4, ctypes.byref(pv), 256, 256, dummy, 0,
                                      None) == tq.TQ_ERR_INVALID
    pp = tq.Params(128, 3, tq.MODE_PROD, 0, dummy, dummy, dummy, dummy, dummy)
    assert lib.tq_attn_output_noalloc(ctypes.byref(pp), dummy, 1, 4, 4, ctypes.byref(pv), 256, 256, dummy, 0,
                                      None) == tq.TQ_ERR_UNSUPPORTED


def test_paged_calls_validate_before_launch(tq):
    lib = tq.LIB
    dummy = ctypes.c_void_p(16)
    f = ctypes.c_float(1.0)
    pp = tq.Params(128, 3, tq.MODE_PROD, 0, dummy, dummy, dummy, dummy, dummy)
    pk = tq.Packed(dummy, dummy, dummy)

    ws = ctypes.c_void_p(1 << 20)

    def call(pages, seq_len=1000):
        return lib.tq_attn_logits_paged(ctypes.byref(pp), dummy, 0, 1, 32, 8, ctypes.byref(pk),
                                        ctypes.byref(pages) if pages is not None else None, seq_len, f, dummy,
                                        ws, 1 << 30, None)

    assert call(None) == tq.TQ_ERR_INVALID
    assert call(tq.Pages(None, 64, 16, 100)) == tq.TQ_ERR_INVALID                  # no table
    assert call(tq.Pages(dummy, 48, 32, 100)) == tq.TQ_ERR_INVALID                 # page not a multiple of 64
    assert call(tq.Pages(dummy, 64, 15, 100)) == tq.TQ_ERR_INVALID                 # 1000 tokens > 15 pages of 64
    assert call(tq.Pages(dummy, 64, 16, 0)) == tq.TQ_ERR_INVALID                   # empty pool
    assert call(tq.Pages(dummy, 256, 16, 1 << 20)) == tq.TQ_ERR_UNSUPPORTED        # pool codes past 2^31 bytes
    assert call(tq.Pages(dummy, 64, 16, 100), seq_len=0) == tq.TQ_OK                # empty: no-op
    app = lib.tq_append_attn_logits_paged
    pg = tq.Pages(dummy, 64, 16, 100)
    assert app(ctypes.byref(pp), dummy, 0, dummy, 0, 1, 32, 8, ctypes.byref(pk), ctypes.byref(pg), 1024, f, dummy,
               ws, 1 << 30, None) == tq.TQ_ERR_INVALID                              # pos 1024: past 16 pages of 64
    assert app(ctypes.byref(pp), dummy, 0, dummy, 0, 1, 32, 8, ctypes.byref(pk), ctypes.byref(pg), -1, f, dummy,
               ws, 1 << 30, None) == tq.TQ_ERR_INVALID



def test_prepared_calls_validate_before_launch(tq):
    """tq_prepare_queries / tq_attn_logits_prepared: bad arguments, short or
    misaligned workspaces, unsupported shapes and bad pages are refused
    before any launch; empty calls are no-ops."""
    lib = tq.LIB
    dummy = ctypes.c_void_p(16)
    f = ctypes.c_float(1.0)
    pp = tq.Params(128, 3, tq.MODE_PROD, 0, dummy, dummy, dummy, dummy, dummy)
    pk = tq.Packed(dummy, dummy, dummy)
    need = ctypes.c_size_t(0)
    assert lib.tq_attn_logits_workspace_size(ctypes.byref(pp), 2, 32, 8, 1, 0, ctypes.byref(need)) == tq.TQ_OK
    ws = ctypes.c_void_p(1 << 20)

    def prep(batch=2, hq=32, hkv=8, q=dummy, dt=0, w=ws, nb=need.value, params=pp):
        return lib.tq_prepare_queries(ctypes.byref(params), q, dt, batch, hq, hkv, w, nb, None)

    assert prep(hq=30) == tq.TQ_ERR_INVALID                       # heads not a multiple of KV heads
    assert prep(batch=-1) == tq.TQ_ERR_INVALID
    assert prep(dt=7) == tq.TQ_ERR_INVALID
    assert prep(q=None) == tq.TQ_ERR_INVALID
    assert prep(nb=need.value - 1) == tq.TQ_ERR_INVALID           # short workspace
    assert prep(w=None) == tq.TQ_ERR_INVALID
    assert prep(w=ctypes.c_void_p((1 << 20) + 64)) == tq.TQ_ERR_UNSUPPORTED   # misaligned
    assert prep(hq=136) == tq.TQ_ERR_UNSUPPORTED                  # 17 query heads per KV head
    assert prep(batch=0, q=None, w=None, nb=0) == tq.TQ_OK        # empty: no-op
    polar = tq.Params(128, 3, tq.MODE_POLAR, 0, dummy, dummy, dummy, dummy, dummy)
    assert prep(params=polar) == tq.TQ_ERR_UNSUPPORTED
    no_s = tq.Params(128, 3, tq.MODE_PROD, 0, dummy, None, dummy, dummy, dummy)
    assert prep(params=no_s) == tq.TQ_ERR_INVALID

    def run(batch=2, hq=32, hkv=8, k=pk, row_tokens=4096, pages=None, seq_len=4096, out=dummy, w=ws,
            nb=need.value):
        return lib.tq_attn_logits_prepared(ctypes.byref(pp), batch, hq, hkv, ctypes.byref(k) if k else None,
                                           row_tokens, ctypes.byref(pages) if pages is not None else None,
                                           seq_len, f, out, w, nb, None)

    assert run(k=None) == tq.TQ_ERR_INVALID
    assert run(row_tokens=4095) == tq.TQ_ERR_INVALID              # seq_len past the stream's rows
    assert run(out=None) == tq.TQ_ERR_INVALID
    assert run(nb=need.value - 1) == tq.TQ_ERR_INVALID
    assert run(k=tq.Packed(dummy, dummy, None)) == tq.TQ_ERR_INVALID   # inner-product keys need rnorm
    assert run(k=tq.Packed(ctypes.c_void_p(18), dummy, dummy)) == tq.TQ_ERR_UNSUPPORTED   # codes not 4-byte aligned
    assert run(seq_len=0, out=None, w=None, nb=0) == tq.TQ_OK
    assert run(batch=0, out=None, w=None, nb=0) == tq.TQ_OK
    assert run(pages=tq.Pages(dummy, 48, 64, 100)) == tq.TQ_ERR_INVALID          # page not a multiple of 64
    assert run(pages=tq.Pages(dummy, 64, 63, 100)) == tq.TQ_ERR_INVALID          # 4096 tokens > 63 pages of 64
    assert run(pages=tq.Pages(dummy, 256, 16, 1 << 20)) == tq.TQ_ERR_UNSUPPORTED  # pool codes past 2^31 bytes
    assert run(row_tokens=0, pages=tq.Pages(dummy, 64, 64, 100), seq_len=0, out=None, w=None, nb=0) == tq.TQ_OK


def test_polar_logit_shapes_and_workspace(tq):
    """Polar-format keys: dense logits take d in {64, 128, 256} and GQA groups
    up to 16; the workspace holds the rotated queries (fp32) and the cos/sin
    table of the centroid angles; top-k is refused."""
    lib = tq.LIB
    dummy = ctypes.c_void_p(16)

    def size(d, batch=2, hq=32, hkv=8, seq=4096, topk=0):
        pp = tq.Params(d, 3, tq.MODE_POLAR, 0, dummy, None, None, dummy, dummy)
        n = ctypes.c_size_t(0)
        st = lib.tq_attn_logits_workspace_size(ctypes.byref(pp), batch, hq, hkv, seq, topk, ctypes.byref(n))
        return st, n.value

    def al(x):
        return (x + 255) // 256 * 256

    for d, levels in ((64, 6), (128, 7), (256, 8)):
        st, n = size(d)
        assert st == tq.TQ_OK and n == al(16 * 4 * d * 4) + al((16 + 4 * (levels - 1)) * 8)
    assert size(128, hq=8 * 17)[0] == tq.TQ_ERR_UNSUPPORTED        # 17 query heads per KV head
    assert size(96)[0] == tq.TQ_ERR_UNSUPPORTED
    assert size(128, topk=10)[0] == tq.TQ_ERR_UNSUPPORTED
    assert size(128, seq=0) == (tq.TQ_OK, 0)
    # logits of one stream past 2^31 bytes
    assert size(128, batch=1, hq=16, hkv=1, seq=1 << 25)[0] == tq.TQ_ERR_UNSUPPORTED


def test_probe_calls_validate_before_launch(tq):
    """tq_probe refuses bad kinds, short sinks, unaligned or empty stream
    buffers and out-of-range loop counts before any launch."""
    lib = tq.LIB
    words = ctypes.c_int64(0)
    assert lib.tq_probe_sink_words(ctypes.byref(words)) == tq.TQ_OK and words.value > 0
    assert lib.tq_probe_sink_words(None) == tq.TQ_ERR_INVALID
    sink = ctypes.c_void_p(1 << 20)
    buf = ctypes.c_void_p(1 << 24)
    n = words.value

    def probe(kind, b=buf, nbytes=1 << 20, iters=1, s=sink, sw=n):
        return lib.tq_probe(kind, b, nbytes, iters, s, sw, None)

    assert probe(-1) == tq.TQ_ERR_INVALID
    assert probe(tq.PROBE_MFMA_I8 + 1) == tq.TQ_ERR_INVALID
    assert probe(tq.PROBE_READ, s=None) == tq.TQ_ERR_INVALID
    assert probe(tq.PROBE_READ, sw=n - 1) == tq.TQ_ERR_INVALID
    assert probe(tq.PROBE_READ, b=None) == tq.TQ_ERR_INVALID
    assert probe(tq.PROBE_WRITE, nbytes=24) == tq.TQ_ERR_INVALID
    assert probe(tq.PROBE_WRITE, b=ctypes.c_void_p((1 << 24) + 8)) == tq.TQ_ERR_INVALID
    assert probe(tq.PROBE_MFMA_F16, iters=0) == tq.TQ_ERR_INVALID
    assert probe(tq.PROBE_MFMA_I8, iters=-3) == tq.TQ_ERR_INVALID
