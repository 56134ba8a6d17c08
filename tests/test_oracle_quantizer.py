"""Pins for quantise / pack / dequantise / logits / top-k of the oracle."""

import itertools
import json
import math
import os

import numpy as np
import pytest

from oracle import codebook as cb
from oracle import quantizer as qz
from oracle import rotation as rot

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "worked_example.json")


def _golden():
    with open(GOLDEN) as f:
        return json.load(f)


def test_worked_example_mse():
    g = _golden()
    e = g["mse_b2"]
    c, t, _ = cb.codebook(3, 2)
    assert np.allclose(c, e["centroids"], atol=1e-14) and np.allclose(t, e["boundaries"], atol=1e-14)
    out = qz.quantize(np.array([g["x"]]), np.eye(3), c, t, qz.MODE_MSE)
    assert out["idx"].tolist() == [e["idx"]]
    assert out["codes"].tolist() == [e["codes"]]
    assert out["norm"].tolist() == [e["norm_fp16_bits"]]
    assert np.allclose(out["u_rot"], [e["u_rot"]], atol=1e-15)
    xh = qz.dequantize(out["codes"], out["norm"], np.eye(3), c, qz.MODE_MSE)
    assert np.allclose(xh, [e["x_hat"]], atol=1e-14)
    lg = qz.logits_rotated(np.array([g["q"]]), out["codes"], out["norm"], np.eye(3), c,
                           qz.MODE_MSE, g["scale"])
    assert lg[0, 0] == pytest.approx(e["logit"], abs=1e-14)


def test_worked_example_prod():
    g = _golden()
    e = g["prod_b3"]
    c, t, _ = cb.codebook(3, 2)
    out = qz.quantize(np.array([g["x"]]), np.eye(3), c, t, qz.MODE_PROD, s_mat=np.eye(3))
    assert out["idx"].tolist() == [e["idx"]]
    assert out["codes"].tolist() == [e["codes"]]
    assert out["sign_bits"].astype(int).tolist() == [e["sign_bits"]]
    assert out["gamma"][0] == pytest.approx(e["gamma"], rel=1e-15)
    assert out["rnorm"].tolist() == [e["rnorm_fp16_bits"]]
    assert qz.qjl_kappa(3) == pytest.approx(e["kappa"], rel=1e-15)
    kw = dict(rnorm=out["rnorm"], s_mat=np.eye(3))
    xh = qz.dequantize(out["codes"], out["norm"], np.eye(3), c, qz.MODE_PROD, **kw)
    assert np.allclose(xh, [e["x_hat"]], atol=1e-9)
    lg = qz.logits_rotated(np.array([g["q"]]), out["codes"], out["norm"], np.eye(3), c,
                           qz.MODE_PROD, 1.0, **kw)
    assert lg[0, 0] == pytest.approx(e["logit"], abs=1e-9)


def test_plane_bit_order_by_hand():
    # d = 40 (two 32-coordinate groups, the second zero-padded), 3 planes:
    # group g holds one little-endian word per plane; bit i of the plane-p word
    # is bit p of the index of coordinate 32 g + i.
    idx = np.zeros((1, 40), dtype=np.int64)
    idx[0, 0] = 5          # planes 0 and 2, group 0, bit 0
    idx[0, 9] = 1          # plane 0, group 0, bit 9 -> byte 1 bit 1
    idx[0, 33] = 6         # planes 1 and 2, group 1, bit 1
    codes = qz.pack_planes(idx, 3)
    want = [0x01, 0x02, 0, 0,   0, 0, 0, 0,   0x01, 0, 0, 0,      # group 0: p0, p1, p2
            0, 0, 0, 0,   0x02, 0, 0, 0,   0x02, 0, 0, 0]         # group 1: p0, p1, p2
    assert codes.tolist() == [want]
    assert qz.code_row_bytes(40, 3) == 24


def test_prod_record_puts_sign_on_top_plane():
    # prod mode, b' = 2: record = idx | sign << 2, three planes per group.
    c, t, _ = cb.codebook(32, 2)
    x = np.zeros((1, 32))
    x[0, 0] = 1.0
    out = qz.quantize(x, np.eye(32), c, t, qz.MODE_PROD, s_mat=np.eye(32))
    rec = qz.unpack_planes(out["codes"], 3, 32)
    assert np.array_equal(rec & 3, out["idx"])
    assert np.array_equal(rec >> 2, out["sign_bits"].astype(np.int64))
    assert out["codes"].shape[1] == 12


@pytest.mark.parametrize("nbits", [1, 2, 3, 4])
def test_pack_roundtrip_bijective(nbits):
    d = 3 if nbits <= 3 else 2
    allidx = np.array(list(itertools.product(range(1 << nbits), repeat=d)))
    assert qz.pack_planes(allidx, nbits).shape[1] == qz.code_row_bytes(d, nbits)
    codes = qz.pack_planes(allidx, nbits)
    assert np.array_equal(qz.unpack_planes(codes, nbits, d), allidx)
    assert len({bytes(r) for r in codes}) == allidx.shape[0]
    big = np.random.default_rng(nbits).integers(0, 1 << nbits, (50, 128))
    assert np.array_equal(qz.unpack_planes(qz.pack_planes(big, nbits), nbits, 128), big)


def _setup(d, bits, mode, seed=0):
    lb = qz.lloyd_bits(bits, mode)
    c, t, dist = cb.codebook(d, lb)
    return rot.haar_rotation(d, seed), rot.qjl_matrix(d, seed), c, t, dist


def test_cosine_at_three_bits():
    # Page section "2단계" (closing): reconstructions reach cosine ~0.983 at
    # 3 bits.  With the Lloyd-Max centroid condition E<u, u_hat> = ||u_hat||^2
    # = 1 - D, so the mean cosine is close to sqrt(1 - D) = 0.9829 at d = 128.
    d = 128
    pi, _, c, t, dist = _setup(d, 3, qz.MODE_MSE)
    x = np.random.default_rng(5).standard_normal((3000, d))
    out = qz.quantize(x, pi, c, t, qz.MODE_MSE)
    xh = qz.dequantize(out["codes"], out["norm"], pi, c, qz.MODE_MSE)
    cos = np.einsum("ij,ij->i", x, xh) / np.linalg.norm(x, axis=1) / np.linalg.norm(xh, axis=1)
    assert cos.mean() >= 0.98
    assert cos.mean() == pytest.approx(math.sqrt(1 - d * dist), abs=2e-3)


@pytest.mark.parametrize("bits", [2, 3, 4])
def test_mse_matches_distortion_and_is_data_oblivious(bits):
    # Per-coordinate MSE of unit vectors within 2% of the integrated
    # distortion, for isotropic data and for data with outlier channels
    # (page section "TurboQuant란": no calibration, data-independent).
    from synthetic import tiny_keys_queries
    d = 128
    pi, _, c, t, dist = _setup(d, bits, qz.MODE_MSE)
    iso = np.random.default_rng(2).standard_normal((4000, d))
    outl, _ = tiny_keys_queries(0, n_keys=4000)
    for x in (iso, outl.astype(np.float64)):
        out = qz.quantize(x, pi, c, t, qz.MODE_MSE)
        u = x / np.linalg.norm(x, axis=1, keepdims=True)
        uh = qz.dequantize(out["codes"], qz.to_fp16_bits(np.ones(len(x))), pi, c, qz.MODE_MSE)
        assert np.mean((u - uh) ** 2) == pytest.approx(dist, rel=0.02)


def test_indices_match_brute_force_nearest_centroid():
    d = 128
    pi, _, c, t, _ = _setup(d, 3, qz.MODE_MSE)
    x = np.random.default_rng(3).standard_normal((200, d))
    out = qz.quantize(x, pi, c, t, qz.MODE_MSE)
    y = (x / np.linalg.norm(x, axis=1, keepdims=True)) @ pi.T
    brute = np.argmin(np.abs(y[:, :, None] - c[None, None, :]), axis=2)
    assert np.array_equal(out["idx"], brute)


def test_qjl_estimator_unbiased():
    # Page section "2단계": the sign sketch corrects the inner-product bias.
    # Fix unit q and x and the rotation; draw 10^5 independent S.  The mean
    # error must be within 3 standard errors of 0, where the variance has the
    # closed form (gamma^2/m) ((pi/2)||q||^2 - <q, r/gamma>^2).
    d = 32
    rng = np.random.default_rng(11)
    pi = rot.haar_rotation(d, 1)
    c, t, _ = cb.codebook(d, 1)
    x = rng.standard_normal(d)
    x /= np.linalg.norm(x)
    q = rng.standard_normal(d)
    q -= (q @ x - 0.3) * x                       # <q, x> = 0.3
    q /= np.linalg.norm(q)
    q_rot = pi @ q
    trials = 100_000
    errs = np.empty(trials)
    stage1 = qz.quantize(x[None], pi, c, t, qz.MODE_MSE)
    c_hat = c[stage1["idx"][0]]
    r = x - c_hat @ pi
    gamma = np.linalg.norm(r)
    chunk = 5000
    for i in range(0, trials, chunk):
        s = rng.standard_normal((chunk, d, d))
        sq = s @ q
        sr = s @ r
        signs = np.where(sr >= 0, 1.0, -1.0)
        est = q_rot @ c_hat + qz.qjl_kappa(d) * gamma * np.einsum("ij,ij->i", sq, signs)
        errs[i:i + chunk] = est - q @ x
    var_cf = gamma ** 2 / d * (math.pi / 2 - (q @ r / gamma) ** 2)
    se = math.sqrt(var_cf / trials)
    assert abs(errs.mean()) < 3 * se
    assert errs.var() == pytest.approx(var_cf, rel=0.05)
    # The same estimate through the oracle's own prod-mode path for one S.
    s_mat = rng.standard_normal((d, d))
    c2, t2, _ = cb.codebook(d, 1)
    out = qz.quantize(x[None], pi, c2, t2, qz.MODE_PROD, s_mat=s_mat)
    assert out["gamma"][0] == pytest.approx(gamma, rel=1e-12)
    lg = qz.logits_rotated(q[None], out["codes"], out["norm"], pi, c2, qz.MODE_PROD, 1.0,
                           rnorm=out["rnorm"], s_mat=s_mat)
    s_bits = np.where(s_mat @ r >= 0, 1.0, -1.0)
    by_hand = q_rot @ c_hat + qz.qjl_kappa(d) * qz.from_fp16_bits(out["rnorm"])[0] * ((s_mat @ q) @ s_bits)
    assert lg[0, 0] == pytest.approx(by_hand * qz.from_fp16_bits(out["norm"])[0], rel=1e-12)


@pytest.mark.parametrize("mode,bits", [(qz.MODE_MSE, 3), (qz.MODE_PROD, 3), (qz.MODE_PROD, 4)])
def test_rotated_logits_equal_dequantize_then_dot(mode, bits):
    d = 128
    pi, s_mat, c, t, _ = _setup(d, bits, mode)
    x = np.random.default_rng(4).standard_normal((300, d)) * 3
    q = np.random.default_rng(6).standard_normal((4, d))
    out = qz.quantize(x, pi, c, t, mode, s_mat=s_mat)
    kw = dict(rnorm=out["rnorm"], s_mat=s_mat) if mode == qz.MODE_PROD else {}
    a = qz.logits_rotated(q, out["codes"], out["norm"], pi, c, mode, 0.125, **kw)
    b = qz.logits_dequant(q, out["codes"], out["norm"], pi, c, mode, 0.125, **kw)
    assert np.max(np.abs(a - b)) <= 1e-12 * np.max(np.abs(b))


def test_zero_gamma_reduces_to_mse():
    d = 64
    pi, s_mat, c, t, _ = _setup(d, 3, qz.MODE_PROD)
    x = np.random.default_rng(7).standard_normal((20, d))
    q = np.random.default_rng(8).standard_normal((2, d))
    out = qz.quantize(x, pi, c, t, qz.MODE_PROD, s_mat=s_mat)
    zero = np.zeros_like(out["rnorm"])
    a = qz.logits_rotated(q, out["codes"], out["norm"], pi, c, qz.MODE_PROD, 1.0,
                          rnorm=zero, s_mat=s_mat)
    # the same indices packed without the sign plane, read in MSE mode
    b = qz.logits_rotated(q, qz.pack_planes(out["idx"], 2), out["norm"], pi, c, qz.MODE_MSE, 1.0)
    assert np.array_equal(a, b)


def test_zero_vector():
    d = 32
    pi, s_mat, c, t, _ = _setup(d, 3, qz.MODE_PROD)
    x = np.zeros((2, d))
    x[1, 0] = 1.0
    out = qz.quantize(x, pi, c, t, qz.MODE_PROD, s_mat=s_mat)
    assert np.all(out["idx"][0] == 2)        # 2^(b'-1): the upper middle cell
    assert out["norm"][0] == 0 and out["rnorm"][0] == 0
    assert np.all(out["sign_bits"][0])
    idx, sb = qz.unpack_records(out["codes"], 2, qz.MODE_PROD, d)
    assert np.all(sb[0] == 1) and np.all(idx[0] == 2)
    xh = qz.dequantize(out["codes"], out["norm"], pi, c, qz.MODE_PROD, rnorm=out["rnorm"], s_mat=s_mat)
    assert np.all(xh[0] == 0.0)


def test_fp16_rounding_is_nearest_even():
    # 1 + 2^-11 is halfway between 1 and 1 + 2^-10: ties to even -> 1.
    assert qz.to_fp16_bits([1 + 2 ** -11])[0] == 0x3C00
    assert qz.to_fp16_bits([1 + 3 * 2 ** -11])[0] == 0x3C02
    assert qz.to_fp16_bits([1 + 2 ** -11 + 2 ** -30])[0] == 0x3C01
    assert qz.to_fp16_bits([65520.0])[0] == 0x7C00      # overflows to +inf
    assert qz.from_fp16_bits([0x3555])[0] == pytest.approx(0.333251953125, abs=0)


def test_gqa_logits_layout():
    d = 32
    pi, s_mat, c, t, _ = _setup(d, 2, qz.MODE_MSE)
    rng = np.random.default_rng(13)
    bsz, hkv, hq, tl = 2, 2, 4, 9
    keys = rng.standard_normal((bsz, hkv, tl, d))
    q = rng.standard_normal((bsz, hq, d))
    out = qz.quantize(keys.reshape(-1, d), pi, c, t, qz.MODE_MSE)
    cache = {"codes": out["codes"].reshape(bsz, hkv, tl, -1), "norm": out["norm"].reshape(bsz, hkv, tl)}
    lg = qz.gqa_logits(q, cache, pi, c, qz.MODE_MSE, 0.5)
    for b in range(bsz):
        for h in range(hq):
            kv = h // 2
            ref = qz.logits_dequant(q[b, h][None], cache["codes"][b, kv], cache["norm"][b, kv],
                                    pi, c, qz.MODE_MSE, 0.5)[0]
            assert np.allclose(lg[b, h], ref, rtol=1e-12, atol=1e-12)


def test_topk_brute_force_with_ties():
    rng = np.random.default_rng(14)
    scores = rng.integers(0, 50, (20, 3000)).astype(np.float64)   # many exact ties
    vals, idx = qz.topk(scores, 10)
    for r in range(20):
        pairs = sorted(((-scores[r, i], i) for i in range(3000)))[:10]
        assert idx[r].tolist() == [p[1] for p in pairs]
        assert vals[r].tolist() == [-p[0] for p in pairs]


def test_recall():
    assert qz.recall_at_k([[1, 2, 3]], [[3, 2, 9]]) == pytest.approx(2 / 3)


def test_exact_topk_equals_full_sort_across_blocks():
    """Blockwise exact top-k = a full sort of all inner products (topk, itself
    pinned by brute force), including exact ties split across blocks."""
    rng = np.random.default_rng(7)
    db = rng.standard_normal((1000, 12))
    db /= np.linalg.norm(db, axis=1, keepdims=True)
    db[700] = db[3]                       # the same row in two blocks: an exact tie
    db[999] = db[3]
    q = rng.standard_normal((9, 12))
    q[2] = db[3] * 5.0                    # rows 3, 700, 999 top this query, tied
    want_v, want_i = qz.topk(q @ db.T, 10)
    for block in (64, 333, 1000):
        got_v, got_i = qz.exact_topk(q, db, 10, block=block)
        np.testing.assert_array_equal(got_i, want_i)
        np.testing.assert_allclose(got_v, want_v, rtol=1e-13, atol=0)
    assert list(want_i[2][:3]) == [3, 700, 999]
