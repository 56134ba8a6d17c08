"""Pins for the oracle's decode attention output (oracle/attention.py).

The attention output o = softmax(l) . V_hat is pinned by its reductions to
cases with a plain answer (equal logits give the mean of the values, one
finite logit gives that token's value, two tokens give the logistic split)
and by invariants (shift of the logits, convex hull of the values, masked
rows); the rotated-domain form the device uses is checked against the
dequantise-then-weight definition.
"""

import numpy as np
import pytest

from oracle import attention as att
from oracle import codebook as cb
from oracle import quantizer as qz
from oracle import rotation as rot


def _cache(d=32, bits=3, hkv=2, t_len=41, seed=3, mode=qz.MODE_MSE):
    pi = rot.haar_rotation(d, 0)
    s_mat = rot.qjl_matrix(d, 0) if mode == qz.MODE_PROD else None
    c, t, _ = cb.codebook(d, qz.lloyd_bits(bits, mode))
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((hkv * t_len, d)) * rng.uniform(0.5, 3.0, (hkv * t_len, 1))
    if x.shape[0] > 5:
        x[5] = 0.0                                      # a zero value vector
    ref = qz.quantize(x, pi, c, t, mode, s_mat=s_mat)
    row = ref["codes"].shape[1]
    cache = {"codes": ref["codes"].reshape(1, hkv, t_len, row), "norm": ref["norm"].reshape(1, hkv, t_len)}
    if mode == qz.MODE_PROD:
        cache["rnorm"] = ref["rnorm"].reshape(1, hkv, t_len)
    vhat = qz.dequantize(ref["codes"], ref["norm"], pi, c, mode, rnorm=ref["rnorm"], s_mat=s_mat)
    return pi, c, s_mat, cache, vhat.reshape(hkv, t_len, d)


def test_equal_logits_give_the_mean():
    pi, c, _, cache, vhat = _cache()
    logits = np.full((1, 4, 41), 0.37)
    out = att.attn_output(logits, cache, pi, c, qz.MODE_MSE)
    for hq in range(4):
        np.testing.assert_allclose(out[0, hq], vhat[hq // 2].mean(axis=0), rtol=0, atol=1e-13)


def test_one_finite_logit_selects_that_value():
    pi, c, _, cache, vhat = _cache()
    logits = np.full((1, 4, 41), -np.inf)
    for hq, tok in enumerate((0, 17, 40, 5)):
        logits[0, hq, tok] = 2.5
    out = att.attn_output(logits, cache, pi, c, qz.MODE_MSE)
    for hq, tok in enumerate((0, 17, 40, 5)):
        np.testing.assert_array_equal(out[0, hq], vhat[hq // 2, tok])


def test_two_tokens_split_by_the_logistic():
    pi, c, _, cache, vhat = _cache(t_len=2)
    a, b = 0.8, -1.3
    logits = np.array([[[a, b], [b, a], [0.0, 0.0], [a, a]]])
    out = att.attn_output(logits, cache, pi, c, qz.MODE_MSE)
    w = 1.0 / (1.0 + np.exp(-(a - b)))                  # softmax of two entries
    np.testing.assert_allclose(out[0, 0], w * vhat[0, 0] + (1 - w) * vhat[0, 1], rtol=1e-14, atol=1e-14)
    np.testing.assert_allclose(out[0, 1], (1 - w) * vhat[0, 0] + w * vhat[0, 1], rtol=1e-14, atol=1e-14)
    np.testing.assert_allclose(out[0, 2], 0.5 * (vhat[1, 0] + vhat[1, 1]), rtol=1e-14, atol=1e-14)


def test_shift_invariance_and_convex_hull():
    pi, c, _, cache, vhat = _cache()
    logits = np.random.default_rng(9).standard_normal((1, 4, 41)) * 4.0
    out = att.attn_output(logits, cache, pi, c, qz.MODE_MSE)
    out2 = att.attn_output(logits + 123.25, cache, pi, c, qz.MODE_MSE)
    np.testing.assert_allclose(out, out2, rtol=1e-12, atol=1e-13)
    for hq in range(4):
        v = vhat[hq // 2]
        assert np.all(out[0, hq] <= v.max(axis=0) + 1e-13)
        assert np.all(out[0, hq] >= v.min(axis=0) - 1e-13)


def test_masked_row_is_zero_and_seq_len_truncates():
    pi, c, _, cache, vhat = _cache()
    logits = np.random.default_rng(1).standard_normal((1, 4, 41))
    logits[0, 3, :] = -np.inf
    out = att.attn_output(logits, cache, pi, c, qz.MODE_MSE)
    assert np.all(out[0, 3] == 0.0)
    # tokens past seq_len are ignored: huge logits there change nothing
    big = logits.copy()
    big[0, :, 30:] = 1e6
    np.testing.assert_allclose(att.attn_output(big, cache, pi, c, qz.MODE_MSE, seq_len=30),
                               att.attn_output(logits, cache, pi, c, qz.MODE_MSE, seq_len=30), rtol=0, atol=0)


def test_heads_read_their_kv_head():
    pi, c, _, cache, vhat = _cache(hkv=2)
    logits = np.zeros((1, 4, 41))
    out = att.attn_output(logits, cache, pi, c, qz.MODE_MSE)
    assert not np.allclose(out[0, 0], out[0, 2])         # heads 0-1 read KV 0, heads 2-3 KV 1
    np.testing.assert_array_equal(out[0, 0], out[0, 1])


@pytest.mark.parametrize("bits", [1, 2, 3, 4])
def test_rotated_form_equals_definition(bits):
    pi, c, _, cache, _ = _cache(bits=bits)
    logits = np.random.default_rng(bits).standard_normal((1, 4, 41)) * 3.0
    out = att.attn_output(logits, cache, pi, c, qz.MODE_MSE)
    for h in range(2):
        rot_form = att.attn_output_rotated(logits[0, 2 * h:2 * h + 2], cache["codes"][0, h], cache["norm"][0, h],
                                           pi, c)
        np.testing.assert_allclose(rot_form, out[0, 2 * h:2 * h + 2], rtol=1e-12, atol=1e-13)


def test_prod_mode_values_follow_the_definition():
    pi, c, s_mat, cache, vhat = _cache(mode=qz.MODE_PROD)
    logits = np.full((1, 4, 41), -1.0)
    out = att.attn_output(logits, cache, pi, c, qz.MODE_PROD, s_mat=s_mat)
    np.testing.assert_allclose(out[0, 1], vhat[0].mean(axis=0), rtol=0, atol=1e-13)
