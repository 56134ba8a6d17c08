"""Pins for the oracle's decode step with append (oracle/decode.py).

The step is pinned by the method's online property (a key's record never
depends on the rest of the cache, so appending the keys of a sequence one at
a time rebuilds exactly the cache and logits of quantising it at once), by
the rows it must leave alone, by the causal prefix of the logits and by the
logit definition through reconstructed keys.
"""

import numpy as np
import pytest

from oracle import codebook as cb
from oracle import decode as dec
from oracle import quantizer as qz
from oracle import rotation as rot


def _setup(mode, d=32, bits=3, bsz=2, hkv=2, group=2, rows=9, seed=5):
    pi = rot.haar_rotation(d, 0)
    s_mat = rot.qjl_matrix(d, 0) if mode == qz.MODE_PROD else None
    c, t, _ = cb.codebook(d, qz.lloyd_bits(bits, mode))
    rng = np.random.default_rng(seed)
    keys = rng.standard_normal((bsz, hkv, rows, d)) * rng.uniform(0.3, 4.0, (bsz, hkv, 1, 1))
    keys[0, 1, 3] = 0.0                                   # a zero key (all signs 1, gamma 0)
    q = rng.standard_normal((bsz, hkv * group, d))
    row = qz.code_row_bytes(d, bits)
    cache = {"codes": np.zeros((bsz, hkv, rows, row), np.uint8), "norm": np.zeros((bsz, hkv, rows), np.uint16)}
    if mode == qz.MODE_PROD:
        cache["rnorm"] = np.zeros((bsz, hkv, rows), np.uint16)
    return pi, s_mat, c, t, keys, q, cache


@pytest.mark.parametrize("mode", [qz.MODE_MSE, qz.MODE_PROD])
def test_online_append_equals_offline_quantisation(mode):
    pi, s_mat, c, t, keys, q, cache = _setup(mode)
    bsz, hkv, rows, d = keys.shape
    for pos in range(rows):
        cache, logits, _ = dec.append_step(cache, keys[:, :, pos], pos, q, pi, c, t, mode, 0.25, s_mat=s_mat)
    whole = qz.quantize(keys.reshape(-1, d), pi, c, t, mode, s_mat=s_mat)
    np.testing.assert_array_equal(cache["codes"].reshape(-1, cache["codes"].shape[-1]), whole["codes"])
    np.testing.assert_array_equal(cache["norm"].reshape(-1), whole["norm"])
    if mode == qz.MODE_PROD:
        np.testing.assert_array_equal(cache["rnorm"].reshape(-1), whole["rnorm"])
    # last step's logits = definition through the reconstructed keys
    group = q.shape[1] // hkv
    for b in range(bsz):
        for h in range(hkv):
            sl = slice((b * hkv + h) * rows, (b * hkv + h + 1) * rows)
            kw = dict(rnorm=whole["rnorm"][sl], s_mat=s_mat) if mode == qz.MODE_PROD else {}
            want = qz.logits_dequant(q[b, h * group:(h + 1) * group], whole["codes"][sl], whole["norm"][sl],
                                     pi, c, mode, 0.25, **kw)
            np.testing.assert_allclose(logits[b, h * group:(h + 1) * group], want, rtol=1e-12, atol=1e-12)


def test_other_rows_untouched_and_causal_prefix():
    mode = qz.MODE_PROD
    pi, s_mat, c, t, keys, q, cache = _setup(mode)
    bsz, hkv, rows, d = keys.shape
    for pos in range(rows):
        cache, _, _ = dec.append_step(cache, keys[:, :, pos], pos, q, pi, c, t, mode, 1.0, s_mat=s_mat)
    full = cache
    # rewrite token 4 with another key: only row 4 changes, and the logits
    # over tokens 0..4 agree with the full cache's on tokens 0..3
    other = keys[:, :, 6] * 0.5
    new, logits, ref = dec.append_step(full, other, 4, q, pi, c, t, mode, 1.0, s_mat=s_mat)
    for name in ("codes", "norm", "rnorm"):
        keep = np.ones(rows, bool)
        keep[4] = False
        np.testing.assert_array_equal(new[name][:, :, keep], full[name][:, :, keep])
    assert not np.array_equal(new["codes"][:, :, 4], full["codes"][:, :, 4])
    _, logits_full, _ = dec.append_step(full, keys[:, :, rows - 1], rows - 1, q, pi, c, t, mode, 1.0, s_mat=s_mat)
    np.testing.assert_allclose(logits[:, :, :4], logits_full[:, :, :4], rtol=0, atol=0)
    assert logits.shape == (bsz, q.shape[1], 5)


def test_zero_key_and_position_bounds():
    mode = qz.MODE_PROD
    pi, s_mat, c, t, keys, q, cache = _setup(mode)
    x = keys[:, :, 0].copy()
    x[1, 0] = 0.0
    new, logits, ref = dec.append_step(cache, x, 0, q, pi, c, t, mode, 1.0, s_mat=s_mat)
    idx, sg = qz.unpack_records(new["codes"][1, 0, 0:1], qz.lloyd_bits(3, mode), mode, keys.shape[-1])
    assert np.all(idx == 1 << (qz.lloyd_bits(3, mode) - 1)) and np.all(sg == 1)
    assert new["norm"][1, 0, 0] == 0 and new["rnorm"][1, 0, 0] == 0
    np.testing.assert_array_equal(logits[1, 0:2, 0], 0.0)  # a zero key has logit 0
    with pytest.raises(ValueError):
        dec.append_step(cache, x, cache["codes"].shape[2], q, pi, c, t, mode, 1.0, s_mat=s_mat)


def _paged_from(cache, page_tokens, n_pages_spare, seed):
    """Scatter a contiguous cache [B, Hkv, R, ...] into a pool of pages in a
    random order (with spare pages never referenced); returns (pool, table)."""
    bsz, hkv, rows = cache["norm"].shape
    per_seq = -(-rows // page_tokens)
    n_pages = bsz * per_seq + n_pages_spare
    order = np.random.default_rng(seed).permutation(n_pages)
    table = order[:bsz * per_seq].reshape(bsz, per_seq)
    rng = np.random.default_rng(seed + 1)
    pool = {}
    for name, arr in cache.items():
        shape = (n_pages * hkv * page_tokens,) + arr.shape[3:]
        pool[name] = rng.integers(0, 255, size=shape).astype(arr.dtype)      # garbage in unused rows
    for b in range(bsz):
        for h in range(hkv):
            r = dec.paged_rows(table, page_tokens, hkv, b, h, np.arange(rows))
            for name in cache:
                pool[name][r] = cache[name][b, h]
    return pool, table


@pytest.mark.parametrize("mode", [qz.MODE_MSE, qz.MODE_PROD])
def test_paged_step_equals_contiguous_step_after_gather(mode):
    """A decode step on a paged pool (pages in random order, spare pages full
    of garbage) gives exactly the logits and records of the same step on the
    contiguous cache; gathering the pool through the block table gives back
    the contiguous cache."""
    pi, s_mat, c, t, keys, q, cache = _setup(mode, rows=12)
    bsz, hkv, rows, d = keys.shape
    cache, _, _ = dec.append_step(cache, keys[:, :, 0], 0, q, pi, c, t, mode, 0.5, s_mat=s_mat)
    for pos in range(1, 7):
        cache, _, _ = dec.append_step(cache, keys[:, :, pos], pos, q, pi, c, t, mode, 0.5, s_mat=s_mat)
    pool, table = _paged_from(cache, 4, 3, seed=mode + 3)
    g = dec.gather_paged(pool, table, 4, hkv, rows)
    for name in cache:
        np.testing.assert_array_equal(g[name], cache[name])
    pos = 7
    ccache, clog, cref = dec.append_step(cache, keys[:, :, pos], pos, q, pi, c, t, mode, 0.5, s_mat=s_mat)
    ppool, plog, pref = dec.append_step_paged(pool, table, 4, keys[:, :, pos], pos, q, pi, c, t, mode, 0.5,
                                              s_mat=s_mat)
    np.testing.assert_array_equal(plog, clog)
    np.testing.assert_array_equal(pref["codes"], cref["codes"])
    g = dec.gather_paged(ppool, table, 4, hkv, rows)
    for name in cache:
        np.testing.assert_array_equal(g[name], ccache[name])


def test_paged_step_touches_only_the_new_rows():
    """Every pool row but the new token's row of each (sequence, KV head) is
    bit-identical after the step, including the spare pages."""
    mode = qz.MODE_PROD
    pi, s_mat, c, t, keys, q, cache = _setup(mode, rows=12)
    bsz, hkv, rows, d = keys.shape
    pool, table = _paged_from(cache, 4, 2, seed=11)
    pos = 9
    new, _, _ = dec.append_step_paged(pool, table, 4, keys[:, :, pos], pos, q, pi, c, t, mode, 1.0, s_mat=s_mat)
    changed = np.zeros(len(pool["norm"]), bool)
    for b in range(bsz):
        for h in range(hkv):
            changed[dec.paged_rows(table, 4, hkv, b, h, [pos])] = True
    for name in pool:
        assert np.array_equal(new[name][~changed], pool[name][~changed]), name
    assert changed.sum() == bsz * hkv


def test_paged_rows_layout():
    """Page g holds every KV head's rows of its tokens, head-major."""
    table = np.array([[5, 2], [0, 7]])
    assert list(dec.paged_rows(table, 64, 8, 0, 0, [0, 63, 64, 127])) == [5 * 512, 5 * 512 + 63, 2 * 512, 2 * 512 + 63]
    assert list(dec.paged_rows(table, 64, 8, 1, 3, [65])) == [(7 * 8 + 3) * 64 + 1]
