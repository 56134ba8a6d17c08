"""GPU parity of every entry point against the fp64 oracle (small and ragged sizes).

All inputs are seeded synthetic data; the GPU logit / dequantize / search
kernels are fed oracle-packed codes, so they are judged on identical codes.
"""

import numpy as np
import pytest
import torch

from oracle import quantizer as oqz
from synthetic import bf16_bits, bf16_to_f32, channel_scales, kv_block, search_vectors, tiny_keys_queries

from parity import (OracleTables, cache_from_oracle, check_dequant, check_logits, check_norms,
                    check_polar_codes, check_records, dev_bf16, dev_u16)

pytestmark = pytest.mark.gpu

DEV = torch.device("cuda:0")


@pytest.fixture(scope="module")
def tq():
    import online_vector_quantization_amd as pkg
    return pkg


def _keys_bf16(d, n, seed=0, head=0):
    scales = channel_scales(seed, 2, "k", 2, d) if d == 128 else \
        np.exp(np.random.default_rng(seed).standard_normal((2, d)))
    return kv_block(seed, 2, "k", 0, head, n, scales)


def _special_rows(x64, edge=False):
    """Rows 3, 7, 11, 13: zero, one-hot and tiny vectors.  With ``edge``, also
    row 17 with ||x|| above 65520 (its fp16 norm is +inf; the codes come from
    the direction) and rows 19 and 23 holding a NaN and an infinity (codes
    unspecified, the call must still succeed and leave every other row right)."""
    x64 = x64.copy()
    x64[3] = 0.0                     # zero vector
    x64[7] = 0.0
    x64[7, 5] = 2.5                  # one nonzero coordinate
    d = x64.shape[1]
    j = np.arange(d)
    sign = np.where(j % 3 == 0, -1.0, 1.0)
    # tiny vectors, exact in bf16 and fp32: normal numbers with the largest
    # exponent -118, and subnormals k * 2^-133 (bf16's smallest step); their
    # fp16 norms round to 0, their directions still define the codes
    x64[11] = sign * (1.0 + (j * 37 % 128) / 128.0) * np.ldexp(1.0, -118 - (j % 5))
    x64[13] = sign * (1 + j * 11 % 127) * np.ldexp(1.0, -133)
    if edge:
        # exact in bf16: 12032 = 47 * 2^8, times 1, 1.25 or 1.5; ||x|| >= 96256
        x64[17] = sign * 12032.0 * np.array([1.0, 1.25, 1.5, 1.0])[j % 4]
        x64[19, 9] = np.nan
        x64[23, 2] = np.inf
    return x64


NONFINITE_ROWS = [19, 23]


QUANT_CASES = [(128, b, "mse", dt) for b in (1, 2, 3, 4) for dt in ("bf16", "f32")] + \
              [(128, b, "prod", dt) for b in (2, 3, 4, 5) for dt in ("bf16", "f32")] + \
              [(64, 3, "mse", "bf16"), (64, 3, "prod", "bf16"), (64, 5, "prod", "f32"),
               (256, 2, "mse", "f32"), (256, 4, "mse", "f32"), (256, 3, "mse", "bf16"),
               (256, 3, "prod", "bf16"), (256, 5, "prod", "f32"), (256, 2, "prod", "bf16")]


@pytest.mark.parametrize("d,bits,mode,dtype", QUANT_CASES)
def test_quantize_parity(tq, d, bits, mode, dtype):
    mcode = oqz.MODE_PROD if mode == "prod" else oqz.MODE_MSE
    n = 1000                                      # 31 full tiles + a ragged one
    if dtype == "bf16":
        xb = _keys_bf16(d, n)
        x64 = _special_rows(bf16_to_f32(xb).astype(np.float64), edge=True)
        xb = bf16_bits(x64.astype(np.float32))     # NaN and inf map to bf16 NaN and inf
        stride = d + 8                            # rows further apart than d
        buf = np.zeros((n, stride), dtype=np.uint16)
        buf[:, :d] = xb
        xt = dev_bf16(buf, DEV)[:, :d]
    else:
        rng = np.random.default_rng(d + bits)
        x32 = (rng.standard_normal((n, d)) * np.where(np.arange(d) % 37 == 0, 10.0, 1.0)).astype(np.float32)
        x64 = _special_rows(x32.astype(np.float64), edge=True)
        xt = torch.from_numpy(x64.astype(np.float32)).to(DEV)
    finite = np.all(np.isfinite(x64), axis=1)
    assert list(np.nonzero(~finite)[0]) == NONFINITE_ROWS
    ot = OracleTables(d, bits, mcode)
    ref = ot.quantize(x64[finite])
    qz = tq.Quantizer(d, bits, mcode, seed=0, device=DEV)
    off = 5
    cache = qz.new_cache(n + 9)
    qz.quantize(xt, out=cache, out_offset=off)
    torch.cuda.synchronize()
    codes = cache.codes.cpu().numpy()[off:off + n]
    rn = cache.rnorm.cpu().numpy()[off:off + n][finite] if mcode == oqz.MODE_PROD else None
    check_records(codes[finite], cache.norm.cpu().numpy()[off:off + n][finite], rn, ref, ot)
    # the row with ||x|| > 65520: norm +inf, every other field as the oracle's
    assert cache.norm.cpu().numpy().view(np.uint16)[off + 17] == 0x7C00
    idx3, sg3 = oqz.unpack_records(codes[3:4], ot.lb, mcode, d)
    assert np.all(idx3 == 1 << (ot.lb - 1))
    if mcode == oqz.MODE_PROD:
        assert np.all(sg3 == 1)
        assert cache.rnorm.cpu().numpy()[off + 3] == 0


@pytest.mark.parametrize("d,mode", [(128, "prod"), (128, "mse"), (256, "prod")])
def test_quantize_parity_several_tiles_per_workgroup(tq, d, mode):
    """Every output against the oracle when each workgroup of the persistent
    grid loops over several tiles (at least four per workgroup at up to three
    workgroups per CU, plus a ragged tail), so the kernels' buffer rotation
    wraps several times."""
    mcode = oqz.MODE_PROD if mode == "prod" else oqz.MODE_MSE
    bits = 3
    n = 4 * 32 * 3 * torch.cuda.get_device_properties(DEV).multi_processor_count + 17
    xb = _keys_bf16(d, n, seed=5)
    x64 = _special_rows(bf16_to_f32(xb).astype(np.float64))
    xt = dev_bf16(bf16_bits(x64.astype(np.float32)), DEV)
    ot = OracleTables(d, bits, mcode)
    ref = ot.quantize(x64)
    qz = tq.Quantizer(d, bits, mcode, seed=0, device=DEV)
    cache = qz.quantize(xt)
    torch.cuda.synchronize()
    rn = cache.rnorm.cpu().numpy() if mcode == oqz.MODE_PROD else None
    check_records(cache.codes.cpu().numpy(), cache.norm.cpu().numpy(), rn, ref, ot)


def _gqa_case(d, bits, mode, bsz, hkv, group, seq, qdtype, seed=0, row_tokens=None):
    """Oracle-packed cache [bsz, hkv, row_tokens] and queries; returns everything."""
    mcode = oqz.MODE_PROD if mode == "prod" else oqz.MODE_MSE
    ot = OracleTables(d, bits, mcode, seed=seed)
    row_tokens = seq if row_tokens is None else row_tokens
    rng = np.random.default_rng(100 + seq + group)
    scales = np.exp(rng.standard_normal((hkv, d)))
    keys = (rng.standard_normal((bsz, hkv, row_tokens, d)) * scales[None, :, None, :]).astype(np.float32)
    keys = bf16_to_f32(bf16_bits(keys)).astype(np.float64)
    q = rng.standard_normal((bsz, hkv * group, d)) * np.repeat(scales, group, axis=0)[None]
    if qdtype == "bf16":
        qb = bf16_bits(q.astype(np.float32))
        q64 = bf16_to_f32(qb).astype(np.float64)
        qt = dev_bf16(qb, DEV)
    else:
        q64 = q.astype(np.float32).astype(np.float64)
        qt = torch.from_numpy(q64.astype(np.float32)).to(DEV)
    ref = ot.quantize(keys.reshape(-1, d))
    return ot, mcode, keys, q64, qt, ref


LOGIT_CASES = [
    # d, bits, mode, batch, kv heads, group, seq, q dtype
    (128, 3, "prod", 1, 2, 4, 3000, "bf16"),
    (128, 4, "prod", 2, 2, 4, 2049, "bf16"),
    (128, 2, "prod", 1, 1, 4, 700, "f32"),
    (128, 5, "prod", 1, 1, 2, 513, "f32"),
    (128, 3, "mse", 1, 1, 16, 4096, "f32"),
    (128, 1, "mse", 1, 3, 1, 1000, "bf16"),
    (128, 2, "mse", 2, 1, 3, 999, "bf16"),
    (128, 4, "mse", 1, 2, 8, 1500, "f32"),
    (128, 3, "prod", 1, 1, 13, 300, "f32"),
    (256, 2, "mse", 1, 1, 4, 1100, "f32"),
    (256, 3, "prod", 1, 2, 4, 777, "bf16"),
    (64, 3, "prod", 1, 2, 4, 1300, "bf16"),
    (64, 5, "prod", 1, 1, 6, 517, "f32"),
    (64, 2, "prod", 2, 1, 16, 640, "bf16"),
    (64, 1, "mse", 1, 2, 1, 999, "f32"),
    (64, 4, "mse", 1, 1, 12, 2000, "bf16"),
]


@pytest.mark.parametrize("d,bits,mode,bsz,hkv,group,seq,qdtype", LOGIT_CASES)
def test_logits_parity(tq, d, bits, mode, bsz, hkv, group, seq, qdtype):
    ot, mcode, keys, q64, qt, ref = _gqa_case(d, bits, mode, bsz, hkv, group, seq, qdtype)
    qz = tq.Quantizer(d, bits, mcode, seed=0, device=DEV)
    cache = cache_from_oracle(tq, ref, d, bits, mcode, DEV)
    scale = 1.0 / np.sqrt(d)
    out = qz.attn_logits(qt, cache, n_kv_heads=hkv, seq_len=seq, scale=scale).cpu().numpy()
    codes = ref["codes"].reshape(bsz, hkv, seq, -1)
    norm = ref["norm"].reshape(bsz, hkv, seq)
    for b in range(bsz):
        for h in range(hkv):
            kw = {}
            if mcode == oqz.MODE_PROD:
                kw = dict(rnorm=ref["rnorm"].reshape(bsz, hkv, seq)[b, h], s_mat=ot.s)
            qq = q64[b, h * group:(h + 1) * group]
            want = oqz.logits_rotated(qq, codes[b, h], norm[b, h], ot.pi, ot.c, mcode, scale, **kw)
            check_logits(out[b, h * group:(h + 1) * group], want, scale, norm[b, h], qq)


def test_logits_row_tokens_capacity(tq):
    """Streams of capacity 600 holding 437 valid tokens: tokens past seq_len are never read into results."""
    d, bits, hkv, group, cap, seq = 128, 3, 2, 4, 600, 437
    ot, mcode, keys, q64, qt, ref = _gqa_case(d, bits, "prod", 1, hkv, group, seq, "bf16", row_tokens=cap)
    qz = tq.Quantizer(d, bits, mcode, seed=0, device=DEV)
    cache = cache_from_oracle(tq, ref, d, bits, mcode, DEV)
    out = qz.attn_logits(qt, cache, n_kv_heads=hkv, seq_len=seq, scale=0.5, row_tokens=cap).cpu().numpy()
    assert out.shape == (1, hkv * group, seq)
    for h in range(hkv):
        sl = slice(h * cap, h * cap + seq)
        qq = q64[0, h * group:(h + 1) * group]
        want = oqz.logits_rotated(qq, ref["codes"][sl], ref["norm"][sl], ot.pi, ot.c, mcode, 0.5,
                                  rnorm=ref["rnorm"][sl], s_mat=ot.s)
        check_logits(out[0, h * group:(h + 1) * group], want, 0.5, ref["norm"][sl], qq)


DEQ_CASES = [(128, b, "mse") for b in (1, 2, 3, 4)] + [(128, b, "prod") for b in (2, 3, 4, 5)] + \
            [(64, 3, "mse"), (64, 4, "prod"), (256, 2, "mse"), (256, 4, "mse"), (256, 3, "prod"),
             (256, 5, "prod")]


@pytest.mark.parametrize("d,bits,mode", DEQ_CASES)
def test_dequantize_parity(tq, d, bits, mode):
    mcode = oqz.MODE_PROD if mode == "prod" else oqz.MODE_MSE
    ot = OracleTables(d, bits, mcode)
    n = 777
    x64 = _special_rows(np.random.default_rng(d * bits).standard_normal((n, d)) * 3.0)
    ref = ot.quantize(x64)
    qz = tq.Quantizer(d, bits, mcode, seed=0, device=DEV)
    cache = cache_from_oracle(tq, ref, d, bits, mcode, DEV)
    want = oqz.dequantize(ref["codes"], ref["norm"], ot.pi, ot.c, mcode, rnorm=ref["rnorm"],
                          s_mat=ot.s)
    got = qz.dequantize(cache, n).cpu().numpy()
    check_dequant(got, want)
    assert np.all(got[3] == 0.0)
    gotb = qz.dequantize(cache, n, out_dtype=torch.bfloat16).float().cpu().numpy()
    assert np.max(np.abs(gotb - want)) <= 2.0 ** -8 * np.max(np.abs(want)) + 1e-6


@pytest.mark.parametrize("bits", [2, 4])
def test_search_parity(tq, bits):
    d, n_db, n_q, k = 256, 20000, 300, 10
    db = search_vectors(0, "db", 0, n_db)
    qv = search_vectors(0, "dbq", 0, n_q)
    ot = OracleTables(d, bits, oqz.MODE_MSE)
    ref = ot.quantize(db.astype(np.float64))
    qz = tq.Quantizer(d, bits, oqz.MODE_MSE, seed=0, device=DEV)
    cache = cache_from_oracle(tq, ref, d, bits, oqz.MODE_MSE, DEV)
    qt = torch.from_numpy(qv.reshape(1, n_q, d)).to(DEV)
    vals, idx = qz.search(qt, cache, n_kv_heads=1, seq_len=n_db, topk=k)
    vals, idx = vals.cpu().numpy()[0], idx.cpu().numpy()[0]
    scores = oqz.logits_rotated(qv.astype(np.float64), ref["codes"], ref["norm"], ot.pi, ot.c,
                                oqz.MODE_MSE, 1.0)
    ov, oi = oqz.topk(scores, k)
    for r in range(n_q):
        # returned pairs carry the oracle's score for that index
        assert np.all(np.abs(vals[r] - scores[r, idx[r]]) <= 1e-4 * np.maximum(np.abs(scores[r, idx[r]]), 1e-3))
        assert np.all(np.diff(vals[r]) <= 1e-6)
        # same set, up to near-ties with the oracle's 10th score
        tol = 1e-4 * max(abs(ov[r, -1]), 1e-3)
        diff = set(idx[r].tolist()) ^ set(oi[r].tolist())
        for i in diff:
            assert abs(scores[r, i] - ov[r, -1]) <= tol, (r, i)


@pytest.mark.parametrize("d,bits,n_db", [(64, 3, 3001), (64, 1, 3001), (128, 4, 3001), (128, 2, 700)])
def test_search_parity_gqa(tq, d, bits, n_db):
    """Top-k over two KV heads of n_db keys each (a ragged last tile), 40
    query heads per KV head, at d = 64 and 128: 3001 keys take a sample pass
    (192 keys) that seeds the bounds of the main pass, 700 keys one pass."""
    hkv, group, k = 2, 40, 10
    rng = np.random.default_rng(d + bits)
    scales = np.exp(0.5 * rng.standard_normal((hkv, d)))
    db = rng.standard_normal((hkv, n_db, d)) * scales[:, None, :]
    qv = (rng.standard_normal((hkv * group, d)) * np.repeat(scales, group, axis=0)).astype(np.float32)
    ot = OracleTables(d, bits, oqz.MODE_MSE)
    ref = ot.quantize(db.reshape(-1, d))
    qz = tq.Quantizer(d, bits, oqz.MODE_MSE, seed=0, device=DEV)
    cache = cache_from_oracle(tq, ref, d, bits, oqz.MODE_MSE, DEV)
    qt = torch.from_numpy(qv.reshape(1, hkv * group, d)).to(DEV)
    vals, idx = qz.search(qt, cache, n_kv_heads=hkv, seq_len=n_db, topk=k)
    vals, idx = vals.cpu().numpy()[0], idx.cpu().numpy()[0]
    for h in range(hkv):
        sl = slice(h * n_db, (h + 1) * n_db)
        qq = qv[h * group:(h + 1) * group].astype(np.float64)
        scores = oqz.logits_rotated(qq, ref["codes"][sl], ref["norm"][sl], ot.pi, ot.c, oqz.MODE_MSE, 1.0)
        ov, oi = oqz.topk(scores, k)
        for r in range(group):
            row = h * group + r
            got = scores[r, idx[row]]
            assert np.all(np.abs(vals[row] - got) <= 1e-4 * np.maximum(np.abs(got), 1e-3)), row
            assert np.all(np.diff(vals[row]) <= 1e-6)
            tol = 1e-4 * max(abs(ov[r, -1]), 1e-3)
            for i in set(idx[row].tolist()) ^ set(oi[r].tolist()):
                assert abs(scores[r, i] - ov[r, -1]) <= tol, (row, i)


@pytest.mark.parametrize("k", [1, 16])
def test_search_topk_extremes(tq, k):
    """topk = 1 and the largest list (16) over 5000 keys (sample and main
    passes), 300 queries, d = 128, b = 3."""
    d, bits, n_db, n_q = 128, 3, 5000, 300
    rng = np.random.default_rng(40 + k)
    db = rng.standard_normal((n_db, d)) * np.exp(0.5 * rng.standard_normal(d))
    qv = (rng.standard_normal((n_q, d)) * np.exp(0.5 * rng.standard_normal(d))).astype(np.float32)
    ot = OracleTables(d, bits, oqz.MODE_MSE)
    ref = ot.quantize(db)
    qz = tq.Quantizer(d, bits, oqz.MODE_MSE, seed=0, device=DEV)
    cache = cache_from_oracle(tq, ref, d, bits, oqz.MODE_MSE, DEV)
    vals, idx = qz.search(torch.from_numpy(qv.reshape(1, n_q, d)).to(DEV), cache, n_kv_heads=1, seq_len=n_db, topk=k)
    vals, idx = vals.cpu().numpy()[0], idx.cpu().numpy()[0]
    scores = oqz.logits_rotated(qv.astype(np.float64), ref["codes"], ref["norm"], ot.pi, ot.c, oqz.MODE_MSE, 1.0)
    ov, oi = oqz.topk(scores, k)
    for r in range(n_q):
        got = scores[r, idx[r]]
        assert np.all(np.abs(vals[r] - got) <= 1e-4 * np.maximum(np.abs(got), 1e-3)), r
        assert np.all(np.diff(vals[r]) <= 1e-6)
        tol = 1e-4 * max(abs(ov[r, -1]), 1e-3)
        for i in set(idx[r].tolist()) ^ set(oi[r].tolist()):
            assert abs(scores[r, i] - ov[r, -1]) <= tol, (r, i)


@pytest.mark.parametrize("scale", [1.0, -0.5, 0.0])
def test_search_ties_zeros_and_scale(tq, scale):
    """Exact ties (duplicated database rows), zero rows, a zero query, and a
    negative or zero scale (d = 128, 3 bits, several key tiles and splits).

    Duplicated rows have identical codes, so their scores tie exactly on both
    sides and the smaller index must win; with scale 0 (or a zero query)
    every score is 0 and the top-k are the first k keys."""
    d, bits, k = 128, 3, 16
    rng = np.random.default_rng(11)
    base = rng.standard_normal((700, d))
    db = base[rng.integers(0, 700, 9000)]               # every vector about 13 times
    db[[5, 77, 4000]] = 0.0
    n_db = db.shape[0]
    qv = rng.standard_normal((37, d))
    qv[4] = 0.0
    ot = OracleTables(d, bits, oqz.MODE_MSE)
    ref = ot.quantize(db)
    qz = tq.Quantizer(d, bits, oqz.MODE_MSE, seed=0, device=DEV)
    cache = cache_from_oracle(tq, ref, d, bits, oqz.MODE_MSE, DEV)
    qt = torch.from_numpy(qv.astype(np.float32).reshape(1, -1, d)).to(DEV)
    vals, idx = qz.search(qt, cache, n_kv_heads=1, seq_len=n_db, topk=k, scale=scale)
    vals, idx = vals.cpu().numpy()[0], idx.cpu().numpy()[0]
    scores = oqz.logits_rotated(qv.astype(np.float32).astype(np.float64), ref["codes"], ref["norm"],
                                ot.pi, ot.c, oqz.MODE_MSE, scale)
    ov, oi = oqz.topk(scores, k)
    # groups of identical packed rows (same codes and norm -> same score)
    rows = np.concatenate([ref["codes"].view(np.uint8).reshape(n_db, -1),
                           ref["norm"].view(np.uint8).reshape(n_db, -1)], axis=1)
    _, group = np.unique(rows, axis=0, return_inverse=True)
    group = group.reshape(-1)
    for r in range(qv.shape[0]):
        assert len(set(idx[r].tolist())) == k
        got = scores[r, idx[r]]
        assert np.all(np.abs(vals[r] - got) <= 1e-4 * np.maximum(np.abs(got), 1e-3)), r
        if scale == 0.0 or r == 4:
            assert idx[r].tolist() == list(range(k)), (r, idx[r])
            continue
        tol = 1e-4 * max(abs(ov[r, -1]), 1e-3)
        for i in set(idx[r].tolist()) ^ set(oi[r].tolist()):
            assert abs(scores[r, i] - ov[r, -1]) <= tol, (r, i)
        # among exact duplicates, the smaller indices are taken first
        chosen = set(idx[r].tolist())
        for i in idx[r]:
            same = np.nonzero(group == group[i])[0]
            assert all(j in chosen for j in same[same < i]), (r, i)


def test_end_to_end_quantize_then_logits(tq):
    """GPU quantise -> GPU logits vs oracle quantise -> oracle logits (keys with identical codes)."""
    d, bits, seq, group = 128, 3, 2000, 4
    kb = _keys_bf16(d, seq)
    k64 = bf16_to_f32(kb).astype(np.float64)
    ot = OracleTables(d, bits, oqz.MODE_PROD)
    ref = ot.quantize(k64)
    qz = tq.Quantizer(d, bits, oqz.MODE_PROD, seed=0, device=DEV)
    cache = qz.quantize(dev_bf16(kb, DEV))
    q64 = bf16_to_f32(bf16_bits(np.random.default_rng(5).standard_normal((group, d)).astype(np.float32)))
    q64 = q64.astype(np.float64)
    out = qz.attn_logits(torch.from_numpy(q64.astype(np.float32)).reshape(1, group, d).to(DEV), cache,
                         n_kv_heads=1, seq_len=seq, scale=1 / np.sqrt(d)).cpu().numpy()[0]
    # rows whose record differs carry counted, in-window mismatches; the rest are compared
    same = check_records(cache.codes.cpu().numpy(), cache.norm.cpu().numpy(), cache.rnorm.cpu().numpy(), ref, ot)
    want = oqz.logits_rotated(q64, ref["codes"], ref["norm"], ot.pi, ot.c, oqz.MODE_PROD, 1 / np.sqrt(d),
                              rnorm=ref["rnorm"], s_mat=ot.s)
    check_logits(out[:, same], want[:, same], 1 / np.sqrt(d), ref["norm"][same], q64)


def _midpoint_rows(d):
    """bf16 rows whose exact norms sit on or next to fp16 rounding midpoints.
    (1, 2^-5, 2^-11) has |x|^2 = (1 + 2^-11)^2: exactly halfway between fp16
    1 and 1 + 2^-10, so nearest-even gives 1 (0x3C00); one more element of
    2^-20 lifts it past the midpoint (0x3C01) by 2^-41 relative, which an
    fp32 sum of the squares loses and the fp64 sums keep.  (1, 2^-5 x 3, 2^-11 x 9) has
    |x| = 1 + 3 * 2^-11, halfway between 1 + 2^-10 and 1 + 2^-9, so the tie goes
    up to the even 0x3C02.  Each row also appears scaled by 2^-10 and 2^12
    (exact in bf16, still fp16 normals; the exponent field moves by -10 and
    +12).  Returns
    the rows and the expected fp16 norm bits."""
    base = []
    r = np.zeros(d); r[0], r[1], r[2] = 1.0, 2.0 ** -5, 2.0 ** -11
    base.append((r, 0x3C00))
    r = r.copy(); r[3] = 2.0 ** -20
    base.append((r, 0x3C01))
    r = np.zeros(d); r[0] = 1.0; r[1:4] = 2.0 ** -5; r[4:13] = 2.0 ** -11
    base.append((r, 0x3C02))
    rows, want = [], []
    for k in (0, -10, 12):
        for r, bits in base:
            rows.append(r * 2.0 ** k)
            want.append(bits + (k << 10))
    return np.array(rows), np.array(want, dtype=np.uint16)


@pytest.mark.parametrize("d,mode", [(128, oqz.MODE_MSE), (128, oqz.MODE_PROD), (64, oqz.MODE_MSE), (256, oqz.MODE_PROD)])
def test_norm_rounding_at_fp16_midpoints(tq, d, mode):
    """The fp16 norm is the nearest-even rounding of the exact norm on exact
    ties and just past them, wherever the kernel forms its sums of squares
    (fp32 with an exact fallback in the one-kind kernels, fp64 in the split
    key kernel); checked against the hand values and the oracle."""
    x64, want = _midpoint_rows(d)
    xb = bf16_bits(x64.astype(np.float32))
    assert np.array_equal(bf16_to_f32(xb).astype(np.float64), x64)      # exact in bf16
    ot = OracleTables(d, 3, mode)
    ref = ot.quantize(x64)
    assert np.array_equal(ref["norm"].view(np.uint16), want)
    qz = tq.Quantizer(d, 3, mode, seed=0, device=DEV)
    cache = qz.quantize(dev_bf16(xb, DEV))
    torch.cuda.synchronize()
    got = cache.norm.cpu().numpy().view(np.uint16)[:len(want)]
    assert np.array_equal(got, want), (got, want)


def test_empty_and_single(tq):
    qz = tq.Quantizer(128, 3, oqz.MODE_PROD, seed=0, device=DEV)
    cache = qz.new_cache(4)
    qz.quantize(torch.zeros((0, 128), dtype=torch.bfloat16, device=DEV), out=cache)
    x = torch.zeros((1, 128), dtype=torch.float32, device=DEV)
    x[0, 0] = 1.0
    qz.quantize(x, out=cache)
    lg = qz.attn_logits(torch.ones((1, 4, 128), device=DEV), cache, n_kv_heads=1, seq_len=1, scale=1.0)
    torch.cuda.synchronize()
    assert lg.shape == (1, 4, 1) and torch.isfinite(lg).all()
    empty = qz.attn_logits(torch.ones((1, 4, 128), device=DEV), cache, n_kv_heads=1, seq_len=0, scale=1.0)
    assert empty.shape == (1, 4, 0)


ATTN_CASES = [  # d, bits, batch, n_kv_heads, group, seq_len, extra row capacity
    (128, 3, 1, 2, 4, 1000, 0),      # 15 chunks + a ragged one, two KV heads
    (128, 2, 2, 3, 1, 33, 5),        # batch 2, no GQA, one partial chunk, row_tokens > seq_len
    (128, 4, 1, 1, 8, 5000, 0),      # several splits
    (128, 1, 1, 2, 2, 1, 0),         # a single token
    (256, 2, 1, 1, 16, 700, 3),      # padded search width, the largest GQA group
    (256, 4, 2, 1, 3, 2100, 0),      # group padded to 4
    (64, 3, 1, 2, 2, 1500, 2),       # d = 64: two token halves per lane, 24-byte rows
    (64, 1, 2, 1, 1, 70, 0),         # d = 64, 8-byte rows, a chunk and a partial one
    (64, 4, 1, 1, 6, 3000, 0),       # d = 64 on the matrix-core kernel, group padded to 8
    (64, 3, 1, 3, 16, 999, 1),       # d = 64, the largest group, odd bit width
]


@pytest.mark.parametrize("d,bits,batch,hkv,group,seq,extra", ATTN_CASES)
def test_attn_output_parity(tq, d, bits, batch, hkv, group, seq, extra):
    """softmax(logits) . V_hat from packed MSE values vs the fp64 oracle."""
    from oracle import attention as oatt
    rows = seq + extra
    rng = np.random.default_rng(1000 * d + 10 * bits + group)
    x = rng.standard_normal((batch * hkv * rows, d)) * rng.uniform(0.2, 4.0, (batch * hkv * rows, 1))
    x[7 % x.shape[0]] = 0.0
    ot = OracleTables(d, bits, oqz.MODE_MSE)
    ref = ot.quantize(x)
    qz = tq.Quantizer(d, bits, oqz.MODE_MSE, seed=0, device=DEV)
    cache = cache_from_oracle(tq, ref, d, bits, oqz.MODE_MSE, DEV)
    hq = hkv * group
    logits = (rng.standard_normal((batch, hq, seq)) * 3.0).astype(np.float32)
    logits[:, :, rng.integers(0, seq, max(1, seq // 7))] = -np.inf      # masked tokens
    if hq > 1:
        logits[0, hq - 1, :] = -np.inf                                    # a fully masked head
    lt = torch.from_numpy(logits).to(DEV)
    got = qz.attn_output(lt, cache, n_kv_heads=hkv, seq_len=seq, row_tokens=rows).cpu().numpy()
    rb = ref["codes"].shape[1]
    ocache = {"codes": ref["codes"].reshape(batch, hkv, rows, rb), "norm": ref["norm"].reshape(batch, hkv, rows)}
    want = oatt.attn_output(logits.astype(np.float64), ocache, ot.pi, ot.c, oqz.MODE_MSE, seq_len=seq)
    err = np.linalg.norm(got - want, axis=2)
    scale = np.linalg.norm(want, axis=2)
    assert np.all(err <= 1e-4 * scale + 1e-6), float(np.max(err - 1e-4 * scale))
    if hq > 1:
        assert np.all(got[0, hq - 1] == 0.0)
    gotb = qz.attn_output(lt, cache, n_kv_heads=hkv, seq_len=seq, row_tokens=rows,
                          out_dtype=torch.bfloat16).float().cpu().numpy()
    assert np.all(np.abs(gotb - want) <= 2.0 ** -8 * np.abs(want).max(axis=2, keepdims=True) + 1e-6)


def test_attn_output_empty_and_unsupported(tq):
    d, bits = 128, 3
    ot = OracleTables(d, bits, oqz.MODE_MSE)
    ref = ot.quantize(np.random.default_rng(2).standard_normal((64, d)))
    qz = tq.Quantizer(d, bits, oqz.MODE_MSE, seed=0, device=DEV)
    cache = cache_from_oracle(tq, ref, d, bits, oqz.MODE_MSE, DEV)
    out = torch.full((1, 4, d), 7.0, device=DEV)
    qz.attn_output(torch.zeros((1, 4, 0), device=DEV), cache, n_kv_heads=1, seq_len=0, row_tokens=64, out=out)
    assert torch.all(out == 0.0)
    otp = OracleTables(d, bits, oqz.MODE_PROD)
    refp = otp.quantize(np.random.default_rng(3).standard_normal((64, d)))
    qp = tq.Quantizer(d, bits, oqz.MODE_PROD, seed=0, device=DEV)
    cp = cache_from_oracle(tq, refp, d, bits, oqz.MODE_PROD, DEV)
    with pytest.raises(tq.TQError):
        qp.attn_output(torch.zeros((1, 4, 64), device=DEV), cp, n_kv_heads=1, seq_len=64)


APPEND_CASES = [
    # d, bits, mode, batch, kv heads, group, row_tokens, pos, x dtype, q dtype
    (128, 3, "prod", 1, 8, 4, 600, 437, "bf16", "bf16"),
    (128, 3, "mse", 2, 2, 4, 300, 0, "f32", "f32"),
    (128, 5, "prod", 1, 2, 2, 1000, 999, "f32", "bf16"),
    (128, 2, "prod", 2, 1, 16, 260, 259, "bf16", "f32"),
    (128, 1, "mse", 1, 3, 1, 70, 33, "bf16", "bf16"),
    (256, 3, "prod", 1, 1, 4, 513, 512, "bf16", "f32"),
    (256, 2, "mse", 1, 2, 8, 257, 100, "f32", "f32"),
    (64, 3, "prod", 2, 2, 4, 400, 399, "bf16", "bf16"),
    (64, 3, "mse", 1, 3, 2, 129, 64, "f32", "bf16"),
]


@pytest.mark.parametrize("d,bits,mode,bsz,hkv,group,rows,pos,xdtype,qdtype", APPEND_CASES)
def test_append_attn_logits_parity(tq, d, bits, mode, bsz, hkv, group, rows, pos, xdtype, qdtype):
    """New keys quantised into token pos by the logit call: the row against the
    oracle's quantiser, every other row untouched, logits over tokens 0..pos."""
    from oracle import decode as odec
    ot, mcode, keys, q64, qt, ref = _gqa_case(d, bits, mode, bsz, hkv, group, rows, qdtype, row_tokens=rows)
    rng = np.random.default_rng(pos + 7 * d)
    x = rng.standard_normal((bsz, hkv, d)) * np.exp(rng.standard_normal((1, hkv, d)))
    x[0, hkv - 1] = 0.0                                   # a zero key
    if xdtype == "bf16":
        xb = bf16_bits(x.astype(np.float32))
        x64 = bf16_to_f32(xb).astype(np.float64)
        xt = dev_bf16(xb, DEV)
    else:
        x64 = x.astype(np.float32).astype(np.float64)
        xt = torch.from_numpy(x64.astype(np.float32)).to(DEV)
    qz = tq.Quantizer(d, bits, mcode, seed=0, device=DEV)
    cache = cache_from_oracle(tq, ref, d, bits, mcode, DEV)
    before = {n: getattr(cache, n).cpu().numpy().copy() for n in ("codes", "norm", "rnorm")
              if getattr(cache, n) is not None}
    scale = 1.0 / np.sqrt(d)
    out = qz.append_attn_logits(xt, qt, cache, n_kv_heads=hkv, pos=pos, scale=scale, row_tokens=rows)
    torch.cuda.synchronize()
    assert out.shape == (bsz, hkv * group, pos + 1)
    out = out.cpu().numpy()
    after = {n: getattr(cache, n).cpu().numpy() for n in before}
    # every row but token pos of each stream is unchanged
    keep = np.ones(bsz * hkv * rows, bool)
    keep[np.arange(bsz * hkv) * rows + pos] = False
    for n in before:
        assert np.array_equal(after[n][keep], before[n][keep]), n
    # the appended rows follow the quantiser's rules
    oc = {"codes": ref["codes"].reshape(bsz, hkv, rows, -1), "norm": ref["norm"].reshape(bsz, hkv, rows)}
    if mcode == oqz.MODE_PROD:
        oc["rnorm"] = ref["rnorm"].reshape(bsz, hkv, rows)
    ocache, want, nref = odec.append_step(oc, x64, pos, q64, ot.pi, ot.c, ot.t, mcode, scale, s_mat=ot.s)
    new_rows = np.arange(bsz * hkv) * rows + pos
    gcodes = after["codes"][new_rows]
    same = check_records(gcodes, after["norm"][new_rows],
                         after["rnorm"][new_rows] if mcode == oqz.MODE_PROD else None, nref, ot)
    if mcode == oqz.MODE_PROD:
        assert after["rnorm"][new_rows][hkv - 1] == 0
    # logits on identical records: tokens before pos always, token pos where
    # the appended record equals the oracle's
    for b in range(bsz):
        for h in range(hkv):
            qq = q64[b, h * group:(h + 1) * group]
            norm = ocache["norm"][b, h, :pos + 1]
            cols = pos + 1 if same[b * hkv + h] else pos
            gl = out[b, h * group:(h + 1) * group, :cols]
            live = norm[:cols] != 0                       # zero keys: logit exactly 0
            assert np.all(gl[:, ~live] == 0.0)
            if live.any():
                check_logits(gl[:, live], want[b, h * group:(h + 1) * group, :cols][:, live], scale,
                             norm[:cols][live], qq)
            if not x64[b, h].any():
                assert np.all(out[b, h * group:(h + 1) * group, pos] == 0.0)


def test_append_attn_logits_bounds(tq):
    d, bits = 128, 3
    ot = OracleTables(d, bits, oqz.MODE_PROD)
    ref = ot.quantize(np.random.default_rng(4).standard_normal((2 * 50, d)))
    qz = tq.Quantizer(d, bits, oqz.MODE_PROD, seed=0, device=DEV)
    cache = cache_from_oracle(tq, ref, d, bits, oqz.MODE_PROD, DEV)
    x = torch.zeros((1, 2, d), device=DEV)
    q = torch.zeros((1, 8, d), device=DEV)
    for bad in (50, -1):
        with pytest.raises(tq.TQError):
            qz.append_attn_logits(x, q, cache, n_kv_heads=2, pos=bad, scale=1.0, row_tokens=50)
    out = qz.append_attn_logits(x[:0], q[:0], cache, n_kv_heads=2, pos=3, scale=1.0, row_tokens=50)
    assert out.shape == (0, 8, 4)


# ---------------------------------------------------------------- polar format
@pytest.mark.parametrize("d,dtype", [(128, "bf16"), (128, "f32"), (64, "bf16"), (64, "f32"), (256, "bf16"),
                                     (256, "f32")])
def test_polar_quantize_parity(tq, d, dtype):
    from oracle import polar as opq
    from oracle import rotation as orot
    n = 1000
    if dtype == "bf16":
        xb = _keys_bf16(d, n, seed=3)
        x64 = _special_rows(bf16_to_f32(xb).astype(np.float64))
        xt = dev_bf16(bf16_bits(x64.astype(np.float32)), DEV)
    else:
        rng = np.random.default_rng(11)
        x64 = _special_rows((rng.standard_normal((n, d)) * np.exp(rng.standard_normal(d))).astype(np.float32)
                            .astype(np.float64))
        xt = torch.from_numpy(x64.astype(np.float32)).to(DEV)
    pi = orot.haar_rotation(d, 0)
    ref = opq.quantize(x64, pi)
    qz = tq.Quantizer(d, 3, tq.MODE_POLAR, seed=0, device=DEV)
    off = 3
    cache = qz.new_cache(n + 7)
    qz.quantize(xt, out=cache, out_offset=off)
    torch.cuda.synchronize()
    codes = cache.codes.cpu().numpy()[off:off + n]
    check_polar_codes(codes, ref, d)
    check_norms(cache.norm.cpu().numpy()[off:off + n], {"norm": ref["norm"]})
    assert not codes[3].any()                               # the zero vector: every angle 0


@pytest.mark.parametrize("d,out_dtype", [(128, "f32"), (128, "bf16"), (64, "f32"), (256, "f32"), (256, "bf16")])
def test_polar_dequantize_parity(tq, d, out_dtype):
    from oracle import polar as opq
    from oracle import rotation as orot
    n = 777
    rng = np.random.default_rng(12)
    x64 = rng.standard_normal((n, d)) * np.exp(rng.standard_normal(d))
    x64[5] = 0.0
    pi = orot.haar_rotation(d, 0)
    ref = opq.quantize(x64, pi)
    want = opq.dequantize(ref["codes"], ref["norm"], pi)
    qz = tq.Quantizer(d, 3, tq.MODE_POLAR, seed=0, device=DEV)
    cache = tq.PackedKV.from_tensors(d, 3, tq.MODE_POLAR, torch.from_numpy(ref["codes"]).to(DEV),
                                     dev_u16(ref["norm"], DEV))
    if out_dtype == "f32":
        got = qz.dequantize(cache, n).cpu().numpy()
        check_dequant(got, want)
    else:
        got = qz.dequantize(cache, n, out_dtype=torch.bfloat16).float().cpu().numpy()
        assert np.all(np.abs(got - want) <= 2.0 ** -8 * np.abs(want) + 1e-3 * np.abs(want).max(axis=1, keepdims=True))
    assert np.all(got[5] == 0.0)


def test_polar_round_trip_and_unsupported_calls(tq):
    """GPU quantise then GPU dequantise against the oracle's reconstruction of
    the GPU's own codes (decoding is exact given the codes), and the calls the
    polar format does not have."""
    from oracle import polar as opq
    from oracle import rotation as orot
    d, n = 128, 4096
    rng = np.random.default_rng(13)
    x = torch.from_numpy((rng.standard_normal((n, d)) * 2.0).astype(np.float32)).to(DEV)
    qz = tq.Quantizer(d, 3, tq.MODE_POLAR, seed=0, device=DEV)
    cache = qz.new_cache(n)
    qz.quantize(x, out=cache)
    got = qz.dequantize(cache, n).cpu().numpy()
    pi = orot.haar_rotation(d, 0)
    want = opq.dequantize(cache.codes.cpu().numpy(), cache.norm.cpu().numpy().view(np.uint16), pi)
    check_dequant(got, want)
    xs = x.cpu().numpy().astype(np.float64)
    cos = np.sum(xs * got, 1) / np.linalg.norm(xs, axis=1) / np.linalg.norm(got, axis=1)
    assert 0.98 < cos.mean() < 0.99
    # the polar format has dense one-shot logits only: no top-k, append,
    # paged or prepared-query calls
    q = torch.zeros((1, 4, d), device=DEV)
    with pytest.raises(tq.TQError):
        qz.search(q, cache, n_kv_heads=1, seq_len=n, topk=10)
    with pytest.raises(tq.TQError):
        qz.append_attn_logits(x[:1].view(1, 1, d), q, cache, n_kv_heads=1, pos=0, scale=1.0, row_tokens=n)
    with pytest.raises(tq.TQError):
        qz.prepare_queries(q, n_kv_heads=1)
    table = torch.zeros((1, n // 64), dtype=torch.int32, device=DEV)
    with pytest.raises(tq.TQError):
        qz.attn_logits_paged(q, cache, table, 64, 1, n, 1.0)


@pytest.mark.parametrize("d", [64, 256])
def test_polar_round_trip_other_widths(tq, d):
    """GPU quantise then GPU dequantise at d = 64 and 256 (6 and 8 levels):
    the reconstruction against the oracle's decoding of the GPU's own codes,
    and the codes against the oracle's."""
    from oracle import polar as opq
    from oracle import rotation as orot
    n = 2048
    rng = np.random.default_rng(14 + d)
    x64 = (rng.standard_normal((n, d)) * 2.0).astype(np.float32).astype(np.float64)
    x = torch.from_numpy(x64.astype(np.float32)).to(DEV)
    qz = tq.Quantizer(d, 3, tq.MODE_POLAR, seed=0, device=DEV)
    cache = qz.new_cache(n)
    qz.quantize(x, out=cache)
    pi = orot.haar_rotation(d, 0)
    check_polar_codes(cache.codes.cpu().numpy(), opq.quantize(x64, pi), d)
    got = qz.dequantize(cache, n).cpu().numpy()
    want = opq.dequantize(cache.codes.cpu().numpy(), cache.norm.cpu().numpy().view(np.uint16), pi)
    check_dequant(got, want)
    cos = np.sum(x64 * got, 1) / np.linalg.norm(x64, axis=1) / np.linalg.norm(got, axis=1)
    assert cos.mean() > 0.97


def test_cache_save_and_reload_round_trip(tq):
    """A packed cache is its bytes plus (d, b, mode, seed): the page keeps no
    stored constants, Pi and S regenerate from the seed.  Raw bytes copied to
    the host and back, read by a quantiser built afresh from the same seed,
    give bit-identical logits and reconstructions; another seed does not."""
    d, bits, n, hkv, group = 128, 3, 2000, 2, 4
    rng = np.random.default_rng(21)
    x = torch.from_numpy((rng.standard_normal((n, d)) * 3.0).astype(np.float32)).to(DEV)
    q = torch.from_numpy(rng.standard_normal((1, hkv * group, d)).astype(np.float32)).to(DEV)
    qz = tq.Quantizer(d, bits, tq.MODE_PROD, seed=5, device=DEV)
    cache = qz.quantize(x)
    seq = n // hkv
    want_l = qz.attn_logits(q, cache, n_kv_heads=hkv, seq_len=seq, scale=0.25).cpu().numpy()
    want_x = qz.dequantize(cache, n).cpu().numpy()
    saved = {k: getattr(cache, k).cpu().numpy().tobytes() for k in ("codes", "norm", "rnorm")}
    del cache, qz
    torch.cuda.synchronize()

    def load(name, dtype, shape):
        return torch.from_numpy(np.frombuffer(saved[name], dtype=dtype).reshape(shape).copy()).to(DEV)

    rb = bits * d // 8
    qz2 = tq.Quantizer(d, bits, tq.MODE_PROD, seed=5, device=DEV)
    cache2 = tq.PackedKV.from_tensors(d, bits, tq.MODE_PROD, load("codes", np.uint8, (n, rb)),
                                      load("norm", np.int16, (n,)), load("rnorm", np.int16, (n,)))
    got_l = qz2.attn_logits(q, cache2, n_kv_heads=hkv, seq_len=seq, scale=0.25).cpu().numpy()
    got_x = qz2.dequantize(cache2, n).cpu().numpy()
    assert np.array_equal(got_l, want_l)
    assert np.array_equal(got_x, want_x)
    qz3 = tq.Quantizer(d, bits, tq.MODE_PROD, seed=6, device=DEV)
    other = qz3.dequantize(cache2, n).cpu().numpy()
    assert not np.allclose(other, want_x, atol=1e-3)


# ---------------------------------------------------------------- paged cache
PAGED_CASES = [
    # d, bits, mode, batch, kv heads, group, page tokens, seq, append pos, q dtype
    (128, 3, "prod", 2, 3, 4, 64, 1000, 777, "bf16"),
    (128, 4, "prod", 1, 2, 4, 256, 2049, 2048, "f32"),
    (128, 2, "mse", 2, 2, 2, 128, 700, 300, "bf16"),
    (256, 2, "mse", 1, 1, 4, 64, 300, 0, "f32"),
    (64, 4, "prod", 2, 2, 8, 64, 650, 649, "bf16"),
]


def _scatter_pool(ref, d, bits, mode, bsz, hkv, seq, page_tokens, spare, seed):
    """Oracle-packed rows [bsz, hkv, seq] scattered into a pool of pages in a
    random order; unused rows hold garbage.  Returns (pool dict, table)."""
    from oracle import decode as odec
    per_seq = -(-seq // page_tokens)
    n_pages = bsz * per_seq + spare
    rng = np.random.default_rng(seed)
    table = rng.permutation(n_pages)[:bsz * per_seq].reshape(bsz, per_seq).astype(np.int32)
    rows = n_pages * hkv * page_tokens
    pool = {"codes": rng.integers(0, 256, (rows, ref["codes"].shape[1])).astype(np.uint8),
            "norm": rng.integers(0, 0x7C00, rows).astype(np.uint16)}
    if mode == oqz.MODE_PROD:
        pool["rnorm"] = rng.integers(0, 0x3C00, rows).astype(np.uint16)
    for b in range(bsz):
        for h in range(hkv):
            r = odec.paged_rows(table, page_tokens, hkv, b, h, np.arange(seq))
            src = slice((b * hkv + h) * seq, (b * hkv + h + 1) * seq)
            pool["codes"][r] = ref["codes"][src]
            pool["norm"][r] = ref["norm"][src]
            if mode == oqz.MODE_PROD:
                pool["rnorm"][r] = ref["rnorm"][src]
    return pool, table


@pytest.mark.parametrize("d,bits,mode,bsz,hkv,group,page,seq,pos,qdtype", PAGED_CASES)
def test_paged_logits_and_append_parity(tq, d, bits, mode, bsz, hkv, group, page, seq, pos, qdtype):
    """Logits over a paged pool (pages in random order, garbage in unused
    rows) against the oracle; then a decode step with append into the pool:
    the new rows follow the quantiser's rules, every other pool row stays
    bit-identical, and the logits over tokens 0..pos match the oracle's."""
    from oracle import decode as odec
    ot, mcode, keys, q64, qt, ref = _gqa_case(d, bits, mode, bsz, hkv, group, seq, qdtype)
    pool, table = _scatter_pool(ref, d, bits, mcode, bsz, hkv, seq, page, 5, seed=seq)
    qz = tq.Quantizer(d, bits, mcode, seed=0, device=DEV)
    cache = tq.PackedKV.from_tensors(d, bits, mcode, torch.from_numpy(pool["codes"]).to(DEV),
                                     dev_u16(pool["norm"], DEV),
                                     dev_u16(pool["rnorm"], DEV) if mcode == oqz.MODE_PROD else None)
    tt = torch.from_numpy(table).to(DEV)
    scale = 1.0 / np.sqrt(d)
    out = qz.attn_logits_paged(qt, cache, tt, page, hkv, seq, scale).cpu().numpy()
    codes = ref["codes"].reshape(bsz, hkv, seq, -1)
    norm = ref["norm"].reshape(bsz, hkv, seq)
    for b in range(bsz):
        for h in range(hkv):
            kw = {}
            if mcode == oqz.MODE_PROD:
                kw = dict(rnorm=ref["rnorm"].reshape(bsz, hkv, seq)[b, h], s_mat=ot.s)
            qq = q64[b, h * group:(h + 1) * group]
            want = oqz.logits_rotated(qq, codes[b, h], norm[b, h], ot.pi, ot.c, mcode, scale, **kw)
            check_logits(out[b, h * group:(h + 1) * group], want, scale, norm[b, h], qq)
    # decode step with append into the pool
    rng = np.random.default_rng(pos + 3)
    x = (rng.standard_normal((bsz, hkv, d)) * 2.0).astype(np.float32)
    x[0, 0] = 0.0
    x64 = x.astype(np.float64)
    new_pool, want, nref = odec.append_step_paged(pool, table, page, x64, pos, q64, ot.pi, ot.c, ot.t, mcode,
                                                  scale, s_mat=ot.s)
    got = qz.append_attn_logits_paged(torch.from_numpy(x).to(DEV), qt, cache, tt, page, hkv, pos, scale)
    torch.cuda.synchronize()
    got = got.cpu().numpy()
    after = {"codes": cache.codes.cpu().numpy(), "norm": cache.norm.cpu().numpy().view(np.uint16)}
    if mcode == oqz.MODE_PROD:
        after["rnorm"] = cache.rnorm.cpu().numpy().view(np.uint16)
    new_rows = np.array([odec.paged_rows(table, page, hkv, b, h, [pos])[0] for b in range(bsz) for h in range(hkv)])
    keep = np.ones(len(pool["norm"]), bool)
    keep[new_rows] = False
    for name in pool:
        assert np.array_equal(after[name][keep], pool[name][keep]), name
    same = check_records(after["codes"][new_rows], after["norm"][new_rows],
                         after["rnorm"][new_rows] if mcode == oqz.MODE_PROD else None, nref, ot)
    for b in range(bsz):
        for h in range(hkv):
            qq = q64[b, h * group:(h + 1) * group]
            rows = odec.paged_rows(table, page, hkv, b, h, np.arange(pos + 1))
            cols = pos + 1 if same[b * hkv + h] else pos
            nrm = new_pool["norm"][rows][:cols]
            live = nrm != 0
            gl = got[b, h * group:(h + 1) * group, :cols]
            assert np.all(gl[:, ~live] == 0.0)
            if live.any():
                check_logits(gl[:, live], want[b, h * group:(h + 1) * group, :cols][:, live], scale, nrm[live], qq)


PREPARED_CASES = [
    # d, bits, mode, batch, kv heads, group, seq, q dtype
    (128, 4, "prod", 2, 2, 4, 2049, "bf16"),
    (128, 3, "mse", 1, 2, 5, 1000, "f32"),
    (64, 3, "prod", 1, 2, 4, 700, "bf16"),
    (256, 2, "mse", 1, 1, 8, 513, "f32"),
]


@pytest.mark.parametrize("d,bits,mode,bsz,hkv,group,seq,qdtype", PREPARED_CASES)
def test_prepared_logits_match_one_shot(tq, d, bits, mode, bsz, hkv, group, seq, qdtype):
    """One query preparation serves three streaming calls: the cache it came
    with (checked against the oracle), a second cache scored with another
    scale, and the first cache scattered into a paged pool.  Each result equals
    the matching one-shot call bit for bit."""
    ot, mcode, keys, q64, qt, ref = _gqa_case(d, bits, mode, bsz, hkv, group, seq, qdtype)
    qz = tq.Quantizer(d, bits, mcode, seed=0, device=DEV)
    cache = cache_from_oracle(tq, ref, d, bits, mcode, DEV)
    scale = 1.0 / np.sqrt(d)
    prep = qz.prepare_queries(qt, n_kv_heads=hkv)
    got = qz.attn_logits_prepared(prep, cache, seq, scale)
    one = qz.attn_logits(qt, cache, n_kv_heads=hkv, seq_len=seq, scale=scale)
    assert torch.equal(got, one)
    got = got.cpu().numpy()
    codes = ref["codes"].reshape(bsz, hkv, seq, -1)
    norm = ref["norm"].reshape(bsz, hkv, seq)
    for b in range(bsz):
        for h in range(hkv):
            kw = {}
            if mcode == oqz.MODE_PROD:
                kw = dict(rnorm=ref["rnorm"].reshape(bsz, hkv, seq)[b, h], s_mat=ot.s)
            qq = q64[b, h * group:(h + 1) * group]
            want = oqz.logits_rotated(qq, codes[b, h], norm[b, h], ot.pi, ot.c, mcode, scale, **kw)
            check_logits(got[b, h * group:(h + 1) * group], want, scale, norm[b, h], qq)
    # a second cache (other keys, a shorter prefix of rows) and another scale
    rng = np.random.default_rng(seq + 11)
    seq2 = seq // 2 + 1
    keys2 = rng.standard_normal((bsz * hkv * seq2, d)).astype(np.float32)
    cache2 = qz.quantize(torch.from_numpy(keys2).to(DEV))
    got2 = qz.attn_logits_prepared(prep, cache2, seq2, -0.75)
    assert torch.equal(got2, qz.attn_logits(qt, cache2, n_kv_heads=hkv, seq_len=seq2, scale=-0.75))
    # the first cache as a paged pool
    page = 64
    pool, table = _scatter_pool(ref, d, bits, mcode, bsz, hkv, seq, page, 3, seed=seq + 1)
    pc = tq.PackedKV.from_tensors(d, bits, mcode, torch.from_numpy(pool["codes"]).to(DEV),
                                  dev_u16(pool["norm"], DEV),
                                  dev_u16(pool["rnorm"], DEV) if mcode == oqz.MODE_PROD else None)
    tt = torch.from_numpy(table).to(DEV)
    got3 = qz.attn_logits_prepared(prep, pc, seq, scale, block_table=tt, page_tokens=page)
    assert torch.equal(got3, qz.attn_logits_paged(qt, pc, tt, page, hkv, seq, scale))
    assert torch.equal(got3, one)


def test_prepared_queries_shared_by_two_streams(tq):
    """Tables prepared once are only read by the streaming calls: two calls
    queued on two other streams at once give the one-shot results."""
    d, bits, mode, bsz, hkv, group, seq = 128, 3, "prod", 1, 2, 4, 3000
    ot, mcode, keys, q64, qt, ref = _gqa_case(d, bits, mode, bsz, hkv, group, seq, "bf16")
    qz = tq.Quantizer(d, bits, mcode, seed=0, device=DEV)
    cache = cache_from_oracle(tq, ref, d, bits, mcode, DEV)
    one = qz.attn_logits(qt, cache, n_kv_heads=hkv, seq_len=seq, scale=0.125)
    prep = qz.prepare_queries(qt, n_kv_heads=hkv)
    torch.cuda.synchronize()
    outs = []
    streams = [torch.cuda.Stream(device=DEV) for _ in range(2)]
    for st in streams:
        with torch.cuda.stream(st):
            outs.append(qz.attn_logits_prepared(prep, cache, seq, 0.125))
    torch.cuda.synchronize()
    for o in outs:
        assert torch.equal(o, one)


POLAR_LOGIT_CASES = [
    # d, batch, kv heads, group, seq, q dtype
    (128, 1, 2, 4, 3000, "bf16"),
    (128, 2, 1, 8, 1000, "f32"),
    (128, 1, 1, 1, 257, "f32"),
    (64, 1, 2, 3, 777, "bf16"),
    (64, 1, 1, 16, 513, "f32"),
    (256, 1, 2, 4, 700, "bf16"),
    (256, 1, 1, 12, 300, "f32"),
]


@pytest.mark.parametrize("d,bsz,hkv,group,seq,qdtype", POLAR_LOGIT_CASES)
def test_polar_logits_parity(tq, d, bsz, hkv, group, seq, qdtype):
    """Dense logits from oracle-packed polar keys (zero rows included) against
    the oracle's definition, scale * <q, x_hat>: GQA groups 1 to 16, ragged
    lengths, bf16 and fp32 queries, d = 64, 128, 256."""
    from oracle import polar as opq
    from oracle import rotation as orot
    pi = orot.haar_rotation(d, 0)
    rng = np.random.default_rng(200 + seq + group)
    scales = np.exp(rng.standard_normal((hkv, d)))
    keys = (rng.standard_normal((bsz, hkv, seq, d)) * scales[None, :, None, :]).reshape(-1, d)
    keys[5] = 0.0
    ref = opq.quantize(keys, pi)
    q = rng.standard_normal((bsz, hkv * group, d)) * np.repeat(scales, group, axis=0)[None]
    if qdtype == "bf16":
        qb = bf16_bits(q.astype(np.float32))
        q64 = bf16_to_f32(qb).astype(np.float64)
        qt = dev_bf16(qb, DEV)
    else:
        q64 = q.astype(np.float32).astype(np.float64)
        qt = torch.from_numpy(q64.astype(np.float32)).to(DEV)
    qz = tq.Quantizer(d, 3, tq.MODE_POLAR, seed=0, device=DEV)
    cache = tq.PackedKV.from_tensors(d, 3, tq.MODE_POLAR, torch.from_numpy(ref["codes"]).to(DEV),
                                     dev_u16(ref["norm"], DEV))
    scale = 1.0 / np.sqrt(d)
    out = qz.attn_logits(qt, cache, n_kv_heads=hkv, seq_len=seq, scale=scale).cpu().numpy()
    codes = ref["codes"].reshape(bsz, hkv, seq, -1)
    norm = ref["norm"].reshape(bsz, hkv, seq)
    for b in range(bsz):
        for h in range(hkv):
            qq = q64[b, h * group:(h + 1) * group]
            want = opq.logits(qq, codes[b, h], norm[b, h], pi, scale)
            live = norm[b, h] != 0                     # zero keys: logit exactly 0
            got = out[b, h * group:(h + 1) * group]
            check_logits(got[:, live], want[:, live], scale, norm[b, h][live], qq)
            assert np.all(got[:, ~live] == 0.0)
    assert norm[0, 0, 5] == 0


def test_polar_logits_end_to_end_and_row_capacity(tq):
    """GPU polar quantisation, then logits over streams of capacity 600 holding
    437 tokens, against the oracle's logits of the GPU's own codes (decoding
    is exact given the codes) and against the unquantised inner products
    (cosine of the logit rows)."""
    from oracle import polar as opq
    from oracle import rotation as orot
    d, hkv, group, cap, seq = 128, 2, 4, 600, 437
    rng = np.random.default_rng(77)
    x = (rng.standard_normal((hkv * cap, d)) * 1.5).astype(np.float32)
    qz = tq.Quantizer(d, 3, tq.MODE_POLAR, seed=0, device=DEV)
    cache = qz.quantize(torch.from_numpy(x).to(DEV))
    q = rng.standard_normal((1, hkv * group, d)).astype(np.float32)
    out = qz.attn_logits(torch.from_numpy(q).to(DEV), cache, n_kv_heads=hkv, seq_len=seq, scale=1.0,
                         row_tokens=cap).cpu().numpy()
    assert out.shape == (1, hkv * group, seq)
    pi = orot.haar_rotation(d, 0)
    codes = cache.codes.cpu().numpy()
    norm = cache.norm.cpu().numpy().view(np.uint16)
    for h in range(hkv):
        sl = slice(h * cap, h * cap + seq)
        qq = q[0, h * group:(h + 1) * group].astype(np.float64)
        want = opq.logits(qq, codes[sl], norm[sl], pi, 1.0)
        check_logits(out[0, h * group:(h + 1) * group], want, 1.0, norm[sl], qq)
        exact = qq @ x[sl].astype(np.float64).T
        cos = np.sum(exact * want, 1) / np.linalg.norm(exact, axis=1) / np.linalg.norm(want, axis=1)
        assert np.all(cos > 0.95)
