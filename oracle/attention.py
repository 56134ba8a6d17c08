"""Decode attention output over a quantised value cache (fp64).

Test infrastructure: only the tests, the smoke check and the benchmark's CPU
baseline use this module; the GPU path never calls it.

Page "TurboQuant 설명: 무엇인지와 LLM 메모리 6배 절약 구현 방법":
* section "TurboQuant란 무엇인가요?": the KV cache holds the key and the value
  vectors of every token, and both are what the method compresses;
* section "2단계: QJL 잔차 보정", closing paragraph: attention is computed from
  the compressed indices, without a full dequantisation during inference.

Reading (the page does not write the attention out): the decode attention
output of query head h is o_h = sum_t p_t v_hat_t with p = softmax(l_h) over
the seq_len valid tokens, l_h the attention logits of the head and v_hat the
dequantised value vectors of its KV head (grouped-query attention: query head
h reads KV head h // (Hq / Hkv)).  A row of logits that is entirely -inf (a
fully masked query) gives o_h = 0.

``attn_output`` follows that definition literally: dequantise the values,
then weight them.  ``attn_output_rotated`` is the same value in the rotated
domain, o_h = n-weighted sum of centroid rows, rotated back once:
o_h = Pi^T (sum_t p_t n_t c[idx_t]) / sum_t p_t (MSE-mode values), which is how
the device computes it; the tests check the two against each other.
"""

import math

import numpy as np

from . import quantizer as qz


def softmax_weights(logits):
    """Unnormalised weights exp(l - max l) and their sum; (None, 0) if all -inf."""
    l = np.asarray(logits, dtype=np.float64)
    m = np.max(l)
    if m == -np.inf:
        return None, 0.0
    p = np.exp(l - m)
    return p, float(np.sum(p))


def attn_output(logits, cache, pi, centroids, mode, s_mat=None, seq_len=None):
    """o [B, Hq, d] for logits [B, Hq, T] over a packed value cache.

    ``cache`` holds ``codes`` [B, Hkv, T, row], ``norm`` [B, Hkv, T] and, in
    prod mode, ``rnorm`` [B, Hkv, T].
    """
    logits = np.asarray(logits, dtype=np.float64)
    bsz, hq, _ = logits.shape
    hkv = cache["codes"].shape[1]
    t_len = cache["codes"].shape[2] if seq_len is None else seq_len
    group = hq // hkv
    d = pi.shape[0]
    out = np.zeros((bsz, hq, d))
    for b in range(bsz):
        for h in range(hkv):
            kw = {}
            if mode == qz.MODE_PROD:
                kw = dict(rnorm=cache["rnorm"][b, h, :t_len], s_mat=s_mat)
            vhat = qz.dequantize(cache["codes"][b, h, :t_len], cache["norm"][b, h, :t_len], pi,
                                 centroids, mode, **kw)
            for g in range(group):
                p, s = softmax_weights(logits[b, h * group + g, :t_len])
                if p is not None:
                    out[b, h * group + g] = (p @ vhat) / s
    return out


def attn_output_rotated(logits, codes, norm, pi, centroids):
    """Rotated-domain form for one KV head (MSE-mode values): [G, d] from [G, T]."""
    c = np.asarray(centroids, dtype=np.float64)
    d = pi.shape[0]
    nbits = int(round(math.log2(c.size)))
    idx, _ = qz.unpack_records(codes, nbits, qz.MODE_MSE, d)
    rows = qz.from_fp16_bits(norm)[:, None] * c[idx]          # n_t c[idx_t], rotated domain
    logits = np.asarray(logits, dtype=np.float64)
    out = np.zeros((logits.shape[0], d))
    for g in range(logits.shape[0]):
        p, s = softmax_weights(logits[g])
        if p is not None:
            out[g] = ((p @ rows) / s) @ pi                    # Pi^T applied once
    return out
