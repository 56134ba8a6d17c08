"""Decode step with append over a packed key cache (fp64).

Test infrastructure: only the tests, the smoke check and the benchmark's CPU
baseline use this module; the GPU path never calls it.

Page "TurboQuant 설명: 무엇인지와 LLM 메모리 6배 절약 구현 방법":
* section "TurboQuant 구현 방법": the key of every new token is quantised
  when the cache is updated, and logits are then formed against the query
  rotated once;
* sections "TurboQuant 작동 방식" and "터보퀀트 vs. 전통적인 양자화 방법": the
  method is online and data-oblivious, so quantising a vector never depends on
  the other vectors of the cache.

Reading: a decode step writes the packed new key of every (batch, KV head)
stream at token ``pos`` of a preallocated cache (rows of ``row_tokens``
tokens per stream; the other rows are left as they are) and returns the
logits of the step's queries over tokens 0..pos.
"""

import numpy as np

from . import quantizer as qz


def append_step(cache, x_new, pos, q, pi, centroids, boundaries, mode, scale, s_mat=None):
    """One decode step.

    ``cache``: dict with ``codes`` [B, Hkv, R, row] (uint8), ``norm`` [B, Hkv, R]
    (fp16 bits) and, in prod mode, ``rnorm``; ``x_new`` [B, Hkv, d]; ``q``
    [B, Hq, d].  Returns (updated copy of the cache, logits [B, Hq, pos + 1],
    the quantiser's record of the new keys).
    """
    x_new = np.asarray(x_new, dtype=np.float64)
    bsz, hkv, d = x_new.shape
    rows = cache["codes"].shape[2]
    if not 0 <= pos < rows:
        raise ValueError("pos outside the cache")
    ref = qz.quantize(x_new.reshape(-1, d), pi, centroids, boundaries, mode, s_mat=s_mat)
    out = {k: v.copy() for k, v in cache.items()}
    out["codes"][:, :, pos] = ref["codes"].reshape(bsz, hkv, -1)
    out["norm"][:, :, pos] = ref["norm"].reshape(bsz, hkv)
    if mode == qz.MODE_PROD:
        out["rnorm"][:, :, pos] = ref["rnorm"].reshape(bsz, hkv)
    q = np.asarray(q, dtype=np.float64)
    hq = q.shape[1]
    group = hq // hkv
    logits = np.zeros((bsz, hq, pos + 1))
    for b in range(bsz):
        for h in range(hkv):
            kw = {}
            if mode == qz.MODE_PROD:
                kw = dict(rnorm=out["rnorm"][b, h, :pos + 1], s_mat=s_mat)
            logits[b, h * group:(h + 1) * group] = qz.logits_rotated(
                q[b, h * group:(h + 1) * group], out["codes"][b, h, :pos + 1], out["norm"][b, h, :pos + 1],
                pi, centroids, mode, scale, **kw)
    return out, logits, ref


# ------------------------------------------------------------- paged cache
# Reading (the page says only that the cache is updated with every new token,
# section "TurboQuant 구현 방법"): a serving cache is a pool of pages of P
# tokens; page g of the pool holds the rows of every KV head for its P tokens,
# head-major: pool row (g * Hkv + h) * P + (t mod P) holds token t of KV
# head h of a sequence whose block-table entry t // P is g.  Sequences own
# disjoint pages in any order; the packed record of a token does not depend
# on where it is stored.

def paged_rows(block_table, page_tokens, n_kv_heads, b, h, tokens):
    """Pool rows of ``tokens`` of KV head h of sequence b."""
    tokens = np.asarray(tokens, dtype=np.int64)
    pages = np.asarray(block_table, dtype=np.int64)[b, tokens // page_tokens]
    return (pages * n_kv_heads + h) * page_tokens + tokens % page_tokens


def gather_paged(pool, block_table, page_tokens, n_kv_heads, seq_len):
    """The contiguous cache view ([B, Hkv, seq_len, ...] for every field of
    ``pool``) of the first seq_len tokens of every sequence."""
    bsz = np.asarray(block_table).shape[0]
    out = {}
    for name, arr in pool.items():
        view = np.empty((bsz, n_kv_heads, seq_len) + arr.shape[1:], dtype=arr.dtype)
        for b in range(bsz):
            for h in range(n_kv_heads):
                view[b, h] = arr[paged_rows(block_table, page_tokens, n_kv_heads, b, h, np.arange(seq_len))]
        out[name] = view
    return out


def append_step_paged(pool, block_table, page_tokens, x_new, pos, q, pi, centroids, boundaries, mode, scale,
                      s_mat=None):
    """One decode step on a paged cache: the new key of every (sequence, KV
    head) goes to its pool row for token ``pos``; the logits of the step's
    queries cover tokens 0..pos read through the block table.

    ``pool``: dict with ``codes`` [rows, row bytes], ``norm`` [rows] and, in
    prod mode, ``rnorm``; ``block_table`` [B, max_pages]; ``x_new`` [B, Hkv, d];
    ``q`` [B, Hq, d].  Returns (updated copy of the pool, logits [B, Hq, pos + 1],
    the quantiser's record of the new keys).
    """
    x_new = np.asarray(x_new, dtype=np.float64)
    bsz, hkv, d = x_new.shape
    ref = qz.quantize(x_new.reshape(-1, d), pi, centroids, boundaries, mode, s_mat=s_mat)
    out = {k: v.copy() for k, v in pool.items()}
    for b in range(bsz):
        for h in range(hkv):
            row = paged_rows(block_table, page_tokens, hkv, b, h, [pos])[0]
            out["codes"][row] = ref["codes"][b * hkv + h]
            out["norm"][row] = ref["norm"][b * hkv + h]
            if mode == qz.MODE_PROD:
                out["rnorm"][row] = ref["rnorm"][b * hkv + h]
    q = np.asarray(q, dtype=np.float64)
    hq = q.shape[1]
    group = hq // hkv
    logits = np.zeros((bsz, hq, pos + 1))
    for b in range(bsz):
        for h in range(hkv):
            rows = paged_rows(block_table, page_tokens, hkv, b, h, np.arange(pos + 1))
            kw = {}
            if mode == qz.MODE_PROD:
                kw = dict(rnorm=out["rnorm"][rows], s_mat=s_mat)
            logits[b, h * group:(h + 1) * group] = qz.logits_rotated(
                q[b, h * group:(h + 1) * group], out["codes"][rows], out["norm"][rows], pi, centroids, mode,
                scale, **kw)
    return out, logits, ref
