"""Seeded synthetic workloads shared by the tests, the oracle checks and bench.py.

This module holds no arithmetic of the quantiser: it only draws inputs.  The
pages measure on model KV caches (Gemma / Mistral / Llama / Qwen families on
LongBench, needle-in-a-haystack, RULER) and on GloVe-200 vector search; none of
those weights or datasets is available, so every input is drawn here with the
shapes and value distributions of those workloads.

Randomness: numpy ``SeedSequence(seed, spawn_key=(config, tensor, batch,
head))`` streams, so any (batch, head) slice can be regenerated on its own.
bf16 values are produced by round-to-nearest-even of fp32 through bit
manipulation and returned as raw uint16 bits.
"""

import numpy as np

TENSOR_CODES = {"k": 1, "v": 2, "q": 3, "scales_k": 4, "scales_v": 5, "db": 6,
                "dbq": 7, "sigma": 8}

# name -> parameters of the five workloads
CONFIGS = {
    "tiny": dict(cfg=1, d=128, n_keys=4096, n_queries=16, bits=3, mode="mse",
                 dtype="f32", outlier_channels=2, outlier_scale=10.0),
    "decode": dict(cfg=2, d=128, batch=1, kv_heads=8, q_heads=32, seq=32768,
                   k_bits=3, k_mode="prod", v_bits=3, v_mode="mse", dtype="bf16"),
    "long_context": dict(cfg=3, d=128, batch=8, kv_heads=8, q_heads=32, seq=131072,
                         k_bits=4, k_mode="prod", dtype="bf16"),
    "prefill": dict(cfg=4, d=128, tokens=65536, kv_heads=8, bits_sweep=(2, 3, 4),
                    k_mode="prod", v_mode="mse", dtype="bf16"),
    "search": dict(cfg=5, d=200, d_pad=256, n_db=1_000_000, n_queries=10_000,
                   bits_sweep=(2, 4), mode="mse", dtype="f32", topk=10),
}


def _rng(seed, cfg, tensor, batch=0, head=0):
    ss = np.random.SeedSequence(seed, spawn_key=(cfg, TENSOR_CODES[tensor], batch, head))
    return np.random.default_rng(ss)


def bf16_bits(x):
    """fp32 -> bf16 raw bits, round to nearest even (finite inputs)."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    r = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return r.astype(np.uint16)


def bf16_to_f32(bits):
    """bf16 raw bits -> fp32 (exact)."""
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


# ---------------------------------------------------------------- config 1
def tiny_keys_queries(seed=0, n_keys=4096, n_queries=16, d=128):
    """fp32 keys and queries ~ N(0,1) with 2 of the d channels scaled x10."""
    rng = _rng(seed, 1, "scales_k")
    ch = rng.choice(d, 2, replace=False)
    scale = np.ones(d)
    scale[ch] = 10.0
    k = (_rng(seed, 1, "k").standard_normal((n_keys, d)) * scale).astype(np.float32)
    q = (_rng(seed, 1, "q").standard_normal((n_queries, d)) * scale).astype(np.float32)
    return k, q


# --------------------------------------------------------- configs 2, 3, 4
def channel_scales(seed, cfg, tensor, kv_heads, d, n_outliers=None, outlier_scale=20.0):
    """Per (head, dim) scales exp(N(0,1)); 1% of the H*d channels scaled x20."""
    rng = _rng(seed, cfg, "scales_" + tensor)
    s = np.exp(rng.standard_normal((kv_heads, d)))
    n_ch = kv_heads * d
    n_out = max(1, round(0.01 * n_ch)) if n_outliers is None else n_outliers
    flat = s.reshape(-1)
    flat[rng.choice(n_ch, n_out, replace=False)] *= outlier_scale
    return s


def kv_block(seed, cfg, tensor, batch, head, tokens, scales, start=0):
    """bf16 bits [tokens, d] for one (batch, head) stream: scale * N(0,1).

    ``start`` skips the first tokens of the stream so a slice can be drawn on
    its own (the stream is drawn in blocks of 4096 tokens).
    """
    d = scales.shape[1]
    out = np.empty((tokens, d), dtype=np.uint16)
    blk = 4096
    first = start // blk
    last = (start + tokens + blk - 1) // blk
    pos = 0
    for b in range(first, last):
        rng = _rng(seed, cfg, tensor, batch, head * 65536 + b)
        vals = (rng.standard_normal((blk, d)) * scales[head]).astype(np.float32)
        lo = max(start, b * blk) - b * blk
        hi = min(start + tokens, (b + 1) * blk) - b * blk
        out[pos:pos + hi - lo] = bf16_bits(vals[lo:hi])
        pos += hi - lo
    return out


def gqa_queries(seed, cfg, batch, q_heads, kv_heads, k_scales):
    """bf16 bits [batch, q_heads, d]; head h uses KV head h // (q_heads/kv_heads)'s K scales."""
    group = q_heads // kv_heads
    d = k_scales.shape[1]
    out = np.empty((batch, q_heads, d), dtype=np.uint16)
    for b in range(batch):
        rng = _rng(seed, cfg, "q", b)
        z = rng.standard_normal((q_heads, d))
        for h in range(q_heads):
            out[b, h] = bf16_bits((z[h] * k_scales[h // group]).astype(np.float32))
    return out


# ---------------------------------------------------------------- config 5
def search_sigma(seed, d=200):
    """Per-dimension standard deviations ~ U[0.1, 3], shared by db and queries."""
    return _rng(seed, 5, "sigma").uniform(0.1, 3.0, d)


def search_vectors(seed, tensor, start, count, d=200, d_pad=256, block=65536):
    """Rows [start, start+count) of the unit-normalised anisotropic Gaussian set.

    Returns fp32 [count, d_pad], zero-padded past ``d``.  Rows are drawn in
    blocks of ``block`` so any slice is reproducible.
    """
    sigma = search_sigma(seed, d)
    out = np.zeros((count, d_pad), dtype=np.float32)
    first = start // block
    last = (start + count + block - 1) // block
    pos = 0
    for b in range(first, last):
        rng = _rng(seed, 5, tensor, b)
        v = rng.standard_normal((block, d)) * sigma
        v /= np.sqrt(np.einsum("ij,ij->i", v, v))[:, None]
        lo = max(start, b * block) - b * block
        hi = min(start + count, (b + 1) * block) - b * block
        out[pos:pos + hi - lo, :d] = v[lo:hi].astype(np.float32)
        pos += hi - lo
    return out


# ------------------------------------------------- device-side draws (torch)
def device_kv(torch, seed, cfg, tensor, batch, heads, tokens, d, device):
    """bf16 [batch * heads * tokens, d] drawn on the device: the channel scales
    of ``channel_scales`` (lognormal, 1% outliers x20) times N(0,1) from torch's
    seeded Philox generator, rounded to bf16 (nearest even).  For workloads too
    large to draw on the host; a test that needs some of the values for the
    oracle copies those rows back."""
    sc = torch.tensor(channel_scales(seed, cfg, tensor, heads, d), dtype=torch.float32, device=device)
    gen = torch.Generator(device=device)
    gen.manual_seed(1000 * seed + 10 * cfg + TENSOR_CODES[tensor])
    out = torch.empty((batch, heads, tokens, d), dtype=torch.bfloat16, device=device)
    for b in range(batch):
        z = torch.randn((heads, tokens, d), generator=gen, device=device)
        out[b] = (z * sc[:, None, :]).to(torch.bfloat16)
        del z
    return out.view(-1, d)


def device_queries(torch, seed, cfg, batch, q_heads, kv_heads, d, device):
    """bf16 [batch, q_heads, d] on the device, query head h scaled like KV head
    h // (q_heads / kv_heads) (same channel scales as the keys)."""
    group = q_heads // kv_heads
    sc = torch.tensor(channel_scales(seed, cfg, "k", kv_heads, d), dtype=torch.float32, device=device)
    gen = torch.Generator(device=device)
    gen.manual_seed(1000 * seed + 10 * cfg + TENSOR_CODES["q"])
    z = torch.randn((batch, q_heads, d), generator=gen, device=device)
    return (z * sc.repeat_interleave(group, dim=0)[None]).to(torch.bfloat16)
