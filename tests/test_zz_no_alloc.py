"""The entry point that allocates nothing (tq_attn_output_noalloc), through the C ABI.

Its output must equal tq_attn_output's on the same inputs (same kernels; the
partials only live elsewhere), on two calls in a row, the second with a
smaller input, so the second reads a fixed array that still holds the first
call's partials.  The oracle bar (as for tq_attn_output) is checked too.
"""

import numpy as np
import pytest
import torch

from oracle import attention as oatt
from oracle import quantizer as oqz
from parity import OracleTables, cache_from_oracle

pytestmark = pytest.mark.gpu

DEV = torch.device("cuda:0")


def _case(tq, d, bits, batch, hkv, group, seq, seed):
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((batch * hkv * seq, d)) * rng.uniform(0.2, 4.0, (batch * hkv * seq, 1))
    ot = OracleTables(d, bits, oqz.MODE_MSE)
    ref = ot.quantize(x)
    cache = cache_from_oracle(tq, ref, d, bits, oqz.MODE_MSE, DEV)
    logits = (rng.standard_normal((batch, hkv * group, seq)) * 3.0).astype(np.float32)
    logits[:, :, rng.integers(0, seq, max(1, seq // 9))] = -np.inf
    want = oatt.attn_output(logits.astype(np.float64),
                            {"codes": ref["codes"].reshape(batch, hkv, seq, -1),
                             "norm": ref["norm"].reshape(batch, hkv, seq)}, ot.pi, ot.c, oqz.MODE_MSE)
    return cache, torch.from_numpy(logits).to(DEV), want


def test_noalloc_matches_workspace_call_twice():
    import online_vector_quantization_amd as tq
    d, bits = 128, 3
    qz = tq.Quantizer(d, bits, oqz.MODE_MSE, seed=0, device=DEV)
    # first call: the decode shape (8 KV heads x 4 query heads, 32768 tokens);
    # second: smaller (2 KV heads x 2 query heads, 1000 tokens)
    for batch, hkv, group, seq, seed in ((1, 8, 4, 32768, 1), (1, 2, 2, 1000, 2)):
        assert qz.attn_output_workspace_size(batch, hkv * group, hkv, seq) <= tq.NOALLOC_SCRATCH_BYTES
        cache, lt, want = _case(tq, d, bits, batch, hkv, group, seq, seed)
        outs = {}
        for out_dtype in (torch.float32, torch.bfloat16):
            ref_out = qz.attn_output(lt, cache, hkv, seq, out_dtype=out_dtype)
            out = torch.full_like(ref_out, 7.0)
            qz.attn_output_noalloc(lt, cache, hkv, seq, out)
            torch.cuda.synchronize()
            assert torch.equal(out, ref_out), (seq, out_dtype)
            outs[out_dtype] = out
        got = outs[torch.float32].cpu().numpy()
        err = np.linalg.norm(got - want, axis=2)
        assert np.all(err <= 1e-4 * np.linalg.norm(want, axis=2) + 1e-6)


def test_noalloc_refuses_oversized_partials():
    import online_vector_quantization_amd as tq
    d, bits = 256, 3
    qz = tq.Quantizer(d, bits, oqz.MODE_MSE, seed=0, device=DEV)
    batch, hkv, group, seq = 64, 64, 16, 256
    assert qz.attn_output_workspace_size(batch, hkv * group, hkv, seq) > tq.NOALLOC_SCRATCH_BYTES
    cache = qz.new_cache(batch * hkv * seq)
    lt = torch.zeros((batch, hkv * group, seq), device=DEV)
    out = torch.zeros((batch, hkv * group, d), device=DEV)
    with pytest.raises(tq.TQError) as e:
        qz.attn_output_noalloc(lt, cache, hkv, seq, out)
    assert e.value.status == tq.TQ_ERR_UNSUPPORTED
