"""Benchmark of the online KV-cache quantizer hot path on one MI355X.

python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload decode|prefill|search]

Without --warmup the untimed warmup runs as many steps as take about one
second (at least 5): the GPU reaches its sustained clock only after that much
load, and the timed steps then measure the sustained rate.  The line reports
the warmup steps actually run.

A step is one pass of the whole path over one batch of synthetic input:
quantise the keys (inner-product mode) and the values (MSE mode), compute the
attention logits of every query head straight from the packed keys, and
reconstruct the values.  The default workload is the decode step of one
layer: batch 1, 8 KV heads x head_dim 128, 32768 cached bf16 tokens, keys and
values at 3 bits, 32 query heads (GQA 4:1).  ``value`` is attention-logit
keys per second of the whole step (cached keys / step time) with every input
resident in HBM.  The line also carries the roofline of the dominant kernel
(algorithmic bytes per launch / its mean duration, measured with HIP events
on the launch stream), the fp64 CPU oracle timed on a bounded sample of the
same workload, a per-call breakdown, the long-context logit leg (batch 8,
8 KV heads, 131072 tokens, 4-bit keys) and, timed beside the step, the decode
attention output softmax(logits) . V straight from the packed values.

Two more workloads print a line of the same form: ``prefill`` quantises
65536 new bf16 tokens x 8 KV heads (keys inner-product, values MSE) at b = 2,
3 and 4 (value: vectors/s, roofline against the fp16 MFMA peak), and
``search`` scores 10^4 queries against 10^6 quantised unit vectors (d = 200
padded to 256, MSE b = 2 and 4) with a fused top-10 (value: query-key scores
per second, roofline against the fp16 MFMA peak).

Only one GPU is used; --gpus above 1 exits with a message.
"""

import argparse
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "attention-logit keys/s + HBM GB/s on packed 3-bit KV; quantize vectors/s"
HBM_PEAK_GBS = 8000.0
MFMA_F16_PEAK_TFS = 2500.0
PROFILES = os.path.join(ROOT, "profiles")
CSRC = os.path.join(ROOT, "online_vector_quantization_amd", "csrc")
WARMUP_S = 1.0      # default untimed warmup: the clocks settle under about a second of load


def _args():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=None,
                    help="untimed warmup steps (default: as many as take about one second, at least 5; "
                         "the GPU reaches its sustained clock only under sustained load)")
    ap.add_argument("--workload", default="decode", choices=["decode", "prefill", "search"])
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-long-context", action="store_true")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="run one 512 MiB device copy first (reference kernel for HBM counters)")
    return ap.parse_args()


def _source_hash(files):
    h = hashlib.sha256()
    for f in files:
        with open(os.path.join(CSRC, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def _traffic(kernel, src_files):
    """HBM bytes per launch from committed counter summaries, or None.

    profiles/hbm_traffic.json maps a kernel to FETCH_SIZE / WRITE_SIZE per
    dispatch (KiB), the copy-kernel scale factor and the hash of the sources
    the counters were taken on; a changed source makes the figure stale.
    """
    path = os.path.join(PROFILES, "hbm_traffic.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        table = json.load(f)
    ent = table.get(kernel)
    if not ent or ent.get("source_sha") != _source_hash(src_files):
        return None
    kib = ent["fetch_kib"] * ent["fetch_scale"] + ent["write_kib"] * ent["write_scale"]
    return kib * 1024.0


class Timer:
    """Mean duration of a callable over n launches, HIP events on the current stream."""

    def __init__(self, torch):
        self.torch = torch

    def __call__(self, fn, n):
        t = self.torch
        start = t.cuda.Event(enable_timing=True)
        end = t.cuda.Event(enable_timing=True)
        t.cuda.synchronize()
        start.record()
        for _ in range(n):
            fn()
        end.record()
        t.cuda.synchronize()
        return start.elapsed_time(end) * 1e-3 / n


def _host_kv(torch, seed, cfg, tensor, heads, tokens, d, device):
    """bf16 [heads*tokens, d] from the shared numpy recipe (reproducible on the host)."""
    import numpy as np
    from synthetic import channel_scales, kv_block
    sc = channel_scales(seed, cfg, tensor, heads, d)
    blocks = [kv_block(seed, cfg, tensor, 0, h, tokens, sc) for h in range(heads)]
    arr = np.concatenate(blocks, axis=0)
    return torch.from_numpy(arr.view(np.int16)).to(device).view(torch.bfloat16), sc


def decode_workload(torch, tq, args, device):
    import numpy as np
    from synthetic import bf16_to_f32, gqa_queries
    d, heads, qheads, seq, bits = 128, 8, 32, 32768, 3
    n = heads * seq
    k, ksc = _host_kv(torch, 0, 2, "k", heads, seq, d, device)
    v, _ = _host_kv(torch, 0, 2, "v", heads, seq, d, device)
    qb = gqa_queries(0, 2, 1, qheads, heads, ksc)
    q = torch.from_numpy(qb.view(np.int16)).to(device).view(torch.bfloat16)
    qk = tq.Quantizer(d, bits, tq.MODE_PROD, seed=0, device=device)
    qv = tq.Quantizer(d, bits, tq.MODE_MSE, seed=0, device=device)
    ck, cv = qk.new_cache(n), qv.new_cache(n)
    logits = torch.empty((1, qheads, seq), dtype=torch.float32, device=device)
    vhat = torch.empty((n, d), dtype=torch.bfloat16, device=device)
    scale = 1.0 / math.sqrt(d)
    calls = {
        "quantize_k": lambda: qk.quantize(k, out=ck),
        "quantize_v": lambda: qv.quantize(v, out=cv),
        "attn_logits": lambda: qk.attn_logits(q, ck, heads, seq, scale, out=logits),
        "dequantize_v": lambda: qv.dequantize(cv, n, out=vhat),
    }
    rb_k, rb_v = bits * d // 8 + 4, bits * d // 8 + 2
    work = {  # algorithmic HBM bytes and flops per launch, main kernel, sources
        "quantize_k": (n * (2 * d + rb_k), n * 4 * d * d, "quantize_pc_kernel",
                       ["quantize.hip", "tq_device.h"]),
        "quantize_v": (n * (2 * d + rb_v), n * 2 * d * d, "quantize_kernel",
                       ["quantize.hip", "tq_device.h"]),
        "attn_logits": (n * (rb_k + 4 * (qheads // heads)) + qheads * d * 2, None, "logit_kernel",
                        ["logits.hip", "tq_device.h"]),
        "dequantize_v": (n * (rb_v + 2 * d), n * 2 * d * d, "dequant_kernel",
                         ["dequant.hip", "tq_device.h"]),
    }
    cfg = {"workload": "decode step: 1 layer, batch 1, 8 KV heads x 128, 32768 bf16 tokens; "
                       "keys inner-product b=3, values MSE b=3; 32 query heads (GQA 4:1)",
           "batch": 1, "kv_heads": heads, "q_heads": qheads, "head_dim": d, "seq_len": seq,
           "key_bits": bits, "value_bits": bits, "units_per_step": n}
    # Timed beside the step, not in it: the attention output softmax(l) . V
    # straight from the packed values, on the step's logits.
    attn = torch.empty((1, qheads, d), dtype=torch.float32, device=device)
    # The decode step with append: the new key of every head (here token
    # seq - 1 again, so the cache is unchanged) quantised into the cache by the
    # logit call, then logits over all seq tokens.
    x_new = k.view(heads, seq, d)[:, seq - 1].contiguous().view(1, heads, d)
    logits2 = torch.empty_like(logits)
    extras = {"attn_output": (lambda: qv.attn_output(logits, cv, heads, seq, out=attn),
                              n * rb_v + qheads * seq * 4 + qheads * d * 4, "attend_mfma_kernel",
                              ["attend.hip", "tq_device.h"]),
              "append_attn_logits": (lambda: qk.append_attn_logits(x_new, q, ck, heads, seq - 1, scale,
                                                                   row_tokens=seq, out=logits2),
                                     n * (rb_k + 4 * (qheads // heads)) + qheads * d * 2 + heads * (2 * d + rb_k),
                                     "logit_kernel", ["logits.hip", "tq_device.h"])}
    # The PolarQuant variant of stage 1 on the same values (3 bits per coordinate).
    qp = tq.Quantizer(d, 3, tq.MODE_POLAR, seed=0, device=device)
    cp = qp.new_cache(n)
    vhat_p = torch.empty((n, d), dtype=torch.bfloat16, device=device)
    rb_p = 3 * d // 8 + 2
    extras["polar_quantize"] = (lambda: qp.quantize(v, out=cp), n * (2 * d + rb_p), "quantize_polar_kernel",
                                ["quantize.hip", "tq_device.h"])
    extras["polar_dequantize"] = (lambda: qp.dequantize(cp, n, out=vhat_p), n * (rb_p + 2 * d), "dequant_kernel",
                                  ["dequant.hip", "tq_device.h"])
    return calls, work, cfg, n, extras


def prefill_workload(torch, tq, args, device):
    d, heads, tokens = 128, 8, 65536
    n = heads * tokens
    k, _ = _host_kv(torch, 0, 4, "k", heads, tokens, d, device)
    v, _ = _host_kv(torch, 0, 4, "v", heads, tokens, d, device)
    calls, work = {}, {}
    src = ["quantize.hip", "tq_device.h"]
    for b in (2, 3, 4):
        qk = tq.Quantizer(d, b, tq.MODE_PROD, seed=0, device=device)
        qv = tq.Quantizer(d, b, tq.MODE_MSE, seed=0, device=device)
        ck, cv = qk.new_cache(n), qv.new_cache(n)
        calls["quantize_k_b%d" % b] = lambda qk=qk, ck=ck: qk.quantize(k, out=ck)
        calls["quantize_v_b%d" % b] = lambda qv=qv, cv=cv: qv.quantize(v, out=cv)
        rb = b * d // 8
        work["quantize_k_b%d" % b] = (n * (2 * d + rb + 4), n * 4 * d * d, "quantize_pc_kernel", src)
        work["quantize_v_b%d" % b] = (n * (2 * d + rb + 2), n * 2 * d * d, "quantize_kernel", src)
    cfg = {"workload": "prefill quantisation: 65536 new bf16 tokens x 8 KV heads x 128; keys "
                       "inner-product and values MSE at b = 2, 3, 4 (six calls per step)",
           "tokens": tokens, "kv_heads": heads, "head_dim": d, "bits": [2, 3, 4],
           "units_per_step": 6 * n}
    return calls, work, cfg, 6 * n, {}


def search_workload(torch, tq, args, device):
    from synthetic import search_vectors
    d, n_db, n_q, k = 256, 1_000_000, 10_000, 10
    db = torch.from_numpy(search_vectors(0, "db", 0, n_db)).to(device)
    q = torch.from_numpy(search_vectors(0, "dbq", 0, n_q).reshape(1, n_q, d)).to(device)
    calls, work = {}, {}
    for b in (2, 4):
        qz = tq.Quantizer(d, b, tq.MODE_MSE, seed=0, device=device)
        cache = qz.quantize(db)          # the index is built once, outside the step
        calls["search_b%d" % b] = lambda qz=qz, cache=cache: qz.search(q, cache, 1, n_db, k)
        byts = n_db * (b * d // 8 + 2) + n_q * d * 4 + n_q * k * 8
        work["search_b%d" % b] = (byts, 2 * d * n_db * n_q, "search_score_kernel",
                                  ["search.hip", "tq_device.h"])
    del db
    cfg = {"workload": "vector search: 10^4 queries x 10^6 unit vectors (d = 200 padded to 256), "
                       "MSE b = 2 and 4, fused top-10 (two calls per step)",
           "n_db": n_db, "n_queries": n_q, "head_dim": d, "bits": [2, 4], "topk": k,
           "units_per_step": 2 * n_q * n_db}
    return calls, work, cfg, 2 * n_q * n_db, {}


def _oracle_threads():
    try:
        from threadpoolctl import threadpool_info
        return max((i.get("num_threads") or 0) for i in threadpool_info()) or os.cpu_count()
    except Exception:
        return os.cpu_count()


def cpu_baseline_prefill(budget_s=12.0):
    """The oracle quantising whole KV heads of the prefill workload (b = 3) until the budget is spent."""
    import numpy as np
    from oracle import codebook as ocb
    from oracle import quantizer as oqz
    from oracle import rotation as orot
    from synthetic import bf16_to_f32, channel_scales, kv_block
    d, tokens, b = 128, 65536, 3
    pi, s = orot.haar_rotation(d, 0), orot.qjl_matrix(d, 0)
    ck, tk, _ = ocb.codebook(d, b - 1)
    cv, tv, _ = ocb.codebook(d, b)
    ksc, vsc = channel_scales(0, 4, "k", 8, d), channel_scales(0, 4, "v", 8, d)
    done, heads, t_used = 0, 0, 0.0
    while heads < 8 and (t_used < budget_s or heads == 0):
        kx = bf16_to_f32(kv_block(0, 4, "k", 0, heads, tokens, ksc)).astype(np.float64)
        vx = bf16_to_f32(kv_block(0, 4, "v", 0, heads, tokens, vsc)).astype(np.float64)
        t0 = time.perf_counter()
        oqz.quantize(kx, pi, ck, tk, oqz.MODE_PROD, s_mat=s)
        oqz.quantize(vx, pi, cv, tv, oqz.MODE_MSE)
        t_used += time.perf_counter() - t0
        done += 2 * tokens
        heads += 1
    return {"value": done / t_used, "unit": "vectors/s", "cores": _oracle_threads(), "kind": "oracle",
            "sample": "%d of 8 KV heads (%d tokens each), keys prod b=3 and values MSE b=3; %.1f s of "
                      "CPU time" % (heads, tokens, t_used)}


def cpu_baseline_search(budget_s=12.0):
    """The oracle scoring queries against 65536 database vectors (MSE b=2) with top-10."""
    import numpy as np
    from oracle import codebook as ocb
    from oracle import quantizer as oqz
    from oracle import rotation as orot
    from synthetic import search_vectors
    d, n_db, k = 256, 65536, 10
    pi = orot.haar_rotation(d, 0)
    c, t, _ = ocb.codebook(d, 2)
    ref = oqz.quantize(search_vectors(0, "db", 0, n_db).astype(np.float64), pi, c, t, oqz.MODE_MSE)
    qs = search_vectors(0, "dbq", 0, 256).astype(np.float64)
    done, t_used, i = 0, 0.0, 0
    while i < len(qs) and (t_used < budget_s or i == 0):
        t0 = time.perf_counter()
        sc = oqz.logits_rotated(qs[i:i + 8], ref["codes"], ref["norm"], pi, c, oqz.MODE_MSE, 1.0)
        oqz.topk(sc, k)
        t_used += time.perf_counter() - t0
        done += 8 * n_db
        i += 8
    return {"value": done / t_used, "unit": "keys/s", "cores": _oracle_threads(), "kind": "oracle",
            "sample": "%d queries x the first %d database vectors (MSE b=2): oracle scores and top-10; "
                      "%.1f s of CPU time" % (i, n_db, t_used)}


def cpu_baseline_decode(budget_s=12.0):
    """The fp64 oracle on whole KV heads of the same decode workload until the budget is spent."""
    import numpy as np
    from oracle import codebook as ocb
    from oracle import quantizer as oqz
    from oracle import rotation as orot
    from synthetic import bf16_to_f32, channel_scales, gqa_queries, kv_block
    d, seq, bits = 128, 32768, 3
    ksc = channel_scales(0, 2, "k", 8, d)
    vsc = channel_scales(0, 2, "v", 8, d)
    q = bf16_to_f32(gqa_queries(0, 2, 1, 32, 8, ksc)).astype(np.float64)[0]
    pi, s = orot.haar_rotation(d, 0), orot.qjl_matrix(d, 0)
    ck, tk, _ = ocb.codebook(d, bits - 1)
    cvv, tv, _ = ocb.codebook(d, bits)
    done, heads, t_used = 0, 0, 0.0
    while heads < 8 and (t_used < budget_s or heads == 0):
        kx = bf16_to_f32(kv_block(0, 2, "k", 0, heads, seq, ksc)).astype(np.float64)
        vx = bf16_to_f32(kv_block(0, 2, "v", 0, heads, seq, vsc)).astype(np.float64)
        t0 = time.perf_counter()
        rk = oqz.quantize(kx, pi, ck, tk, oqz.MODE_PROD, s_mat=s)
        rv = oqz.quantize(vx, pi, cvv, tv, oqz.MODE_MSE)
        oqz.logits_rotated(q[4 * heads:4 * heads + 4], rk["codes"], rk["norm"], pi, ck, oqz.MODE_PROD,
                           1 / math.sqrt(d), rnorm=rk["rnorm"], s_mat=s)
        oqz.dequantize(rv["codes"], rv["norm"], pi, cvv, oqz.MODE_MSE)
        t_used += time.perf_counter() - t0
        done += seq
        heads += 1
    return {"value": done / t_used, "unit": "keys/s", "cores": _oracle_threads(),
            "kind": "oracle",
            "sample": "%d of 8 KV heads (%d tokens each): oracle quantise K (prod b=3) and V (MSE b=3), "
                      "logits of the 4 GQA query heads, dequantise V; %.1f s of CPU time" %
                      (heads, seq, t_used)}


def long_context_leg(torch, tq, timer, reps, device):
    d, batch, heads, qheads, seq, bits = 128, 8, 8, 32, 131072, 4
    from synthetic import device_kv, device_queries
    x = device_kv(torch, 0, 3, "k", batch, heads, seq, d, device)
    qz = tq.Quantizer(d, bits, tq.MODE_PROD, seed=0, device=device)
    cache = qz.quantize(x)
    del x
    q = device_queries(torch, 0, 3, batch, qheads, heads, d, device)
    out = torch.empty((batch, qheads, seq), dtype=torch.float32, device=device)
    call = lambda: qz.attn_logits(q, cache, heads, seq, 1.0 / math.sqrt(d), out=out)
    call()
    t = timer(call, reps)
    keys = batch * heads * seq
    byts = keys * (bits * d // 8 + 4) + keys * (qheads // heads) * 4 + batch * qheads * d * 2
    del cache, out
    torch.cuda.empty_cache()
    return {"workload": "batch 8, 8 KV heads x 128, 131072 tokens, keys inner-product b=4, "
                        "32 query heads", "us_per_call": t * 1e6, "keys_per_s": keys / t,
            "hbm_gbs": byts / t / 1e9, "frac_of_peak": byts / t / 1e9 / HBM_PEAK_GBS,
            "algorithmic_bytes": byts}


def main():
    args = _args()
    if args.gpus != 1:
        print("bench.py measures one GPU only (the library has no multi-GPU path); "
              "run it with --gpus 1", file=sys.stderr)
        sys.exit(2)
    import torch
    import online_vector_quantization_amd as tq
    assert torch.cuda.is_available(), "bench.py needs a GPU"
    device = torch.device("cuda:0")
    timer = Timer(torch)
    if args.copy_calibration:
        a = torch.empty(512 << 20, dtype=torch.uint8, device=device)
        b = torch.empty_like(a)
        b.copy_(a)
        torch.cuda.synchronize()
        del a, b

    build = {"decode": decode_workload, "prefill": prefill_workload, "search": search_workload}
    calls, work, cfg, units, extras = build[args.workload](torch, tq, args, device)
    unit = {"decode": "keys/s", "prefill": "vectors/s", "search": "keys/s"}[args.workload]
    step = lambda: [fn() for fn in calls.values()]
    if args.warmup is None:                 # about one second of steps, at least 5
        for _ in range(3):                  # first calls: workspaces, first touches
            step()
        torch.cuda.synchronize()
        tw = time.perf_counter()
        for _ in range(10):
            step()
        torch.cuda.synchronize()
        per = max((time.perf_counter() - tw) / 10, 1e-6)
        args.warmup = 13 + max(5, int(math.ceil(WARMUP_S / per)))
        for _ in range(args.warmup - 13):
            step()
    else:
        for _ in range(args.warmup):
            step()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    t_step = timer(step, args.steps)
    wall = time.perf_counter() - t0

    breakdown = {}
    for name, fn in calls.items():
        t = timer(fn, args.steps)
        byts, flops, kern, src = work[name]
        breakdown[name] = {"us": t * 1e6, "hbm_gbs": byts / t / 1e9,
                           "frac_hbm": byts / t / 1e9 / HBM_PEAK_GBS,
                           "tflops": (flops / t / 1e12) if flops else None,
                           "vectors_per_s": units / t}
    dom = max(breakdown, key=lambda k: breakdown[k]["us"])
    byts, flops, kern, src = work[dom]
    tdom = breakdown[dom]["us"] * 1e-6
    traffic = _traffic(kern + ":" + dom, src)
    if args.workload == "decode":
        roofline = {"kernel": kern, "call": dom, "bound": "hbm", "achieved": byts / tdom / 1e9,
                    "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": byts / tdom / 1e9 / HBM_PEAK_GBS,
                    "traffic": traffic, "algorithmic_bytes_per_launch": byts}
    else:   # fp16 MFMA contraction: algorithmic flops of the call against the dense fp16 peak
        roofline = {"kernel": kern, "call": dom, "bound": "mfma", "achieved": flops / tdom / 1e12,
                    "peak": MFMA_F16_PEAK_TFS, "unit": "TFLOP/s", "frac": flops / tdom / 1e12 / MFMA_F16_PEAK_TFS,
                    "traffic": traffic, "algorithmic_flops_per_launch": flops,
                    "algorithmic_bytes_per_launch": byts}

    line = {"metric": METRIC, "value": units / t_step, "unit": unit, "n_gpus": 1,
            "steps": args.steps, "warmup": args.warmup, "ms_per_step": t_step * 1e3,
            "wall_s_timed": wall, "higher_is_better": True, "scaling": "weak",
            "vs_baseline": None, "dtype": "bf16 in; f16 split + i8 MFMA, f32/i32 accumulate",
            "data": "synthetic", "config": cfg, "roofline": roofline, "breakdown": breakdown}
    if extras:
        line["extras"] = {}
        for name, (fn, byts, kern, src) in extras.items():
            for _ in range(max(args.warmup, 1)):     # first calls size the library's workspace
                fn()
            t = timer(fn, args.steps)
            line["extras"][name] = {"us": t * 1e6, "hbm_gbs": byts / t / 1e9,
                                    "frac_hbm": byts / t / 1e9 / HBM_PEAK_GBS, "kernel": kern,
                                    "algorithmic_bytes_per_launch": byts,
                                    "traffic": _traffic(kern + ":" + name, src),
                                    "in_step": False}
    if args.workload == "decode" and not args.no_long_context:
        line["long_context_logits"] = long_context_leg(torch, tq, timer, args.steps, device)
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = {"decode": cpu_baseline_decode, "prefill": cpu_baseline_prefill,
                                "search": cpu_baseline_search}[args.workload]()
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
