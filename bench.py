"""Benchmark of the online KV-cache quantizer hot path on one MI355X.

python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload decode|prefill|search]

Before the W warmup steps the bench runs steps untimed for --settle seconds
(default 1): the GPU reaches its sustained clock only under sustained load
(a 5-step warmup alone timed the decode step 15-20% slower than the sustained
rate).  The line reports the settle time and steps next to W.

Cold and warm: the decode step's inputs and outputs (about 232 MB) fit the
256 MB MALL, so the timed steps rotate over three buffer sets (each step's
buffers were last touched two steps earlier, with about 460 MB of other
traffic in between): ``value`` is that cold rate.  The same steps on one set
(warm, cache-resident) are reported beside it.  Per-call times are
per-launch HIP events (median, min and mean).

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


def _args():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=None, help="untimed warmup steps after the settle phase (5)")
    ap.add_argument("--settle", type=float, default=1.0,
                    help="seconds of untimed steps before the warmup steps (clock ramp)")
    ap.add_argument("--workload", default="decode", choices=["decode", "prefill", "search"])
    ap.add_argument("--no-peaks", action="store_true", help="skip the measured-ceiling leg")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-long-context", action="store_true")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="run one 512 MiB device copy first (reference kernel for HBM counters)")
    ap.add_argument("--write-traffic", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"),
                    help="write profiles/hbm_traffic.json from two rocprofv3 --pmc output folders and exit")
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


# The kernel instance (as rocprofv3 names it, template arguments included)
# and the sources behind each traffic entry that bench.py reports.  Calls
# that run the same instance on the same shape share its counters.
_Q, _L, _D, _A = (["quantize.hip", "tq_device.h"], ["logits.hip", "tq_device.h"], ["dequant.hip", "tq_device.h"],
                  ["attend.hip", "tq_device.h"])
TRAFFIC_INSTANCES = {
    "quantize_pc_kernel:quantize_k": ("quantize_pc_kernel<128, 2, false>", _Q),
    "quantize_kernel:quantize_v": ("quantize_kernel<128, 3, false, false>", _Q),
    "logit_kernel:attn_logits": ("logit_kernel<128, 2, true, 1, false>", _L),
    "logit_kernel:append_attn_logits": ("logit_kernel<128, 2, true, 1, false>", _L),
    "logit_kernel:attn_logits_paged": ("logit_kernel<128, 2, true, 1, true>", _L),
    "logit_kernel:append_attn_logits_paged": ("logit_kernel<128, 2, true, 1, true>", _L),
    "dequant_kernel:dequantize_v": ("dequant_kernel<128, 3, false, false, false>", _D),
    "logit_kernel:long_context": ("logit_kernel<128, 3, true, 1, false>", _L),
    "attend_mfma_kernel:attn_output": ("attend_mfma_kernel<128, 3, 4>", _A),
    "attend_combine_kernel:attn_output": ("attend_combine_kernel<128>", _A),
    "quantize_polar_kernel:polar_quantize": ("quantize_polar_kernel<128, false>", _Q),
    "dequant_kernel:polar_dequantize": ("dequant_kernel<128, 1, false, false, true>", _D),
    "polar_logit_kernel:polar_attn_logits": ("polar_logit_kernel<128, 4>", ["polar_logits.hip", "tq_device.h"]),
}


def write_traffic(fetch_dir, write_dir, out_path=None):
    """profiles/hbm_traffic.json from two rocprofv3 --pmc runs (CSV output) of
    `bench.py --copy-calibration`: FETCH_SIZE in fetch_dir, WRITE_SIZE in
    write_dir.  The first copy kernel of each run is the 512 MiB calibration
    copy; each counter is scaled by 512 MiB over its reading there.  Prints
    the table of the summary."""
    import csv
    import glob

    def load(d, counter):
        rows = {}
        for path in sorted(glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True)):
            with open(path) as f:
                for r in csv.DictReader(f):
                    if r["Counter_Name"] != counter:
                        continue
                    key = (path, int(r["Dispatch_Id"]))
                    name, v = rows.get(key, (r["Kernel_Name"], 0.0))
                    rows[key] = (name, v + float(r["Counter_Value"]))
        if not rows:
            raise SystemExit("no %s rows under %s" % (counter, d))
        return rows

    fetch, write = load(fetch_dir, "FETCH_SIZE"), load(write_dir, "WRITE_SIZE")

    def scale(rows, counter):
        copies = sorted((k, v) for k, (n, v) in rows.items() if "copy" in n.lower())
        if not copies:
            raise SystemExit("no calibration copy among the %s dispatches" % counter)
        return 524288.0 / copies[0][1], copies[0][1]

    fs, f_cal = scale(fetch, "FETCH_SIZE")
    ws, w_cal = scale(write, "WRITE_SIZE")
    table = {"_note": "HBM bytes per dispatch from two rocprofv3 --pmc runs (FETCH_SIZE, then WRITE_SIZE) of "
                      "'python bench.py --steps 3 --warmup 1 --no-cpu-baseline --no-peaks --copy-calibration'; "
                      "each counter is scaled by 512 MiB / its reading for the 512 MiB calibration copy in the "
                      "same run (fetch x%.4f, write x%.4f). source_sha is the hash of the kernel sources the "
                      "counters were taken on." % (fs, ws)}
    print("calibration copy: FETCH_SIZE %.1f KiB, WRITE_SIZE %.1f KiB (x%.4f, x%.4f)" % (f_cal, w_cal, fs, ws))
    print("| kernel (call) | instance | dispatches | FETCH KiB raw | WRITE KiB raw | HBM MB scaled |")
    print("|---|---|---|---|---|---|")
    for key, (inst, src) in TRAFFIC_INSTANCES.items():
        fv = [v for n, v in fetch.values() if inst in n]
        wv = [v for n, v in write.values() if inst in n]
        if not fv or not wv:
            continue
        ent = {"fetch_kib": sum(fv) / len(fv), "fetch_scale": fs, "write_kib": sum(wv) / len(wv),
               "write_scale": ws, "source_sha": _source_hash(src), "dispatches": min(len(fv), len(wv))}
        table[key] = ent
        mb = (ent["fetch_kib"] * fs + ent["write_kib"] * ws) * 1024 / 1e6
        print("| %s | %s | %d | %.1f | %.1f | %.2f |" % (key, inst, ent["dispatches"], ent["fetch_kib"],
                                                       ent["write_kib"], mb))
    with open(out_path or os.path.join(PROFILES, "hbm_traffic.json"), "w") as f:
        json.dump(table, f, indent=1)
        f.write("\n")


class Timer:
    """HIP events on the current stream (the stream every call is queued on)."""

    def __init__(self, torch):
        self.torch = torch

    def __call__(self, fn, n):
        """Mean duration of n back-to-back launches of fn (seconds)."""
        t = self.torch
        start = t.cuda.Event(enable_timing=True)
        end = t.cuda.Event(enable_timing=True)
        t.cuda.synchronize()
        start.record()
        for i in range(n):
            fn(i)
        end.record()
        t.cuda.synchronize()
        return start.elapsed_time(end) * 1e-3 / n

    def each(self, fn, n, filler=None):
        """Per-launch durations of n launches of fn (seconds), events around
        each.  With a filler (work queued before each launch, outside its
        events) the GPU stays busy while the host queues the next launch, so
        no event interval of a short call contains host time."""
        t = self.torch
        ev = [(t.cuda.Event(enable_timing=True), t.cuda.Event(enable_timing=True)) for _ in range(n)]
        t.cuda.synchronize()
        for i, (a, b) in enumerate(ev):
            if filler is not None:
                filler(i)
            a.record()
            fn(i)
            b.record()
        t.cuda.synchronize()
        return [a.elapsed_time(b) * 1e-3 for a, b in ev]

    def in_steps(self, calls, n, skip=2):
        """Per-call durations (seconds) from events around every call of n
        steps run back to back, as in the timed region; the first `skip`
        steps (while the host fills the queue) are dropped."""
        t = self.torch
        ev = {k: [] for k in calls}
        t.cuda.synchronize()
        for i in range(n + skip):
            for k, fn in calls.items():
                a, b = t.cuda.Event(enable_timing=True), t.cuda.Event(enable_timing=True)
                a.record()
                fn(i)
                b.record()
                ev[k].append((a, b))
        t.cuda.synchronize()
        return {k: [a.elapsed_time(b) * 1e-3 for a, b in v[skip:]] for k, v in ev.items()}


def _stats(ts):
    ts = sorted(ts)
    return {"median_us": ts[len(ts) // 2] * 1e6, "min_us": ts[0] * 1e6, "mean_us": sum(ts) / len(ts) * 1e6}


def _host_kv(torch, seed, cfg, tensor, heads, tokens, d, device):
    """bf16 [heads*tokens, d] from the shared numpy recipe (reproducible on the host)."""
    import numpy as np
    from synthetic import channel_scales, kv_block
    sc = channel_scales(seed, cfg, tensor, heads, d)
    blocks = [kv_block(seed, cfg, tensor, 0, h, tokens, sc) for h in range(heads)]
    arr = np.concatenate(blocks, axis=0)
    return torch.from_numpy(arr.view(np.int16)).to(device).view(torch.bfloat16), sc


N_SETS = 3   # rotating buffer sets of the decode step: 3 x 232 MB > the 256 MB MALL


def decode_workload(torch, tq, args, device):
    import numpy as np
    from synthetic import gqa_queries
    d, heads, qheads, seq, bits = 128, 8, 32, 32768, 3
    n = heads * seq
    k, ksc = _host_kv(torch, 0, 2, "k", heads, seq, d, device)
    v, _ = _host_kv(torch, 0, 2, "v", heads, seq, d, device)
    qb = gqa_queries(0, 2, 1, qheads, heads, ksc)
    q = torch.from_numpy(qb.view(np.int16)).to(device).view(torch.bfloat16)
    qk = tq.Quantizer(d, bits, tq.MODE_PROD, seed=0, device=device)
    qv = tq.Quantizer(d, bits, tq.MODE_MSE, seed=0, device=device)
    scale = 1.0 / math.sqrt(d)
    # N_SETS copies of every buffer the step touches; call i works on set i % N_SETS
    sets = []
    for j in range(N_SETS):
        sets.append({"k": k if j == 0 else k.clone(), "v": v if j == 0 else v.clone(), "q": q.clone(),
                     "ck": qk.new_cache(n), "cv": qv.new_cache(n),
                     "logits": torch.empty((1, qheads, seq), dtype=torch.float32, device=device),
                     "vhat": torch.empty((n, d), dtype=torch.bfloat16, device=device)})
    S = lambda i: sets[i % N_SETS]
    calls = {
        "quantize_k": lambda i: qk.quantize(S(i)["k"], out=S(i)["ck"]),
        "quantize_v": lambda i: qv.quantize(S(i)["v"], out=S(i)["cv"]),
        "attn_logits": lambda i: qk.attn_logits(S(i)["q"], S(i)["ck"], heads, seq, scale, out=S(i)["logits"]),
        "dequantize_v": lambda i: qv.dequantize(S(i)["cv"], n, out=S(i)["vhat"]),
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
           "key_bits": bits, "value_bits": bits, "units_per_step": n, "buffer_sets": N_SETS}
    # Timed beside the step, not in it (on set 0 after it ran): the attention
    # output softmax(l) . V straight from the packed values, on the step's logits.
    s0 = sets[0]
    attn = torch.empty((1, qheads, d), dtype=torch.float32, device=device)
    # The decode step with append: the new key of every head (here token
    # seq - 1 again, so the cache is unchanged) quantised into the cache by the
    # logit call, then logits over all seq tokens.
    x_new = k.view(heads, seq, d)[:, seq - 1].contiguous().view(1, heads, d)
    logits2 = torch.empty_like(s0["logits"])
    extras = {"attn_output": (lambda i: qv.attn_output(s0["logits"], s0["cv"], heads, seq, out=attn),
                              n * rb_v + qheads * seq * 4 + qheads * d * 4, "attend_mfma_kernel",
                              ["attend.hip", "tq_device.h"]),
              "append_attn_logits": (lambda i: qk.append_attn_logits(x_new, q, s0["ck"], heads, seq - 1, scale,
                                                                     row_tokens=seq, out=logits2),
                                     n * (rb_k + 4 * (qheads // heads)) + qheads * d * 2 + heads * (2 * d + rb_k),
                                     "logit_kernel", ["logits.hip", "tq_device.h"])}
    # The same key cache as a pool of 256-token pages in a random order (and
    # 16 spare pages): logits through the block table, and the step with
    # append into the pool.
    page = 256
    per_seq = seq // page
    n_pages = per_seq + 16
    table = torch.from_numpy(np.random.default_rng(7).permutation(n_pages)[:per_seq].astype(np.int32)
                             .reshape(1, per_seq)).to(device)
    pool = qk.new_cache(n_pages * heads * page)
    rows = ((table.long()[0][:, None, None] * heads + torch.arange(heads, device=device)[None, :, None]) * page
            + torch.arange(page, device=device)[None, None, :])            # [page j, head, token in page]
    rows = rows.permute(1, 0, 2).reshape(-1)                                # head-major, token order
    qk.quantize(k, out=s0["ck"])
    pool.codes[rows] = s0["ck"].codes
    pool.norm[rows] = s0["ck"].norm
    pool.rnorm[rows] = s0["ck"].rnorm
    logits3 = torch.empty_like(s0["logits"])
    extras["attn_logits_paged"] = (lambda i: qk.attn_logits_paged(q, pool, table, page, heads, seq, scale,
                                                                  out=logits3),
                                   n * (rb_k + 4 * (qheads // heads)) + qheads * d * 2 + per_seq * 4,
                                   "logit_kernel", ["logits.hip", "tq_device.h"])
    extras["append_attn_logits_paged"] = (lambda i: qk.append_attn_logits_paged(x_new, q, pool, table, page, heads,
                                                                                seq - 1, scale, out=logits3),
                                          n * (rb_k + 4 * (qheads // heads)) + qheads * d * 2 + per_seq * 4
                                          + heads * (2 * d + rb_k), "logit_kernel", ["logits.hip", "tq_device.h"])
    # The PolarQuant variant of stage 1 on the same values (3 bits per coordinate).
    qp = tq.Quantizer(d, 3, tq.MODE_POLAR, seed=0, device=device)
    cp = qp.new_cache(n)
    vhat_p = torch.empty((n, d), dtype=torch.bfloat16, device=device)
    rb_p = 3 * d // 8 + 2
    extras["polar_quantize"] = (lambda i: qp.quantize(v, out=cp), n * (2 * d + rb_p), "quantize_polar_kernel",
                                ["quantize.hip", "tq_device.h"])
    extras["polar_dequantize"] = (lambda i: qp.dequantize(cp, n, out=vhat_p), n * (rb_p + 2 * d), "dequant_kernel",
                                  ["dequant.hip", "tq_device.h"])
    # Logits straight from polar-format keys (the same keys, 3 bits per
    # coordinate): the angle-tree walk, one key per thread.
    cpk = qp.new_cache(n)
    qp.quantize(k, out=cpk)
    logits4 = torch.empty_like(s0["logits"])
    extras["polar_attn_logits"] = (lambda i: qp.attn_logits(q, cpk, heads, seq, scale, out=logits4),
                                   n * (rb_p + 4 * (qheads // heads)) + qheads * d * 2, "polar_logit_kernel",
                                   ["polar_logits.hip", "tq_device.h"])
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
        calls["quantize_k_b%d" % b] = lambda i, qk=qk, ck=ck: qk.quantize(k, out=ck)
        calls["quantize_v_b%d" % b] = lambda i, qv=qv, cv=cv: qv.quantize(v, out=cv)
        rb = b * d // 8
        work["quantize_k_b%d" % b] = (n * (2 * d + rb + 4), n * 4 * d * d, "quantize_pc_kernel", src)
        work["quantize_v_b%d" % b] = (n * (2 * d + rb + 2), n * 2 * d * d, "quantize_kernel", src)
    cfg = {"workload": "prefill quantisation: 65536 new bf16 tokens x 8 KV heads x 128; keys "
                       "inner-product and values MSE at b = 2, 3, 4 (six calls per step)",
           "tokens": tokens, "kv_heads": heads, "head_dim": d, "bits": [2, 3, 4],
           "units_per_step": 6 * n}
    return calls, work, cfg, 6 * n, {}


def _exact_top10(qv, db, k=10, block=131072):
    """Exact fp64 inner products of unquantised vectors and their top-k per
    query (ties to the smaller index): the ground truth recall is measured
    against."""
    import numpy as np
    q = qv.astype(np.float64)
    best_v = np.full((len(q), 0), -np.inf)
    best_i = np.zeros((len(q), 0), np.int64)
    for start in range(0, len(db), block):
        sc = q @ db[start:start + block].astype(np.float64).T
        part = np.argpartition(-sc, k - 1, axis=1)[:, :k]
        v = np.concatenate([best_v, np.take_along_axis(sc, part, 1)], 1)
        i = np.concatenate([best_i, start + part], 1)
        order = np.lexsort((i, -v), axis=-1)            # by score, ties to the smaller index
        best_v = np.take_along_axis(v, order[:, :k], 1)
        best_i = np.take_along_axis(i, order[:, :k], 1)
    return best_i


def search_workload(torch, tq, args, device):
    import numpy as np
    from synthetic import search_vectors
    d, n_db, n_q, k = 256, 1_000_000, 10_000, 10
    db_host = search_vectors(0, "db", 0, n_db)
    db = torch.from_numpy(db_host).to(device)
    qv_host = search_vectors(0, "dbq", 0, n_q)
    q = torch.from_numpy(qv_host.reshape(1, n_q, d)).to(device)
    calls, work, results = {}, {}, {}
    for b in (2, 4):
        qz = tq.Quantizer(d, b, tq.MODE_MSE, seed=0, device=device)
        cache = qz.quantize(db)          # the index is built once, outside the step
        results[b] = (qz, cache)
        calls["search_b%d" % b] = lambda i, qz=qz, cache=cache: qz.search(q, cache, 1, n_db, k)
        byts = n_db * (b * d // 8 + 2) + n_q * d * 4 + n_q * k * 8
        work["search_b%d" % b] = (byts, 2 * d * n_db * n_q, "search_score_kernel",
                                  ["search.hip", "tq_device.h"])
    del db
    # recall@10 of the GPU top-10 against the exact top-10 of the unquantised
    # 200-d vectors, on 1000 sampled queries
    rq = np.sort(np.random.default_rng(5).choice(n_q, 1000, replace=False))
    exact = _exact_top10(qv_host[rq, :200], db_host[:, :200])
    recall = {}
    for b, (qz, cache) in results.items():
        _, idx = qz.search(q, cache, 1, n_db, k)
        got = idx.cpu().numpy()[0][rq]
        recall["b%d" % b] = float(np.mean([len(set(g.tolist()) & set(e.tolist())) / k for g, e in zip(got, exact)]))
    cfg = {"workload": "vector search: 10^4 queries x 10^6 unit vectors (d = 200 padded to 256), "
                       "MSE b = 2 and 4, fused top-10 (two calls per step)",
           "n_db": n_db, "n_queries": n_q, "head_dim": d, "bits": [2, 4], "topk": k,
           "units_per_step": 2 * n_q * n_db,
           "recall_at_10": dict(recall, queries=len(rq), reference="exact fp64 inner products of the "
                                "unquantised 200-d vectors")}
    return calls, work, cfg, 2 * n_q * n_db, {}


def measured_peaks(torch, tq, timer, device):
    """Ceilings measured on this GPU with the library's probes (tq_probe):
    a plain read stream and a plain write stream over 4 GiB (16-byte
    non-temporal accesses, grid-strided), and register-only loops of
    32x32x16 fp16 and 16x16x64 int8 MFMAs.  Best of 10 launches each."""
    buf = torch.empty(4 << 30, dtype=torch.uint8, device=device)
    out = {}
    for name, kind in (("read_gbs", tq.PROBE_READ), ("write_gbs", tq.PROBE_WRITE)):
        work = tq.probe(kind, buf, device=device)
        t = min(timer.each(lambda i: tq.probe(kind, buf, device=device), 10))
        out[name] = work / t / 1e9
    del buf
    torch.cuda.empty_cache()
    for name, kind in (("mfma_f16_tflops", tq.PROBE_MFMA_F16), ("mfma_i8_tops", tq.PROBE_MFMA_I8)):
        work = tq.probe(kind, iters=2048, device=device)
        t = min(timer.each(lambda i: tq.probe(kind, iters=2048, device=device), 10))
        out[name] = work / t / 1e12
    out["how"] = "tq_probe: best of 10; 4 GiB read / write streams, 2048-step MFMA loops on every wave"
    return out


def _oracle_threads():
    try:
        from threadpoolctl import threadpool_info
        return max((i.get("num_threads") or 0) for i in threadpool_info()) or os.cpu_count()
    except Exception:
        return os.cpu_count()


def _host_info():
    """The host the oracle ran on: CPU model, logical CPUs, BLAS threads."""
    model = None
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    return {"cpu_model": model, "os_cpu_count": os.cpu_count(), "blas_threads": _oracle_threads()}


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


def _settle(torch, fn, seconds):
    """Untimed calls of fn for about `seconds` (the clocks reach their
    sustained level only under sustained load)."""
    torch.cuda.synchronize()
    t0, i = time.perf_counter(), 0
    while time.perf_counter() - t0 < seconds or i < 3:
        fn(i)
        i += 1
        if i % 8 == 0:
            torch.cuda.synchronize()
    torch.cuda.synchronize()


def long_context_leg(torch, tq, timer, reps, device, settle=1.0):
    d, batch, heads, qheads, seq, bits = 128, 8, 8, 32, 131072, 4
    from synthetic import device_kv, device_queries
    x = device_kv(torch, 0, 3, "k", batch, heads, seq, d, device)
    qz = tq.Quantizer(d, bits, tq.MODE_PROD, seed=0, device=device)
    cache = qz.quantize(x)
    del x
    q = device_queries(torch, 0, 3, batch, qheads, heads, d, device)
    out = torch.empty((batch, qheads, seq), dtype=torch.float32, device=device)
    call = lambda i: qz.attn_logits(q, cache, heads, seq, 1.0 / math.sqrt(d), out=out)
    _settle(torch, call, settle)
    st = _stats(timer.each(call, max(reps, 20)))
    t = timer(call, reps)
    keys = batch * heads * seq
    byts = keys * (bits * d // 8 + 4) + keys * (qheads // heads) * 4 + batch * qheads * d * 2
    # the streaming launch alone (queries prepared once): events around each launch
    prep = qz.prepare_queries(q, heads)
    scall = lambda i: qz.attn_logits_prepared(prep, cache, seq, 1.0 / math.sqrt(d), out=out)
    _settle(torch, scall, settle / 2)
    sst = _stats(timer.each(scall, max(reps, 20)))
    ts = timer(scall, reps)
    sbyts = keys * (bits * d // 8 + 4) + keys * (qheads // heads) * 4
    del cache, out, prep
    torch.cuda.empty_cache()
    return {"workload": "batch 8, 8 KV heads x 128, 131072 tokens, keys inner-product b=4, "
                        "32 query heads", "us_per_call": t * 1e6, "per_launch": st, "keys_per_s": keys / t,
            "hbm_gbs": byts / t / 1e9, "frac_of_peak": byts / t / 1e9 / HBM_PEAK_GBS,
            "algorithmic_bytes": byts, "traffic": _traffic("logit_kernel:long_context", _L),
            "streaming_kernel": {"kernel": "logit_kernel", "us_per_launch": ts * 1e6, "per_launch": sst,
                                 "keys_per_s": keys / ts, "hbm_gbs": sbyts / ts / 1e9,
                                 "frac_of_peak": sbyts / ts / 1e9 / HBM_PEAK_GBS, "algorithmic_bytes": sbyts,
                                 "how": "tq_attn_logits_prepared back to back on queries prepared once "
                                        "(tq_prepare_queries): the call's second launch alone"}}


def main():
    args = _args()
    if args.write_traffic:
        write_traffic(*args.write_traffic)
        return
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
    step = lambda i: [fn(i) for fn in calls.values()]
    # clock settle: untimed steps for about args.settle seconds
    torch.cuda.synchronize()
    ts, settle_steps = time.perf_counter(), 0
    while time.perf_counter() - ts < args.settle or settle_steps < 3:
        step(settle_steps)
        settle_steps += 1
        if settle_steps % 8 == 0:
            torch.cuda.synchronize()
    torch.cuda.synchronize()
    settle_s = time.perf_counter() - ts
    if args.warmup is None:
        args.warmup = 5
    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    # the timed region: exactly K steps (rotating buffer sets where the
    # workload has them), synchronised on both sides
    t0 = time.perf_counter()
    t_step = timer(step, args.steps)
    wall = time.perf_counter() - t0
    t_warm = timer(lambda i: step(0), args.steps) if args.workload == "decode" else None

    # per-call durations: events around every call of steps like the timed ones
    per_call = timer.in_steps(calls, args.steps)
    breakdown = {}
    for name, fn in calls.items():
        st = _stats(per_call[name])
        t = st["mean_us"] * 1e-6
        byts, flops, kern, src = work[name]
        breakdown[name] = dict(st, us=st["mean_us"], hbm_gbs=byts / t / 1e9, frac_hbm=byts / t / 1e9 / HBM_PEAK_GBS,
                               tflops=(flops / t / 1e12) if flops else None, vectors_per_s=units / t)
    dom = max(breakdown, key=lambda k: breakdown[k]["us"])
    byts, flops, kern, src = work[dom]
    tdom = breakdown[dom]["us"] * 1e-6
    traffic = _traffic(kern + ":" + dom, src)
    peaks = None if args.no_peaks else measured_peaks(torch, tq, timer, device)
    if args.workload == "decode":
        ach = byts / tdom / 1e9
        roofline = {"kernel": kern, "call": dom, "bound": "hbm", "achieved": ach,
                    "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": ach / HBM_PEAK_GBS,
                    "traffic": traffic, "algorithmic_bytes_per_launch": byts,
                    "launch_us": {k: breakdown[dom][k] for k in ("mean_us", "median_us", "min_us")}}
        if peaks:
            roofline["frac_of_measured_read_stream"] = ach / peaks["read_gbs"]
    else:   # fp16 MFMA contraction: algorithmic flops of the call against the dense fp16 peak
        ach = flops / tdom / 1e12
        # a search call scores in two launches (a sample pass, then the rest);
        # a prefill call is one launch
        per = "call" if args.workload == "search" else "launch"
        roofline = {"kernel": kern, "call": dom, "bound": "mfma", "achieved": ach,
                    "peak": MFMA_F16_PEAK_TFS, "unit": "TFLOP/s", "frac": ach / MFMA_F16_PEAK_TFS,
                    "traffic": traffic, "algorithmic_flops_per_" + per: flops,
                    "algorithmic_bytes_per_" + per: byts,
                    per + "_us": {k: breakdown[dom][k] for k in ("mean_us", "median_us", "min_us")}}
        if peaks:
            roofline["frac_of_measured_mfma_f16"] = ach / peaks["mfma_f16_tflops"]

    line = {"metric": METRIC, "value": units / t_step, "unit": unit, "n_gpus": 1,
            "steps": args.steps, "warmup": args.warmup, "settle_s": settle_s, "settle_steps": settle_steps,
            "ms_per_step": t_step * 1e3, "wall_s_timed": wall, "higher_is_better": True, "scaling": "weak",
            "vs_baseline": None, "dtype": "bf16 in; f16 split + i8 MFMA, f32/i32 accumulate",
            "data": "synthetic", "config": cfg, "roofline": roofline, "breakdown": breakdown}
    if t_warm is not None:
        line["warm"] = {"ms_per_step": t_warm * 1e3, "value": units / t_warm,
                        "note": "the same steps on one buffer set (inputs and outputs resident in the MALL)"}
        line["cold_note"] = "value: steps rotating over %d buffer sets, each last touched two steps earlier" % N_SETS
    if peaks:
        line["measured_peaks"] = peaks
    if extras:
        line["extras"] = {}
        for name, (fn, byts, kern, src) in extras.items():
            for i in range(max(args.warmup, 3)):
                fn(i)
            st = _stats(timer.each(fn, args.steps, filler=step))
            t = st["mean_us"] * 1e-6
            line["extras"][name] = dict(st, us=st["mean_us"], hbm_gbs=byts / t / 1e9,
                                        frac_hbm=byts / t / 1e9 / HBM_PEAK_GBS, kernel=kern,
                                        algorithmic_bytes_per_launch=byts,
                                        traffic=_traffic(kern + ":" + name, src), in_step=False)
    if args.workload == "decode" and not args.no_long_context:
        line["long_context_logits"] = long_context_leg(torch, tq, timer, args.steps, device, args.settle)
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = {"decode": cpu_baseline_decode, "prefill": cpu_baseline_prefill,
                                "search": cpu_baseline_search}[args.workload]()
        line["cpu_baseline"]["host"] = _host_info()
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
