#!/usr/bin/env python3
"""Benchmark of the paged DSA decode step on one MI355X.

Step (one pass of the hot path over one synthetic batch): the decode batch of
8 streams x 131,072 tokens, 1 layer, pages shuffled in the pool, 32 attention
heads, 16 indexer heads x 128, top-512 blocks:
  tf_latent_write (each stream's new row + its pooled key) -> tf_indexer_logits
  -> tf_topk_blocks -> tf_sparse_mla_attn.
The page address is computed inside each kernel; the plan is host-side and
computed once. Inputs are resident in HBM before timing. Consecutive steps
rotate over independent copies of the pool so that no step finds the previous
step's rows in the 256 MB Infinity Cache.

Reported: value = selected latent bytes per step / wall time per step (GB/s),
the dominant kernel against the HBM roofline (durations from HIP events on the
launch stream), the prefill-chunk indexer (T = 2,048 rows against 25,000 pooled
keys) against the bf16 MFMA roofline, and the oracle timed on the host cores.

    python bench.py [--gpus 1] [--steps 50] [--warmup 10]
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
MFMA_BF16_PEAK_TFLOPS = 2500.0
ROW_BYTES = 512 * 2 + 64 * 2


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def kernel_hash(path):
    return hashlib.sha256(open(path, "rb").read()).hexdigest()[:16]


def load_traffic(kernel_name, src_file, launches_note=None):
    """HBM bytes per launch from committed rocprofv3 --pmc summaries, or None when
    the kernel source changed since the counters were taken."""
    p = os.path.join(ROOT, "profiles", f"traffic_{kernel_name}.json")
    if not os.path.exists(p):
        return None
    d = json.load(open(p))
    if d.get("source_sha256_16") != kernel_hash(src_file):
        return None
    return d.get("hbm_bytes_per_launch")


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--replicas", type=int, default=6, help="pool copies rotated between steps")
    ap.add_argument("--no-prefill", action="store_true")
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--cpu-reps", type=int, default=3)
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU: this build has no multi-GPU path (asked for --gpus {args.gpus}).",
              file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import attention_page_table_amd as tf
    from synth.configs import decode_batch, prefill_chunk
    from synth.device import alloc_pool, populate, query_inputs, write_rows  # noqa: F401
    from synth.device import fill_bf16, _rid
    from synth import TAG_LATENT, TAG_PKEY
    from synth.configs import LAT, ROPE, ROW

    assert torch.cuda.is_available(), "bench.py needs the GPU"
    tf.lib()  # fails loudly when the HIP library is missing

    # ------------------------------------------------------------------ decode setup
    wl = decode_batch(0)
    plan = tf.kv_pool_plan(tf.geom(1, wl.Dk))
    log(f"setup: {wl.name}: pool {wl.n_pages} pages x {plan.page_bytes} B, {args.replicas} copies")
    P0 = alloc_pool(wl, plan)
    populate(P0)
    pools = [P0.pool]
    for _ in range(args.replicas - 1):
        pools.append(P0.pool.clone())
    pt = P0.pt
    views = [tf.view(p, pt, wl.pt_stride, wl.n_pages) for p in pools]
    rows = wl.rows
    R = len(rows)
    rs, rp, iq, w, q = query_inputs(wl, 0, rows)
    # the step's own writes: row L-1 of each stream and the pooled key of its block
    lat_new = torch.empty((R, LAT), dtype=torch.bfloat16, device="cuda")
    rope_new = torch.empty((R, ROPE), dtype=torch.bfloat16, device="cuda")
    key_new = torch.empty((R, wl.Dk), dtype=torch.bfloat16, device="cuda")
    for i, (b, t) in enumerate(rows):
        r0 = _rid(0, b, t)
        fill_bf16(lat_new[i:], 1, LAT, wl.seed, TAG_LATENT, r0 * ROW, ROW, ROW)
        fill_bf16(rope_new[i:], 1, ROPE, wl.seed, TAG_LATENT, r0 * ROW + LAT, ROW, ROW)
        fill_bf16(key_new[i:], 1, wl.Dk, wl.seed, TAG_PKEY, _rid(0, b, t // 4) * wl.Dk, wl.Dk, wl.Dk)
    kidx = torch.tensor([t // 4 for _, t in rows], dtype=torch.int32, device="cuda")
    ld = max(t // 4 + 1 for _, t in rows)
    logits = torch.empty((R, ld), dtype=torch.float32, device="cuda")
    nv = torch.empty(R, dtype=torch.int32, device="cuda")
    blocks = torch.empty((R, wl.k), dtype=torch.int32, device="cuda")
    out = torch.empty((R, wl.Hq, 512), dtype=torch.float32, device="cuda")
    lse = torch.empty((R, wl.Hq), dtype=torch.float32, device="cuda")
    ws_topk = torch.empty(max(1, tf.topk_workspace_bytes(R, ld, wl.k)), dtype=torch.uint8, device="cuda")
    ws_attn = torch.empty(max(1, tf.attn_workspace_bytes(R, wl.Hq, wl.k)), dtype=torch.uint8, device="cuda")
    scale = 1.0 / math.sqrt(576.0)
    torch.cuda.synchronize()

    names = ["write", "indexer", "topk", "attention"]

    def step(i, ev=None):
        v = views[i % len(views)]
        if ev is not None:
            ev[0].record()
        tf.latent_write(plan, v, rs, rp, lat_new, rope_new, pkey_stream=rs, pkey_idx=kidx, pkeys=key_new)
        if ev is not None:
            ev[1].record()
        tf.indexer_logits(plan, v, rs, rp, iq, w, logits, n_valid=nv)
        if ev is not None:
            ev[2].record()
        tf.topk_blocks(logits, nv, wl.k, blocks, ws=ws_topk)
        if ev is not None:
            ev[3].record()
        tf.sparse_mla_attn(plan, v, rs, rp, q, scale, blocks, out, lse, ws=ws_attn)
        if ev is not None:
            ev[4].record()

    def run(i, timing=False):
        step(i, evs[i] if timing else None)

    # warmup
    evs = None
    for i in range(args.warmup):
        run(i)
    torch.cuda.synchronize()

    # timed region: exactly K steps
    K = args.steps
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(5)] for _ in range(K)]
    t_start = torch.cuda.Event(enable_timing=True)
    t_end = torch.cuda.Event(enable_timing=True)
    per_kernel = {n: [] for n in names}
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    t_start.record()
    for i in range(K):
        run(i, timing=True)
    t_end.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_total = t_start.elapsed_time(t_end)
    ms_per_step = ms_total / K
    for i in range(K):
        for j, n in enumerate(names):
            per_kernel[n].append(evs[i][j].elapsed_time(evs[i][j + 1]))
    avg_ms = {n: float(np.mean(v)) for n, v in per_kernel.items()}

    lat_bytes = R * wl.k * 4 * ROW_BYTES                       # selected latent + rope rows
    value = lat_bytes / (ms_per_step * 1e-3) / 1e9
    alg_bytes = {
        "write": R * (ROW_BYTES + wl.Dk * 2) * 2,
        "indexer": R * ld * (wl.Dk * 2 + 4) + R * wl.H * (wl.Dk * 2 + 4),
        "topk": R * ld * 4 + R * wl.k * 4,
        "attention": lat_bytes + R * wl.Hq * 576 * 2 + R * wl.Hq * 512 * 4 + R * wl.k * 4,
    }
    kern = {n: {"us": avg_ms[n] * 1e3, "alg_bytes": alg_bytes[n],
                "GBps": alg_bytes[n] / (avg_ms[n] * 1e-3) / 1e9 if avg_ms[n] > 0 else None}
            for n in names}
    dom = max(["indexer", "topk", "attention"], key=lambda n: avg_ms[n])
    src = {"indexer": "indexer.hip", "topk": "topk.hip", "attention": "attention.hip"}[dom]
    traffic = load_traffic(dom, os.path.join(ROOT, "attention_page_table_amd", "csrc", src))
    achieved = kern[dom]["GBps"]
    roofline = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": traffic, "kernel": dom,
                "alg_bytes_per_launch": alg_bytes[dom], "avg_launch_us": round(avg_ms[dom] * 1e3, 2)}

    # ------------------------------------------------------------------ prefill indexer
    prefill = None
    if not args.no_prefill:
        pw = prefill_chunk(0)
        pplan = tf.kv_pool_plan(tf.geom(1, pw.Dk))
        log(f"setup: {pw.name}")
        PP = alloc_pool(pw, pplan)
        populate(PP)
        prs, prp, piq, pww, _ = query_inputs(pw, 0, pw.rows)
        pld = 25000
        plog = torch.empty((len(pw.rows), pld), dtype=torch.float32, device="cuda")
        pnv = torch.empty(len(pw.rows), dtype=torch.int32, device="cuda")
        pv = PP.view()
        for _ in range(3):
            tf.indexer_logits(pplan, pv, prs, prp, piq, pww, plog, n_valid=pnv)
        torch.cuda.synchronize()
        reps = 20
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(reps):
            tf.indexer_logits(pplan, pv, prs, prp, piq, pww, plog, n_valid=pnv)
        e1.record()
        torch.cuda.synchronize()
        us = e0.elapsed_time(e1) / reps * 1e3
        flops = sum(2 * pw.H * pw.Dk * (t // 4 + 1) for _, t in pw.rows)
        tfl = flops / (us * 1e-6) / 1e12
        prefill = {"kernel": "indexer", "workload": pw.name, "us": round(us, 2), "causal_flop": flops,
                   "roofline": {"bound": "mfma", "achieved": round(tfl, 1), "peak": MFMA_BF16_PEAK_TFLOPS,
                                "unit": "TFLOP/s", "frac": round(tfl / MFMA_BF16_PEAK_TFLOPS, 4),
                                "traffic": load_traffic("indexer_prefill", os.path.join(
                                    ROOT, "attention_page_table_amd", "csrc", "indexer.hip"))}}
        del PP, plog

    # ------------------------------------------------------------------ oracle on the host
    cpu = None
    if not args.no_cpu:
        cpu = cpu_baseline(wl, rows, ld, scale, args.cpu_reps, lat_bytes)

    line = {
        "metric": "paged DSA decode: latent GB/s (% HBM peak); prefill chunk indexer % MFMA peak",
        "value": round(value, 1), "unit": "GB/s", "n_gpus": 1, "steps": K, "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": wl.name, "streams": R, "context": wl.lengths[0], "caches": 1,
                   "attn_heads": wl.Hq, "indexer_heads": wl.H, "index_dim": wl.Dk, "topk_blocks": wl.k,
                   "page_rows": 512, "pool_pages": wl.n_pages, "pool_copies": len(views),
                   "launches": "eager, one HIP event between kernels"},
        "roofline": roofline,
        "kernels": {n: {k2: (round(v2, 3) if isinstance(v2, float) else v2) for k2, v2 in d.items()}
                    for n, d in kern.items()},
        "attention_latent_GBps": round(lat_bytes / (avg_ms["attention"] * 1e-3) / 1e9, 1),
        "prefill_indexer": prefill,
        "cpu_baseline": cpu,
        "wall_s_timed": round(wall, 4),
    }
    print(json.dumps(line), flush=True)


def cpu_baseline(wl, rows, ld, scale, reps, lat_bytes):
    """The oracle (fp64 numpy) on the same decode step: logits over every pooled
    key, exact top-k, attention over the selected rows. Inputs are generated before
    timing; only the oracle's arithmetic is timed."""
    import numpy as np
    from oracle import indexer_logits, sparse_mla, topk_blocks
    from oracle import workload as ow
    from synth import bf16_to_f64
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:
        threads = os.cpu_count()
    log("cpu baseline: generating inputs")
    q_i = bf16_to_f64(wl.iq_bits(0, rows))
    w_i = wl.weights(0, rows).astype(np.float64)
    keys = [ow.keys_of(wl, 0, b, t // 4 + 1) for b, t in rows]
    q_a = bf16_to_f64(wl.q_bits(0, rows))
    pos = [t for _, t in rows]
    t_idx = []
    t_att = []
    for _ in range(reps):
        t0 = time.perf_counter()
        lg = indexer_logits(q_i, w_i, keys, pos, ld)
        blk = topk_blocks(lg, [min(t // 4 + 1, ld) for t in pos], wl.k)
        t_idx.append(time.perf_counter() - t0)
        # gather the selected rows (generator work, untimed), then time the attention
        from oracle.attention import selected_tokens
        cache = {}
        for r, (b, t) in enumerate(rows):
            S = selected_tokens(blk[r], t)
            cache[r] = dict(zip(S.tolist(), range(S.size))), ow.rows_reader(wl, 0, b)(S)
        def rows_of(r, S):
            m, (lat, rope) = cache[r]
            ix = [m[s] for s in S.tolist()]
            return lat[ix], rope[ix]
        t0 = time.perf_counter()
        sparse_mla(q_a, rows_of, blk, pos, scale)
        t_att.append(time.perf_counter() - t0)
    sec = float(np.median(t_idx) + np.median(t_att))
    return {"value": round(lat_bytes / sec / 1e9, 4), "unit": "GB/s", "cores": threads, "kind": "oracle",
            "sample": f"the whole decode step ({len(rows)} rows: logits over {ld} keys each, top-{wl.k}, "
                      f"attention), median of {reps}", "seconds_per_step": round(sec, 4),
            "cpu_model": _cpu_model()}


def _cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except Exception:
        pass
    return None


if __name__ == "__main__":
    main()
