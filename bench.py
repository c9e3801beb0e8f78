#!/usr/bin/env python3
"""Benchmark of the paged DSA decode step on one MI355X.

Step (one pass of the hot path over one synthetic batch): the decode batch of
8 streams x 131,072 tokens, 1 layer, pages shuffled in the pool, 32 attention
heads, 16 indexer heads x 128, top-512 blocks:
  tf_latent_write (each stream's new row + its pooled key) -> tf_indexer_logits
  -> tf_topk_blocks -> tf_sparse_mla_attn.
The page address is computed inside each kernel; the plan is host-side and
computed once. Inputs are resident in HBM before timing; the launches are
marshalled once before timing. Consecutive steps rotate over independent copies
of the pool so that no step finds the previous step's rows in the 256 MB
Infinity Cache.

Reported:
* value = paged-cache bytes one step reads (every visible pooled key, scanned by
  the indexer, plus the latent + rope rows of the selected blocks, gathered by
  the attention) / time per step, in GB/s;
* the dominant call against the HBM roofline (algorithmic bytes per launch /
  its average duration from HIP events on the launch stream), with the HBM
  traffic the rocprofv3 counters measured for it when they match the source;
* the prefill-chunk indexer (T = 2,048 rows against 25,000 pooled keys) against
  the bf16 MFMA roofline, and the whole prefill-chunk step call by call;
* the same chunk's indexer and top-k by key blocks (tf_indexer_topk), against the
  whole-buffer calls, and its two-level candidate selection (top-2,048 groups of 8
  keys, then top-512 inside them);
* the dense pass (no indexer or top-k) over a 2,048-row chunk at L = 4,096;
* the oracle timed on the host cores on a bounded sample of the same step;
* the box's achievable rates in the same run (a 1 GiB streaming copy, an 8,192^3
  bf16 GEMM), and every fraction of a nominal peak also against them.

    python bench.py [--gpus 1] [--steps 500] [--warmup 20]

Profile summaries (no GPU needed; reads rocprofv3's SQLite output):
    python bench.py --summarize-trace DB --label NAME --command "..."
    python bench.py --summarize-pmc FETCH_DB WRITE_DB --command "..."
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sqlite3
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)
CSRC = os.path.join(ROOT, "attention_page_table_amd", "csrc")
PROFILES = os.path.join(ROOT, "profiles")

HBM_PEAK_GBS = 8000.0
MFMA_BF16_PEAK_TFLOPS = 2500.0
ROW_BYTES = 512 * 2 + 64 * 2
CAL_BYTES = 1 << 30            # the calibration stream: read 1 GiB, write 1 GiB

# entry point -> (kernels it launches, by name prefix; source file). The decode step's
# calls and the prefill chunk's launch different kernels for top-k and attention, so
# they are separate entries; the latent write is one kernel in both (its decode grid is
# the one launched most often).
ENTRIES = {
    "write": (("tf::latent_write_kernel [grid 768]",), "write.hip"),
    "indexer": (("tf::indexer_rows_kernel<16, 128, 0>",), "indexer.hip"),
    # the shared-prefix decode: row groups whose streams share pages score them once
    "indexer_shared": (("tf::indexer_shared_rows_kernel<128>",), "indexer.hip"),
    "indexer_prefill": (("tf::indexer_tile_kernel<16, 128, 2, 0>",), "indexer.hip"),
    # the prefill chunk's launches (its threshold and selection kernels by grid: the decode
    # batch's comparison launches the same instances at other sizes)
    "indexer_topk_fused": (("tf::indexer_tile_kernel<16, 128, 2, 2>", "tf::fused_threshold_kernel<32> [grid 131072]",
                            "tf::indexer_tile_kernel<16, 128, 2, 3>", "tf::fused_select_kernel<16, 128> [grid 262144]"),
                           "indexer.hip"),
    "topk": (("tf::topk_stage1_kernel<4, true>", "tf::topk_stage2_kernel<4> [grid 8192]"), "topk.hip"),
    "topk_prefill": (("tf::topk_row_kernel<28, true>",), "topk.hip"),
    "attention": (("tf::attn_decode_kernel", "tf::attn_merge_kernel"), "attention.hip"),
    "attention_prefill": (("tf::attn_kernel_w32",), "attention.hip"),
    "attention_dense": (("tf::attn_dense_kernel_w32",), "attention.hip"),
    "attention_fp8": (("tf::attn_kernel_w32_fp8",), "attention.hip"),
    "snapshot": (("tf::snapshot_kernel",), "write.hip"),
}
TRAFFIC_FILE = "traffic_bench_decode_8x131072_prefill_indexer_2048_at_100000.json"
CAL_KERNEL = "neg_kernel"      # torch.neg over CAL_BYTES of float32: a plain streaming copy


class TimingEvent:
    """A HIP event for timing only, created with hipEventDisableSystemFence: recording it
    skips the system-scope fence (an L2 write-back and invalidate) that a default event
    performs, which both lengthens the measured interval and slows the launches after
    it. Recorded on the current stream (the one the library's calls go to); read after
    a device synchronize. Bound to the HIP runtime the process already loaded (torch's)."""
    _hip = None
    FLAGS = 0x20000000   # hipEventDisableSystemFence

    def __init__(self):
        import ctypes
        import torch
        if TimingEvent._hip is None:
            h = ctypes.CDLL(os.path.join(os.path.dirname(torch.__file__), "lib", "libamdhip64.so"))
            h.hipEventCreateWithFlags.argtypes = [ctypes.POINTER(ctypes.c_void_p), ctypes.c_uint]
            h.hipEventRecord.argtypes = [ctypes.c_void_p, ctypes.c_void_p]
            h.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p, ctypes.c_void_p]
            h.hipEventDestroy.argtypes = [ctypes.c_void_p]
            TimingEvent._hip = h
        self._ct = ctypes
        self.ev = ctypes.c_void_p()
        rc = TimingEvent._hip.hipEventCreateWithFlags(ctypes.byref(self.ev), TimingEvent.FLAGS)
        assert rc == 0, f"hipEventCreateWithFlags failed ({rc})"

    def record(self):
        import torch
        rc = TimingEvent._hip.hipEventRecord(self.ev, self._ct.c_void_p(torch.cuda.current_stream().cuda_stream))
        assert rc == 0, f"hipEventRecord failed ({rc})"

    def elapsed_time(self, end) -> float:
        """Milliseconds from this event to `end` (both recorded and complete)."""
        ms = self._ct.c_float()
        rc = TimingEvent._hip.hipEventElapsedTime(self._ct.byref(ms), self.ev, end.ev)
        assert rc == 0, f"hipEventElapsedTime failed ({rc})"
        return float(ms.value)

    def __del__(self):
        if TimingEvent._hip is not None and self.ev:
            TimingEvent._hip.hipEventDestroy(self.ev)


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def source_hash(name):
    return hashlib.sha256(open(os.path.join(CSRC, name), "rb").read()).hexdigest()[:16]


def load_traffic(entry, traffic_file=TRAFFIC_FILE):
    """HBM bytes per launch of an entry point from the committed counter summary, or
    None when there is none or the kernel source changed since it was taken."""
    p = os.path.join(PROFILES, traffic_file)
    if not os.path.exists(p):
        return None
    d = json.load(open(p))
    e = d.get("entries", {}).get(entry)
    if e is None or e.get("source_sha256_16") != source_hash(ENTRIES[entry][1]):
        return None
    return e.get("hbm_bytes_per_launch")


LEGS = ("decode", "prefill", "dense", "c4", "c5", "cpu", "peaks")


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=500)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--replicas", type=int, default=6, help="pool copies rotated between steps")
    ap.add_argument("--legs", default=",".join(LEGS), help="comma list of " + ",".join(LEGS))
    ap.add_argument("--no-prefill", action="store_true", help="same as leaving prefill, dense, c4, c5 out of --legs")
    ap.add_argument("--prefill-reps", type=int, default=5, help="timed passes of the whole prefill-chunk step")
    ap.add_argument("--dense-reps", type=int, default=10, help="timed calls of the dense pass")
    ap.add_argument("--call-steps", type=int, default=100,
                    help="decode steps whose calls are each bracketed by events (after the timed region)")
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=10.0, help="oracle sample length")
    ap.add_argument("--summarize-trace", metavar="DB")
    ap.add_argument("--summarize-pmc", nargs=2, metavar=("FETCH_DB", "WRITE_DB"))
    ap.add_argument("--traffic-file", default=TRAFFIC_FILE, help="profiles/ file --summarize-pmc writes")
    ap.add_argument("--summarize-counters", metavar="DB", help="per-kernel averages of a rocprofv3 --pmc pass")
    ap.add_argument("--kernels", default="", help="comma list of kernel-name prefixes for --summarize-counters")
    ap.add_argument("--label", default="decode_step")
    ap.add_argument("--command", default="")
    ap.add_argument("--bench-json", help="the line an unprofiled run of the same command printed")
    args = ap.parse_args()
    if args.summarize_trace:
        summarize_trace(args.summarize_trace, args.label, args.command, args.bench_json)
        return
    if args.summarize_pmc:
        summarize_pmc(*args.summarize_pmc, args.command, args.traffic_file)
        return
    if args.summarize_counters:
        summarize_counters(args.summarize_counters, args.label, args.command, args.kernels.split(","))
        return
    if args.gpus != 1:
        print(f"bench.py measures one GPU: this library has no multi-GPU path (asked for --gpus {args.gpus}).",
              file=sys.stderr)
        sys.exit(2)
    legs = set(x for x in args.legs.split(",") if x)
    unknown = legs - set(LEGS)
    if unknown:
        print(f"unknown legs {sorted(unknown)}; choose from {','.join(LEGS)}", file=sys.stderr)
        sys.exit(2)
    if args.no_prefill:
        legs -= {"prefill", "dense", "c4", "c5"}
    if args.no_cpu:
        legs.discard("cpu")

    import torch

    import attention_page_table_amd as tf

    assert torch.cuda.is_available(), "bench.py needs the GPU"
    tf.lib()  # fails loudly when the HIP library is missing

    line = {"metric": "paged DSA decode: latent GB/s (% HBM peak); prefill chunk indexer % MFMA peak",
            "value": None, "unit": "GB/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
            "ms_per_step": None, "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
            "dtype": "bf16", "data": "synthetic"}
    dec = None
    if "decode" in legs:
        dec = bench_decode(tf, args)
        line.update(dec["line"])
    if "prefill" in legs:
        line["prefill_indexer"], line["prefill_step"], pcpu = bench_prefill(tf, args, "cpu" in legs)
        line["cpu_baseline_prefill_chunk"] = pcpu
    if "dense" in legs:
        line["dense_pass"] = bench_dense(tf, args.dense_reps)
    if "c4" in legs:
        line["shared_prefix_decode_12_caches"] = bench_shared_prefix(tf)
    if "c5" in legs:
        line["adaptive_prefill"] = bench_adaptive_prefill(tf)
    if "cpu" in legs and dec is not None:
        cpu = cpu_baseline(dec["wl"], dec["rows"], dec["ld"], dec["scale"], args.cpu_seconds, dec["value_bytes"])
        cpu["gpu_over_cpu"] = round(line["value"] / cpu["value"], 1)
        line["cpu_baseline"] = cpu
    if "peaks" in legs:
        line["achievable_peaks"] = measure_peaks(torch)
        annotate_achievable(line, line["achievable_peaks"])
    print(json.dumps(line), flush=True)


def measure_peaks(torch, reps=20):
    """The box's achievable rates, measured in the same run after the legs (warm clocks):
    a streaming copy (torch.neg over 1 GiB of float32: 1 GiB read and 1 GiB written) and
    an 8,192^3 bf16 GEMM (torch.mm, both operands contiguous). Median of `reps` event
    intervals, each holding one launch."""
    torch.cuda.empty_cache()
    src = torch.ones(CAL_BYTES // 4, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    g = torch.Generator(device="cuda")
    g.manual_seed(0)
    n = 8192
    a = torch.randn(n, n, device="cuda", dtype=torch.bfloat16, generator=g)
    b = torch.randn(n, n, device="cuda", dtype=torch.bfloat16, generator=g)
    c = torch.empty(n, n, device="cuda", dtype=torch.bfloat16)

    def timed(fn):
        for _ in range(3):
            fn()
        ev = [TimingEvent() for _ in range(reps + 1)]
        ev[0].record()
        for i in range(reps):
            fn()
            ev[i + 1].record()
        torch.cuda.synchronize()
        return _median([ev[i].elapsed_time(ev[i + 1]) for i in range(reps)])   # ms

    copy_ms = timed(lambda: torch.neg(src, out=dst))
    gemm_ms = timed(lambda: torch.mm(a, b, out=c))
    copy_gbs = 2 * CAL_BYTES / (copy_ms * 1e-3) / 1e9
    gemm_tfl = 2.0 * n ** 3 / (gemm_ms * 1e-3) / 1e12
    del src, dst, a, b, c
    torch.cuda.empty_cache()
    return {"copy_GBps": round(copy_gbs, 1), "copy": "torch.neg over 1 GiB of float32 (bytes read + written)",
            "copy_frac_of_hbm_peak": round(copy_gbs / HBM_PEAK_GBS, 4),
            "gemm_bf16_TFLOPs": round(gemm_tfl, 1), "gemm": "torch.mm, bf16, 8192 x 8192 x 8192",
            "gemm_frac_of_mfma_peak": round(gemm_tfl / MFMA_BF16_PEAK_TFLOPS, 4), "reps": reps}


def annotate_achievable(obj, peaks):
    """Beside every fraction of a nominal peak, the same figure against the measured one:
    roofline objects get `achievable` and `frac_achievable`; fields frac_hbm* and
    frac_mfma* get a twin with the suffix _achievable."""
    if isinstance(obj, list):
        for v in obj:
            annotate_achievable(v, peaks)
        return
    if not isinstance(obj, dict) or obj is peaks:
        return
    hbm, mfma = peaks["copy_GBps"], peaks["gemm_bf16_TFLOPs"]
    if {"bound", "achieved", "peak", "unit"} <= obj.keys():
        ach = hbm if obj["unit"] == "GB/s" else (mfma if obj["unit"] == "TFLOP/s" else None)
        if ach:
            obj["achievable"] = ach
            obj["frac_achievable"] = round(obj["achieved"] / ach, 4)
    for key in list(obj.keys()):
        if key.startswith("frac_hbm") and isinstance(obj[key], (int, float)):
            obj[key + "_achievable"] = round(obj[key] * HBM_PEAK_GBS / hbm, 4)
        elif key.startswith("frac_mfma") and isinstance(obj[key], (int, float)):
            obj[key + "_achievable"] = round(obj[key] * MFMA_BF16_PEAK_TFLOPS / mfma, 4)
    for v in list(obj.values()):
        annotate_achievable(v, peaks)


def _mean(xs):
    return float(sum(xs) / len(xs))


def _median(xs):
    v = sorted(xs)
    n = len(v)
    return float(v[n // 2] if n % 2 else 0.5 * (v[n // 2 - 1] + v[n // 2]))


def bench_decode(tf, args):
    """The decode batch (8 streams x 131,072 tokens): K timed steps of write -> indexer ->
    top-k -> attention, then `call_steps` more steps with an event between every call,
    which give each call's duration (mean over those launches, each with the step's
    other calls around it) and so the dominant call and its roofline."""
    import numpy as np
    import torch

    from synth import TAG_LATENT, TAG_PKEY
    from synth.configs import LAT, ROPE, ROW, decode_batch
    from synth.device import _rid, alloc_pool, fill_bf16, populate, query_inputs

    wl = decode_batch(0)
    plan = tf.kv_pool_plan(tf.geom(1, wl.Dk))
    log(f"setup: {wl.name}: pool {wl.n_pages} pages x {plan.page_bytes} B, {args.replicas} copies")
    P0 = alloc_pool(wl, plan)
    populate(P0)
    pools = [P0.pool] + [P0.pool.clone() for _ in range(args.replicas - 1)]
    views = [tf.view(p, P0.pt, wl.pt_stride, wl.n_pages) for p in pools]
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
    scale = 1.0 / math.sqrt(576.0)
    torch.cuda.synchronize()

    names = ["write", "indexer", "topk", "attention"]
    launches = []
    for v in views:
        launches.append([
            tf.latent_write(plan, v, rs, rp, lat_new, rope_new, pkey_stream=rs, pkey_idx=kidx, pkeys=key_new,
                            prepare=True),
            tf.indexer_logits(plan, v, rs, rp, iq, w, logits, n_valid=nv, prepare=True),
            tf.topk_blocks(logits, nv, wl.k, blocks, prepare=True),
            tf.sparse_mla_attn(plan, v, rs, rp, q, scale, blocks, out, lse, prepare=True),
        ])
    for i in range(max(args.warmup, 3)):
        for f in launches[i % len(launches)]:
            f()
    # calibration stream for the HBM byte counters (outside the timed region)
    cal_src = torch.ones(CAL_BYTES // 4, dtype=torch.float32, device="cuda")
    cal_dst = torch.empty_like(cal_src)
    torch.neg(cal_src, out=cal_dst)
    del cal_src, cal_dst
    torch.cuda.synchronize()

    # ------------------------------------------------------------------ timed region: exactly K steps
    K = args.steps
    t_start, t_end = TimingEvent(), TimingEvent()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    t_start.record()
    for i in range(K):
        for f in launches[i % len(launches)]:
            f()
    t_end.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_per_step = t_start.elapsed_time(t_end) / K

    # ------------------------------------------------------------------ per-call durations
    # Whole steps again, `call_steps` of them for each of five placements of a second event:
    # right after the step's start event (nothing between: what an event itself adds), or
    # after call c. Every step runs all four calls; each interval holds one event's own
    # dispatch, so call c's duration in the step is the difference of the mean intervals
    # ending after c and after the call before it, and the event's cost cancels.
    S = max(50, args.call_steps)
    cum = []
    for c in range(-1, 4):
        e0, e1 = [TimingEvent() for _ in range(S)], [TimingEvent() for _ in range(S)]
        for i in range(S):
            ls = launches[i % len(launches)]
            e0[i].record()
            if c < 0:
                e1[i].record()
            for j in range(4):
                ls[j]()
                if j == c:
                    e1[i].record()
        torch.cuda.synchronize()
        cum.append([e0[i].elapsed_time(e1[i]) * 1e3 for i in range(S)])
    avg_us = {n: _mean(cum[c + 1]) - _mean(cum[c]) for c, n in enumerate(names)}
    med_us = {n: _median(cum[c + 1]) - _median(cum[c]) for c, n in enumerate(names)}
    dom = max(["indexer", "topk", "attention"], key=lambda n: avg_us[n])

    lat_bytes = R * wl.k * 4 * ROW_BYTES                       # selected latent + rope rows
    key_bytes = R * ld * wl.Dk * 2                             # every visible pooled key (all rows see ld)
    alg_bytes = {
        "write": R * (ROW_BYTES + wl.Dk * 2) * 2 + R * 16,
        "indexer": key_bytes + R * ld * 4 + R * wl.H * (wl.Dk * 2 + 4) + R * 12,
        "topk": R * ld * 4 + R * wl.k * 4 + R * 4,
        "attention": lat_bytes + R * wl.Hq * 576 * 2 + R * wl.Hq * (512 + 1) * 4 + R * wl.k * 4 + R * 8,
    }
    value = (lat_bytes + key_bytes) / (ms_per_step * 1e-3) / 1e9
    kern = {n: {"us": round(avg_us[n], 3), "us_median": round(med_us[n], 3), "alg_bytes": alg_bytes[n],
                "GBps": round(alg_bytes[n] / (avg_us[n] * 1e-6) / 1e9, 1)} for n in names}
    achieved = alg_bytes[dom] / (avg_us[dom] * 1e-6) / 1e9
    roofline = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": load_traffic(dom),
                "kernel": f"tf_{'sparse_mla_attn' if dom == 'attention' else dom}",
                "launches": list(ENTRIES[dom][0]), "alg_bytes_per_launch": alg_bytes[dom],
                "avg_launch_us": round(avg_us[dom], 2), "timed_launches": S}
    att_gbs = lat_bytes / (avg_us["attention"] * 1e-6) / 1e9
    headline = {"call": "tf_sparse_mla_attn", "launches": list(ENTRIES["attention"][0]),
                "latent_bytes": lat_bytes, "us": round(avg_us["attention"], 2),
                "latent_GBps": round(att_gbs, 1), "frac_hbm": round(att_gbs / HBM_PEAK_GBS, 4),
                "timed_launches": S,
                "note": "selected latent + rope rows gathered (8 rows x 2,048 tokens x 1,152 B) / the call's "
                        "duration in the step"}
    indexer_scan = {"call": "tf_indexer_logits", "key_bytes": key_bytes, "us": round(avg_us["indexer"], 2),
                    "key_GBps": round(key_bytes / (avg_us["indexer"] * 1e-6) / 1e9, 1)}
    # the fused indexer + top-k on the same rows (no logits written), against the pair
    fb = torch.empty_like(blocks)
    fused = [tf.indexer_topk_fused(plan, v, rs, rp, iq, w, ld, wl.k, fb, prepare=True) for v in views]
    launches[0][1]()
    launches[0][2]()
    fused[0]()
    torch.cuda.synchronize()
    assert torch.equal(fb, blocks), "fused indexer + top-k differs from the pair"
    fev = [TimingEvent() for _ in range(S + 1)]
    fev[0].record()
    for i in range(S):
        fused[i % len(fused)]()
        fev[i + 1].record()
    torch.cuda.synchronize()
    fus = _mean([fev[i].elapsed_time(fev[i + 1]) * 1e3 for i in range(S)])
    fused_res = {"call": "tf_indexer_topk_fused", "us": round(fus, 2),
                 "pair_us": round(avg_us["indexer"] + avg_us["topk"], 2), "equal_to_pair": True,
                 "workspace_bytes": tf.indexer_topk_fused_workspace_bytes(R, ld, wl.k, wl.H),
                 "pair_logits_bytes": R * ld * 4}
    del launches, views, pools, P0, fused
    torch.cuda.empty_cache()
    return {"wl": wl, "rows": rows, "ld": ld, "scale": scale, "value_bytes": lat_bytes + key_bytes,
            "line": {
                "value": round(value, 1), "ms_per_step": round(ms_per_step, 5),
                "config": {"workload": wl.name, "streams": R, "context": wl.lengths[0], "caches": 1,
                           "attn_heads": wl.Hq, "indexer_heads": wl.H, "index_dim": wl.Dk, "topk_blocks": wl.k,
                           "page_rows": 512, "pool_pages": wl.n_pages, "pool_copies": args.replicas,
                           "value_bytes_per_step": lat_bytes + key_bytes,
                           "value": "paged-cache bytes one decode step reads (visible pooled keys + selected "
                                    "latent and rope rows) / time per step",
                           "launches": "eager, marshalled once",
                           "kernels_timing": f"per call: differences of mean event intervals from a step's start to "
                                  f"after the call and after the call before it, {S} steps each"},
                "decode_attention_latent": headline,
                "decode_indexer_keys": indexer_scan,
                "decode_fused_indexer_topk": fused_res,
                "roofline": roofline,
                "kernels": kern,
                "wall_s_timed": round(wall, 4)}}


def bench_prefill(tf, args, with_cpu):
    """The prefill chunk (2,048 rows against 100,000 tokens): the indexer alone against
    the MFMA roofline, then the whole chunk step call by call; optionally the oracle on
    a sample of the chunk's rows."""
    import numpy as np
    import torch

    from synth.configs import prefill_chunk
    from synth.device import alloc_pool, populate, query_inputs
    pw = prefill_chunk(0)
    pplan = tf.kv_pool_plan(tf.geom(1, pw.Dk))
    log(f"setup: {pw.name}")
    PP = alloc_pool(pw, pplan)
    populate(PP)
    prs, prp, piq, pww, _ = query_inputs(pw, 0, pw.rows)
    pld = (pw.rows[-1][1]) // 4 + 1
    plog = torch.empty((len(pw.rows), pld), dtype=torch.float32, device="cuda")
    pnv = torch.empty(len(pw.rows), dtype=torch.int32, device="cuda")
    f = tf.indexer_logits(pplan, PP.view(), prs, prp, piq, pww, plog, n_valid=pnv, prepare=True)
    for _ in range(3):
        f()
    torch.cuda.synchronize()
    reps = 20
    pe = [TimingEvent() for _ in range(reps + 1)]
    pe[0].record()
    for i in range(reps):
        f()
        pe[i + 1].record()
    torch.cuda.synchronize()
    us = float(np.mean([pe[i].elapsed_time(pe[i + 1]) for i in range(reps)])) * 1e3
    flops = sum(2 * pw.H * pw.Dk * (t // 4 + 1) for _, t in pw.rows)
    tfl = flops / (us * 1e-6) / 1e12
    prefill = {"call": "tf_indexer_logits", "launches": list(ENTRIES["indexer_prefill"][0]),
               "workload": pw.name, "rows": len(pw.rows), "keys": pld, "us": round(us, 2), "reps": reps,
               "causal_flop": flops,
               "roofline": {"bound": "mfma", "achieved": round(tfl, 1), "peak": MFMA_BF16_PEAK_TFLOPS,
                            "unit": "TFLOP/s", "frac": round(tfl / MFMA_BF16_PEAK_TFLOPS, 4),
                            "traffic": load_traffic("indexer_prefill")}}
    step = bench_prefill_step(tf, pw, pplan, PP, prs, prp, piq, pww, plog, pnv, args.prefill_reps)
    del PP, plog
    torch.cuda.empty_cache()
    cpu = cpu_baseline_prefill(pw, args.cpu_seconds, step["us_per_step"]) if with_cpu else None
    return prefill, step, cpu


def bench_prefill_step(tf, pw, plan, PP, rs, rp, iq, w, logits, nv, reps):
    """The whole hot path over one prefill chunk (rows [97,952, 100,000) of one stream
    against its 100,000-token prefix): write the chunk's rows and pooled keys, logits
    over every visible key, top-512 per row, attention with 32 heads. Each call is
    timed with fence-free events over `reps` passes; the pool is resident."""
    import numpy as np
    import torch
    from synth import TAG_LATENT, TAG_PKEY, TAG_Q
    from synth.configs import LAT, ROPE, ROW
    from synth.device import _rid, fill_bf16
    T = len(pw.rows)
    t0 = pw.rows[0][1]
    r0 = _rid(0, 0, t0)
    lat = torch.empty((T, LAT), dtype=torch.bfloat16, device="cuda")
    rope = torch.empty((T, ROPE), dtype=torch.bfloat16, device="cuda")
    fill_bf16(lat, T, LAT, pw.seed, TAG_LATENT, r0 * ROW, ROW, ROW)
    fill_bf16(rope, T, ROPE, pw.seed, TAG_LATENT, r0 * ROW + LAT, ROW, ROW)
    j0, j1 = (t0 + 3) // 4, (t0 + T + 3) // 4
    keys = torch.empty((j1 - j0, pw.Dk), dtype=torch.bfloat16, device="cuda")
    fill_bf16(keys, j1 - j0, pw.Dk, pw.seed, TAG_PKEY, _rid(0, 0, j0) * pw.Dk, pw.Dk, pw.Dk)
    ks = torch.zeros(j1 - j0, dtype=torch.int32, device="cuda")
    ki = torch.arange(j0, j1, dtype=torch.int32, device="cuda")
    q = torch.empty((T, pw.Hq, ROW), dtype=torch.bfloat16, device="cuda")
    fill_bf16(q, T * pw.Hq, ROW, pw.seed, TAG_Q, r0 * pw.Hq * ROW, ROW, ROW)
    blocks = torch.empty((T, pw.k), dtype=torch.int32, device="cuda")
    out = torch.empty((T, pw.Hq, 512), dtype=torch.float32, device="cuda")
    lse = torch.empty((T, pw.Hq), dtype=torch.float32, device="cuda")
    scale = 1.0 / math.sqrt(576.0)
    view = PP.view()
    calls = [
        ("write", tf.latent_write(plan, view, rs, rp, lat, rope, pkey_stream=ks, pkey_idx=ki, pkeys=keys,
                                  prepare=True)),
        ("indexer", tf.indexer_logits(plan, view, rs, rp, iq, w, logits, n_valid=nv, prepare=True)),
        ("topk", tf.topk_blocks(logits, nv, pw.k, blocks, prepare=True)),
        ("attention", tf.sparse_mla_attn(plan, view, rs, rp, q, scale, blocks, out, lse, prepare=True)),
    ]
    for _, f in calls:
        f()
    torch.cuda.synchronize()
    ev = [[TimingEvent() for _ in range(len(calls) + 1)] for _ in range(reps)]
    for i in range(reps):
        ev[i][0].record()
        for c, (_, f) in enumerate(calls):
            f()
            ev[i][c + 1].record()
    torch.cuda.synchronize()
    us = {n: float(np.mean([ev[i][c].elapsed_time(ev[i][c + 1]) for i in range(reps)])) * 1e3
          for c, (n, _) in enumerate(calls)}
    step_us = float(np.mean([ev[i][0].elapsed_time(ev[i][-1]) for i in range(reps)])) * 1e3
    nvh = nv.cpu().numpy().astype(np.int64)
    blk = blocks.cpu().numpy()
    sel = 0
    for r, (_, t) in enumerate(pw.rows):                               # exact: tokens s <= t of the selected blocks
        b = blk[r][blk[r] >= 0].astype(np.int64)
        sel += int(np.minimum(4, np.maximum(0, t + 1 - 4 * b)).sum())
    attn_flop = sel * 2 * pw.Hq * (576 + 512)                         # S over 576 dims, P.V over 512
    idx_flop = int(sum(2 * pw.H * pw.Dk * int(n) for n in nvh))
    def mfma(flop, t_us):
        a = flop / (t_us * 1e-6) / 1e12
        return {"bound": "mfma", "achieved": round(a, 1), "peak": MFMA_BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                "frac": round(a / MFMA_BF16_PEAK_TFLOPS, 4)}
    def hbm(nbytes, t_us):
        a = nbytes / (t_us * 1e-6) / 1e9
        return {"bound": "hbm", "achieved": round(a, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(a / HBM_PEAK_GBS, 4)}
    res = {
        "workload": pw.name, "rows": T, "keys": int(logits.shape[1]), "topk_blocks": pw.k, "attn_heads": pw.Hq,
        "us_per_step": round(step_us, 1), "reps": reps,
        "calls": {
            "write": {"us": round(us["write"], 2),
                      "roofline": hbm(2 * (T * ROW_BYTES + (j1 - j0) * pw.Dk * 2), us["write"])},
            "indexer": {"us": round(us["indexer"], 2), "causal_flop": idx_flop,
                        "roofline": mfma(idx_flop, us["indexer"])},
            "topk": {"us": round(us["topk"], 2), "roofline": hbm(int(logits.numel()) * 4, us["topk"])},
            "attention": {"us": round(us["attention"], 2), "selected_tokens": sel, "flop": attn_flop,
                          "gathered_bytes": sel * ROW_BYTES,
                          "gathered_GBps": round(sel * ROW_BYTES / (us["attention"] * 1e-6) / 1e9, 1),
                          "roofline": mfma(attn_flop, us["attention"])},
        },
        "quantizing_write": bench_quantizing_write(tf, pw, rs, rp, lat, rope, ks, ki, keys, reps, hbm),
        "blocked_indexer_topk": bench_blocked_indexer_topk(tf, pw, plan, view, rs, rp, iq, w, logits, blocks, reps,
                                                           idx_flop, us["indexer"] + us["topk"], mfma),
        "fused_indexer_topk": bench_fused_indexer_topk(tf, plan, view, rs, rp, iq, w, logits, blocks, reps,
                                                       idx_flop, us["indexer"] + us["topk"], mfma, dict(calls)),
        "candidate_selection": bench_candidates(tf, logits, nv, pw.k, reps, hbm),
    }
    return res


def bench_fused_indexer_topk(tf, plan, view, rs, rp, iq, w, logits, ref_blocks, reps, flop, unblocked_us, mfma,
                             step_calls):
    """The chunk's top-512 by tf_indexer_topk_fused, which writes no logits: a page
    sample sets each row's threshold, the filtered scoring keeps about 2k candidates a
    row, the last kernel selects among them. Timed inside the step, in place of the
    indexer and top-k calls (write, fused, attention, an event between calls), as the
    pair is: back-to-back launches of one MFMA-bound kernel run slower than the same
    launches between the step's other calls. Its workspace against the [T, 25,000]
    logits buffer; the result is checked equal to the step's. The roofline counts the
    causal flop of one scoring pass (the sample's work is overhead)."""
    import numpy as np
    import torch
    T, ld = logits.shape
    k = ref_blocks.shape[1]
    got = torch.empty_like(ref_blocks)
    ws_bytes = tf.indexer_topk_fused_workspace_bytes(T, ld, k, w.shape[1])
    f = tf.indexer_topk_fused(plan, view, rs, rp, iq, w, ld, k, got, prepare=True)
    f()
    torch.cuda.synchronize()
    assert torch.equal(got, ref_blocks), "fused indexer + top-k differs from the unblocked path"
    calls = [step_calls["write"], f, step_calls["attention"]]
    ev = [[TimingEvent() for _ in range(len(calls) + 1)] for _ in range(reps)]
    for i in range(reps):
        ev[i][0].record()
        for c, g in enumerate(calls):
            g()
            ev[i][c + 1].record()
    torch.cuda.synchronize()
    us = float(np.mean([ev[i][1].elapsed_time(ev[i][2]) for i in range(reps)])) * 1e3
    b2b = TimingEvent(), TimingEvent()
    b2b[0].record()
    for i in range(reps):
        f()
    b2b[1].record()
    torch.cuda.synchronize()
    return {"call": "tf_indexer_topk_fused", "us": round(us, 2), "unblocked_indexer_plus_topk_us": round(unblocked_us, 2),
            "us_back_to_back": round(b2b[0].elapsed_time(b2b[1]) * 1e3 / reps, 2),
            "timing": "in the step in place of the indexer and top-k calls, as they are timed",
            "workspace_bytes": ws_bytes, "unblocked_logits_bytes": T * ld * 4, "causal_flop": flop,
            "roofline": mfma(flop, us), "equal_to_unblocked": True}


def bench_candidates(tf, logits, nv, k, reps, hbm, group=8, n_cand=2048):
    """Two-level selection on the chunk's logits: the candidate layer's top-2,048 groups
    of 8 keys (tf_candidate_groups: reads the logits, writes the group maxima, selects),
    then a consumer's top-512 inside them (tf_topk_in_candidates: the top-k with the
    non-candidates read as -inf). Algorithmic bytes: the logits read and the group
    maxima written; the logits and the candidate lists read."""
    import numpy as np
    import torch
    T, ld = logits.shape
    cand = torch.empty((T, n_cand), dtype=torch.int32, device="cuda")
    f1 = tf.candidate_groups(logits, nv, group, n_cand, cand, prepare=True)
    blk = torch.empty((T, k), dtype=torch.int32, device="cuda")
    f2 = tf.topk_in_candidates(logits, nv, cand, group, k, blk, prepare=True)
    f1()
    f2()
    torch.cuda.synchronize()
    res = {}
    for name, f in (("candidate_groups", f1), ("topk_in_candidates", f2)):
        ev = [TimingEvent() for _ in range(reps + 1)]
        ev[0].record()
        for i in range(reps):
            f()
            ev[i + 1].record()
        torch.cuda.synchronize()
        res[name] = float(np.mean([ev[i].elapsed_time(ev[i + 1]) for i in range(reps)])) * 1e3
    nvh = nv.cpu().numpy().astype(np.int64)
    n_groups = (nvh + group - 1) // group
    b1 = int(nvh.sum()) * 4 + int(n_groups.sum()) * 4
    b2 = int(nvh.sum()) * 4 + int(nvh.size) * n_cand * 4
    return {"group": group, "n_cand": n_cand, "k": k,
            "candidate_groups": {"us": round(res["candidate_groups"], 2), "alg_bytes": b1,
                                 "roofline": hbm(b1, res["candidate_groups"])},
            "topk_in_candidates": {"us": round(res["topk_in_candidates"], 2), "alg_bytes": b2,
                                   "roofline": hbm(b2, res["topk_in_candidates"])}}


def bench_blocked_indexer_topk(tf, pw, plan, view, rs, rp, iq, w, logits, ref_blocks, reps, flop, unblocked_us,
                               mfma, key_block=8192):
    """The same chunk's logits and top-512 by key blocks (tf_indexer_topk): each block of
    8,192 keys scored into a flat workspace, its top-k candidates kept, one merge. Its
    device memory against the whole [T, 25,000] logits buffer, and its time against the
    indexer and top-k calls of the step; the result is checked equal to the step's."""
    import numpy as np
    import torch
    T, ld = logits.shape
    k = ref_blocks.shape[1]
    got = torch.empty_like(ref_blocks)
    ws_bytes = tf.indexer_topk_workspace_bytes(T, ld, k, key_block)
    f = tf.indexer_topk(plan, view, rs, rp, iq, w, ld, k, key_block, got, prepare=True)
    f()
    torch.cuda.synchronize()
    assert torch.equal(got, ref_blocks), "key-blocked top-k differs from the whole-buffer top-k"
    ev = [TimingEvent() for _ in range(reps + 1)]
    ev[0].record()
    for i in range(reps):
        f()
        ev[i + 1].record()
    torch.cuda.synchronize()
    us = float(np.mean([ev[i].elapsed_time(ev[i + 1]) for i in range(reps)])) * 1e3
    return {"call": "tf_indexer_topk", "key_block": key_block, "blocks": (ld + key_block - 1) // key_block,
            "us": round(us, 2), "unblocked_indexer_plus_topk_us": round(unblocked_us, 2),
            "workspace_bytes": ws_bytes, "unblocked_logits_bytes": T * ld * 4, "causal_flop": flop,
            "roofline": mfma(flop, us), "equal_to_unblocked": True}


def bench_quantizing_write(tf, pw, rs, rp, lat, rope, ks, ki, keys, reps, hbm):
    """The same chunk's rows and keys written into fp8 pages by tf_latent_write_quantize
    (the adaptive-prefill workload's row format: e4m3 codes and a row scale, bf16 rope):
    a pool of just the chunk's pages, reached through a table whose other entries are
    empty. Algorithmic bytes: the bf16 rows and keys read, the codes, scales, rope and
    keys written."""
    import numpy as np
    import torch
    plan8 = tf.kv_pool_plan(tf.geom(1, pw.Dk, fp8=True))
    T = lat.shape[0]
    t0 = pw.rows[0][1]
    p0, p1 = t0 // 512, (t0 + T - 1) // 512 + 1
    pool = torch.zeros((p1 - p0) * plan8.page_bytes, dtype=torch.uint8, device="cuda")
    pt = torch.full((1, p1), -1, dtype=torch.int32, device="cuda")
    pt[0, p0:p1] = torch.arange(p1 - p0, dtype=torch.int32, device="cuda")
    view = tf.view(pool, pt, p1, p1 - p0)
    f = tf.latent_write_quantize(plan8, view, rs, rp, lat, rope, ks, ki, keys, prepare=True)
    f()
    torch.cuda.synchronize()
    ev = [TimingEvent() for _ in range(reps + 1)]
    ev[0].record()
    for i in range(reps):
        f()
        ev[i + 1].record()
    torch.cuda.synchronize()
    us = float(np.mean([ev[i].elapsed_time(ev[i + 1]) for i in range(reps)])) * 1e3
    nk = keys.shape[0]
    nbytes = T * (1024 + 128) + nk * pw.Dk * 2 + T * (512 + 4 + 128) + nk * pw.Dk * 2
    return {"call": "tf_latent_write_quantize", "rows": T, "keys": nk, "us": round(us, 2), "alg_bytes": nbytes,
            "roofline": hbm(nbytes, us)}


def bench_dense(tf, reps):
    """The dense pass (tf_dense_mla_attn, no indexer or top-k) over a 2,048-row chunk at
    L = 4,096: rows [2,048, 4,096) of one stream, each over its whole causal range
    (n_blocks = 1,024), 32 heads. Timed with fence-free events over `reps` back-to-back
    calls; the pool is resident. MFMA work: 4 x 32 x 576 flop per (row, attended token),
    the scores and the value product; each attended token is a 1,152-byte row gathered."""
    import numpy as np
    import torch
    from synth.configs import prefill_chunk
    from synth.device import alloc_pool, populate, query_inputs
    dw = prefill_chunk(0, L=4096, T=2048, slack_pages=4)
    plan = tf.kv_pool_plan(tf.geom(1, dw.Dk))
    log(f"setup: dense pass over {dw.name}")
    P = alloc_pool(dw, plan)
    populate(P)
    rs, rp, _, _, q = query_inputs(dw, 0, dw.rows)
    R = len(dw.rows)
    nb = dw.rows[-1][1] // 4 + 1
    out = torch.empty((R, dw.Hq, 512), dtype=torch.float32, device="cuda")
    lse = torch.empty((R, dw.Hq), dtype=torch.float32, device="cuda")
    f = tf.dense_mla_attn(plan, P.view(), rs, rp, q, 1.0 / math.sqrt(576.0), nb, out, lse, prepare=True)
    for _ in range(3):
        f()
    torch.cuda.synchronize()
    ev = [TimingEvent() for _ in range(reps + 1)]
    ev[0].record()
    for i in range(reps):
        f()
        ev[i + 1].record()
    torch.cuda.synchronize()
    us = float(np.mean([ev[i].elapsed_time(ev[i + 1]) for i in range(reps)])) * 1e3
    tokens = sum(min(t + 1, 4 * nb) for _, t in dw.rows)
    flop = tokens * 2 * dw.Hq * (576 + 512)
    a = flop / (us * 1e-6) / 1e12
    del P
    return {"call": "tf_dense_mla_attn", "launches": list(ENTRIES["attention_dense"][0]),
            "workload": f"dense_{R}_at_{dw.lengths[0]}", "rows": R, "n_blocks": nb, "attn_heads": dw.Hq,
            "us": round(us, 2), "reps": reps, "attended_tokens": tokens, "flop": flop,
            "gathered_bytes": tokens * ROW_BYTES,
            "gathered_GBps": round(tokens * ROW_BYTES / (us * 1e-6) / 1e9, 1),
            "roofline": {"bound": "mfma", "achieved": round(a, 1), "peak": MFMA_BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                         "frac": round(a / MFMA_BF16_PEAK_TFLOPS, 4), "traffic": load_traffic("attention_dense")}}


C4_TRAFFIC_FILE = "traffic_shared_prefix_decode_8x1M_12caches.json"


def bench_shared_prefix(tf, reps=5):
    """Decode over 12 caches of 8 streams that share a 1,048,576-token prefix by page
    reference (2,048 shared pages + one private tail page each). One token's step runs the
    decode path once per cache (write -> indexer -> top-k -> attention), the caches one
    after another as a model's layers would; an event between every call. Per cache the
    attention gathers 8 x 2,048 selected rows (18.9 MB) and the indexer scans each row's
    262,144 + tail keys, of which the shared 2,048 pages' keys (67.1 MB) are the same
    bytes for all 8 rows."""
    import numpy as np
    import torch

    from synth import TAG_LATENT, TAG_PKEY
    from synth.configs import LAT, ROPE, ROW, shared_prefix_decode
    from synth.device import _rid, alloc_pool, fill_bf16, populate, query_inputs
    wl = shared_prefix_decode(0)
    plan = tf.kv_pool_plan(tf.geom(wl.n_caches, wl.Dk))
    log(f"setup: {wl.name}: pool {wl.n_pages} pages x {plan.page_bytes} B")
    P = alloc_pool(wl, plan)
    populate(P)
    rows = wl.rows
    R = len(rows)
    # logits rows padded to 16 bytes, so that top-k loads them 16 bytes at a time
    ld = (max(t // 4 + 1 for _, t in rows) + 3) // 4 * 4
    scale = 1.0 / math.sqrt(576.0)
    logits = torch.empty((R, ld), dtype=torch.float32, device="cuda")
    nv = torch.empty(R, dtype=torch.int32, device="cuda")
    blocks = torch.empty((R, wl.k), dtype=torch.int32, device="cuda")
    out = torch.empty((R, wl.Hq, 512), dtype=torch.float32, device="cuda")
    lse = torch.empty((R, wl.Hq), dtype=torch.float32, device="cuda")
    kidx = torch.tensor([t // 4 for _, t in rows], dtype=torch.int32, device="cuda")
    per_cache = []
    keep = []
    for c in range(wl.n_caches):
        rs, rp, iq, w, q = query_inputs(wl, c, rows)
        lat = torch.empty((R, LAT), dtype=torch.bfloat16, device="cuda")
        rope = torch.empty((R, ROPE), dtype=torch.bfloat16, device="cuda")
        key = torch.empty((R, wl.Dk), dtype=torch.bfloat16, device="cuda")
        for i, (b, t) in enumerate(rows):
            r0 = _rid(c, b, t)                      # tail rows are the stream's own (owner b)
            fill_bf16(lat[i:], 1, LAT, wl.seed, TAG_LATENT, r0 * ROW, ROW, ROW)
            fill_bf16(rope[i:], 1, ROPE, wl.seed, TAG_LATENT, r0 * ROW + LAT, ROW, ROW)
            fill_bf16(key[i:], 1, wl.Dk, wl.seed, TAG_PKEY, _rid(c, b, t // 4) * wl.Dk, wl.Dk, wl.Dk)
        v = P.view(c)
        keep.append((rs, rp, iq, w, q, lat, rope, key))
        per_cache.append([
            tf.latent_write(plan, v, rs, rp, lat, rope, pkey_stream=rs, pkey_idx=kidx, pkeys=key, prepare=True),
            tf.indexer_logits(plan, v, rs, rp, iq, w, logits, n_valid=nv, prepare=True),
            tf.topk_blocks(logits, nv, wl.k, blocks, prepare=True),
            tf.sparse_mla_attn(plan, v, rs, rp, q, scale, blocks, out, lse, prepare=True),
        ])
    for _ in range(2):
        for calls in per_cache:
            for f in calls:
                f()
    torch.cuda.synchronize()
    C = wl.n_caches
    ev = [[[TimingEvent() for _ in range(5)] for _ in range(C)] for _ in range(reps)]
    for i in range(reps):
        for c in range(C):
            ev[i][c][0].record()
            for j, f in enumerate(per_cache[c]):
                f()
                ev[i][c][j + 1].record()
    torch.cuda.synchronize()
    names = ["write", "indexer", "topk", "attention"]
    us = {n: [[ev[i][c][j].elapsed_time(ev[i][c][j + 1]) * 1e3 for c in range(C)] for i in range(reps)]
          for j, n in enumerate(names)}
    token_us = _mean([ev[i][0][0].elapsed_time(ev[i][C - 1][4]) * 1e3 for i in range(reps)])
    att = [_mean([us["attention"][i][c] for i in range(reps)]) for c in range(C)]
    idx = [_mean([us["indexer"][i][c] for i in range(reps)]) for c in range(C)]
    lat_bytes = R * wl.k * 4 * ROW_BYTES
    scanned = sum(t // 4 + 1 for _, t in rows) * wl.Dk * 2
    unique = (wl.shared_tokens // 4 + sum(t // 4 + 1 - wl.shared_tokens // 4 for _, t in rows)) * wl.Dk * 2
    att_gbs = [lat_bytes / (u * 1e-6) / 1e9 for u in att]
    res = {"workload": wl.name, "caches": C, "streams": R, "shared_tokens": wl.shared_tokens,
           "tails": [t + 1 - wl.shared_tokens for _, t in rows], "reps": reps,
           "token_step_us": round(token_us, 1),
           "calls_us_mean_over_caches": {n: round(_mean([x for r in us[n] for x in r]), 2) for n in names},
           "attention": {"call": "tf_sparse_mla_attn", "latent_bytes_per_cache": lat_bytes,
                         "us_per_cache": [round(u, 2) for u in att],
                         "latent_GBps_per_cache": [round(g, 1) for g in att_gbs],
                         "latent_GBps_mean": round(_mean(att_gbs), 1),
                         "frac_hbm_mean": round(_mean(att_gbs) / HBM_PEAK_GBS, 4)},
           "indexer": {"call": "tf_indexer_logits", "us_per_cache": [round(u, 2) for u in idx],
                       "keys_scanned_bytes_per_cache": scanned, "unique_key_bytes_per_cache": unique,
                       "scanned_GBps_mean": round(scanned / (_mean(idx) * 1e-6) / 1e9, 1),
                       "unique_GBps_mean": round(unique / (_mean(idx) * 1e-6) / 1e9, 1),
                       "traffic": load_traffic("indexer_shared", C4_TRAFFIC_FILE)}}
    del per_cache, keep, P
    torch.cuda.empty_cache()
    return res


def bench_adaptive_prefill(tf):
    """The 390,000-token prompt in fp8 rows, prefilled in 464 adaptive chunks
    (chunk(L) = clamp(round_down_256(2e8 / L), 256, 2048), the rule tf_prefill_chunk
    applies): per chunk, write its rows and keys, score its rows against every visible
    key, top-512, attention with 32 heads. All inputs are generated into HBM first; an
    event between every call. Then the snapshot of the first 262,144 rows (every plane
    and the keys [0, 65,536)) into another stream's pages, timed alone: each copy after
    1 GiB written (the Infinity Cache cold for the source), and back to back."""
    import numpy as np
    import torch

    from synth import TAG_LAT8, TAG_LATENT, TAG_PKEY, TAG_SCALE8
    from synth.configs import LAT, ROPE, ROW, adaptive_prefill
    from synth.device import _rid, alloc_pool, fill_bf16, fill_e4m3, fill_scale8, query_inputs
    wl = adaptive_prefill(0)
    plan = tf.kv_pool_plan(tf.geom(1, wl.Dk, fp8=True))
    N = wl.lengths[0]
    log(f"setup: {wl.name}: pool {wl.n_pages} pages x {plan.page_bytes} B; generating {N} rows of inputs")
    P = alloc_pool(wl, plan)
    view = P.view()
    sched, L = [], 0
    while L < N:
        T = tf.prefill_chunk(L, N - L)
        sched.append((L, T))
        L += T
    r0 = _rid(0, 0, 0)
    lat = torch.empty((N, LAT), dtype=torch.uint8, device="cuda")
    fill_e4m3(lat, N, LAT, wl.seed, TAG_LAT8, r0 * LAT, LAT)
    sc = torch.empty(N, dtype=torch.float32, device="cuda")
    fill_scale8(sc, N, wl.seed, TAG_SCALE8, r0)
    rope = torch.empty((N, ROPE), dtype=torch.bfloat16, device="cuda")
    fill_bf16(rope, N, ROPE, wl.seed, TAG_LATENT, r0 * ROW + LAT, ROW, ROW)
    nk = (N + 3) // 4
    keys = torch.empty((nk, wl.Dk), dtype=torch.bfloat16, device="cuda")
    fill_bf16(keys, nk, wl.Dk, wl.seed, TAG_PKEY, r0 * wl.Dk, wl.Dk, wl.Dk)
    kstream = torch.zeros(nk, dtype=torch.int32, device="cuda")
    kidx = torch.arange(nk, dtype=torch.int32, device="cuda")
    rs, rp, iq, w, q = query_inputs(wl, 0, [(0, t) for t in range(N)])
    max_log = max(T * ((L + T - 1) // 4 + 1) for L, T in sched)
    logbuf = torch.empty(max_log, dtype=torch.float32, device="cuda")
    nv = torch.empty(2048, dtype=torch.int32, device="cuda")
    blocks = torch.empty((2048, wl.k), dtype=torch.int32, device="cuda")
    out = torch.empty((2048, wl.Hq, 512), dtype=torch.float32, device="cuda")
    lse = torch.empty((2048, wl.Hq), dtype=torch.float32, device="cuda")
    tws = torch.empty(max(16, max(tf.topk_workspace_bytes(T, (L + T - 1) // 4 + 1, wl.k) for L, T in sched)),
                      dtype=torch.uint8, device="cuda")
    aws = torch.zeros(max(16, max(tf.attn_workspace_bytes(T, wl.Hq, wl.k) for _, T in sched)), dtype=torch.uint8,
                      device="cuda")
    scale = 1.0 / math.sqrt(576.0)
    torch.cuda.synchronize()

    def chunk_calls(L, T):
        ld = (L + T - 1) // 4 + 1
        j0, j1 = (L + 3) // 4, (L + T + 3) // 4
        lg = logbuf[:T * ld].view(T, ld)
        return [
            lambda: tf.latent_write(plan, view, rs[L:L + T], rp[L:L + T], lat[L:L + T], rope[L:L + T],
                                    row_scale=sc[L:L + T], pkey_stream=kstream[j0:j1], pkey_idx=kidx[j0:j1],
                                    pkeys=keys[j0:j1]),
            lambda: tf.indexer_logits(plan, view, rs[L:L + T], rp[L:L + T], iq[L:L + T], w[L:L + T], lg,
                                      n_valid=nv[:T]),
            lambda: tf.topk_blocks(lg, nv[:T], wl.k, blocks[:T], ws=tws),
            lambda: tf.sparse_mla_attn(plan, view, rs[L:L + T], rp[L:L + T], q[L:L + T], scale, blocks[:T],
                                       out[:T], lse[:T], ws=aws),
        ]
    log(f"adaptive prefill: {len(sched)} chunks")
    ev = [[TimingEvent() for _ in range(5)] for _ in sched]
    for i, (L, T) in enumerate(sched):
        ev[i][0].record()
        for j, f in enumerate(chunk_calls(L, T)):
            f()
            ev[i][j + 1].record()
    torch.cuda.synchronize()
    names = ["write", "indexer", "topk", "attention"]
    call_us = [[ev[i][j].elapsed_time(ev[i][j + 1]) * 1e3 for j in range(4)] for i in range(len(sched))]
    chunk_us = [sum(c) for c in call_us]
    total_us = ev[0][0].elapsed_time(ev[-1][4]) * 1e3
    bands = {}
    idx_flop = att_flop = 0
    for (L, T), cu, c4 in zip(sched, chunk_us, call_us):
        b = bands.setdefault(T, {"chunks": 0, "tokens": 0, "us": 0.0, "first_L": L, "indexer_us": 0.0,
                                 "attention_us": 0.0})
        b["chunks"] += 1
        b["tokens"] += T
        b["us"] += cu
        b["indexer_us"] += c4[1]
        b["attention_us"] += c4[3]
        # causal work of the chunk: every row t scores t // 4 + 1 keys; attention reads
        # min(2,048, t + 1) tokens (512 blocks, the row's own last block cut at t)
        idx_flop += 2 * wl.H * wl.Dk * sum(t // 4 + 1 for t in range(L, L + T))
        att_flop += 2 * wl.Hq * (576 + 512) * sum(min(4 * wl.k, t + 1) for t in range(L, L + T))
    for T, b in bands.items():
        b["us"] = round(b["us"], 1)
        b["indexer_us"] = round(b["indexer_us"], 1)
        b["attention_us"] = round(b["attention_us"], 1)
        b["tok_per_s"] = round(b["tokens"] / (b["us"] * 1e-6), 1)
    calls_total = {n: round(sum(c[j] for c in call_us), 1) for j, n in enumerate(names)}
    fused = adaptive_fused_pass(tf, plan, view, wl, sched, chunk_calls, rs, rp, iq, w, nv, blocks)
    # snapshot of the first 262,144 rows of stream 0 into stream 1's pages
    at = 262144
    src = torch.tensor([0], dtype=torch.int32, device="cuda")
    dst = torch.tensor([1], dtype=torch.int32, device="cuda")
    f = tf.snapshot_copy(plan, view, view, src, dst, at, prepare=True)
    f()
    torch.cuda.synchronize()
    sreps = 10
    # cold (the figure): 1 GiB written before each copy, outside its events, so that no
    # source line is in the 256 MB Infinity Cache and that cache is full of dirty lines
    flush = torch.empty(1 << 28, dtype=torch.float32, device="cuda")
    cold = []
    for i in range(sreps):
        flush.fill_(float(i))
        e0, e1 = TimingEvent(), TimingEvent()
        e0.record()
        f()
        e1.record()
        torch.cuda.synchronize()
        cold.append(e0.elapsed_time(e1) * 1e3)
    del flush
    # hot: back to back, the source largely in the Infinity Cache from the copy before
    se = [TimingEvent() for _ in range(sreps + 1)]
    se[0].record()
    for i in range(sreps):
        f()
        se[i + 1].record()
    torch.cuda.synchronize()
    snap_hot_us = _mean([se[i].elapsed_time(se[i + 1]) * 1e3 for i in range(sreps)])
    snap_us = _median(cold)
    snap_bytes = at * (plan.lat_row_bytes + 4 + plan.rope_row_bytes) + (at // 4) * plan.pkey_row_bytes
    res = {"workload": wl.name, "tokens": N, "chunks": len(sched), "total_us": round(total_us, 1),
           "tok_per_s": round(N / (total_us * 1e-6), 1), "calls_total_us": calls_total,
           "bands_by_chunk_size": {str(T): bands[T] for T in sorted(bands, reverse=True)},
           "indexer": {"causal_flop": idx_flop, "us": calls_total["indexer"],
                       "TFLOPs": round(idx_flop / (calls_total["indexer"] * 1e-6) / 1e12, 1),
                       "frac_mfma": round(idx_flop / (calls_total["indexer"] * 1e-6) / 1e12 / MFMA_BF16_PEAK_TFLOPS,
                                          4)},
           "attention": {"flop": att_flop, "us": calls_total["attention"],
                         "TFLOPs": round(att_flop / (calls_total["attention"] * 1e-6) / 1e12, 1),
                         "frac_mfma": round(att_flop / (calls_total["attention"] * 1e-6) / 1e12
                                            / MFMA_BF16_PEAK_TFLOPS, 4)},
           "snapshot": {"call": "tf_snapshot_copy", "at": at, "bytes_each_way": snap_bytes, "us": round(snap_us, 2),
                        "reps": sreps, "GBps_read_plus_written": round(2 * snap_bytes / (snap_us * 1e-6) / 1e9, 1),
                        "frac_hbm": round(2 * snap_bytes / (snap_us * 1e-6) / 1e9 / HBM_PEAK_GBS, 4),
                        "timing": "median of copies each after 1 GiB written (Infinity Cache cold and dirty)",
                        "us_back_to_back": round(snap_hot_us, 2)},
           "fused_indexer_topk_pass": fused,
           "timing": "an event between every call; inputs generated into HBM before the first chunk"}
    del P, lat, sc, rope, keys, q, iq, w, logbuf, out
    torch.cuda.empty_cache()
    return res


def adaptive_fused_pass(tf, plan, view, wl, sched, chunk_calls, rs, rp, iq, w, nv, blocks):
    """The same 464 chunks with tf_indexer_topk_fused in place of the indexer and top-k
    calls (no logits written): first every 16th chunk's blocks checked equal to the
    pair's, then the whole prompt timed as the pair is (an event between calls)."""
    import torch
    ws = torch.empty(max(256, max(tf.indexer_topk_fused_workspace_bytes(T, (L + T - 1) // 4 + 1, wl.k, wl.H)
                                  for L, T in sched)), dtype=torch.uint8, device="cuda")
    fb = torch.empty_like(blocks)

    def fused(L, T):
        ld = (L + T - 1) // 4 + 1
        return lambda: tf.indexer_topk_fused(plan, view, rs[L:L + T], rp[L:L + T], iq[L:L + T], w[L:L + T], ld,
                                             wl.k, fb[:T], ws=ws)
    checked = 0
    for L, T in sched[::16]:
        c = chunk_calls(L, T)
        c[1]()
        c[2]()
        fused(L, T)()
        torch.cuda.synchronize()
        assert torch.equal(fb[:T], blocks[:T]), f"fused blocks differ at chunk L={L}"
        checked += 1
    ev = [[TimingEvent() for _ in range(4)] for _ in sched]
    for i, (L, T) in enumerate(sched):
        c = chunk_calls(L, T)
        ev[i][0].record()
        for j, f in enumerate((c[0], fused(L, T), c[3])):
            f()
            ev[i][j + 1].record()
    torch.cuda.synchronize()
    call_us = [[ev[i][j].elapsed_time(ev[i][j + 1]) * 1e3 for j in range(3)] for i in range(len(sched))]
    total = ev[0][0].elapsed_time(ev[-1][3]) * 1e3
    n_tok = sum(T for _, T in sched)
    del ws
    return {"total_us": round(total, 1), "tok_per_s": round(n_tok / (total * 1e-6), 1),
            "calls_total_us": {n: round(sum(c[j] for c in call_us), 1)
                               for j, n in enumerate(("write", "indexer_topk_fused", "attention"))},
            "chunks_checked_equal": checked}


def cpu_baseline(wl, rows, ld, scale, seconds, step_bytes):
    """The oracle (fp64 numpy) on the same decode step: logits over every pooled
    key, exact top-k, attention over the selected rows, repeated for about
    `seconds`. Inputs are generated before timing; only the oracle's arithmetic is
    timed."""
    import numpy as np
    from oracle import indexer_logits, sparse_mla, topk_blocks
    from oracle import workload as ow
    from oracle.attention import selected_tokens
    from synth import bf16_to_f64
    threads = _host_threads()
    log("cpu baseline: generating inputs")
    q_i = bf16_to_f64(wl.iq_bits(0, rows))
    w_i = wl.weights(0, rows).astype(np.float64)
    keys = [ow.keys_of(wl, 0, b, t // 4 + 1) for b, t in rows]
    q_a = bf16_to_f64(wl.q_bits(0, rows))
    pos = [t for _, t in rows]
    lg = indexer_logits(q_i, w_i, keys, pos, ld)
    blk = topk_blocks(lg, [min(t // 4 + 1, ld) for t in pos], wl.k)
    cache = {}
    for r, (b, t) in enumerate(rows):                 # the selected rows (generator work, untimed)
        S = selected_tokens(blk[r], t)
        cache[r] = dict(zip(S.tolist(), range(S.size))), ow.rows_reader(wl, 0, b)(S)

    def rows_of(r, S):
        m, (lat, rope) = cache[r]
        ix = [m[s] for s in S.tolist()]
        return lat[ix], rope[ix]

    steps, busy = 0, 0.0
    while busy < seconds:
        t0 = time.perf_counter()
        lg = indexer_logits(q_i, w_i, keys, pos, ld)
        blk = topk_blocks(lg, [min(t // 4 + 1, ld) for t in pos], wl.k)
        sparse_mla(q_a, rows_of, blk, pos, scale)
        busy += time.perf_counter() - t0
        steps += 1
    sec = busy / steps
    return {"value": round(step_bytes / sec / 1e9, 4), "unit": "GB/s", "cores": threads["cores"], "kind": "oracle",
            "sample": f"{steps} whole decode steps of the same workload ({len(rows)} rows: logits over {ld} "
                      f"keys each, exact top-{wl.k}, attention over the selected rows), {busy:.1f} s",
            "seconds_per_step": round(sec, 4), "blas_threads": threads["blas_threads"], "cpu_model": _cpu_model()}


def _host_threads():
    """Host cores this process may run on (its affinity mask), and the threads the BLAS
    behind numpy uses (the oracle's only multi-threaded part)."""
    cores = len(os.sched_getaffinity(0))
    try:
        from threadpoolctl import threadpool_info
        blas = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:
        blas = None
    return {"cores": cores, "blas_threads": blas}


def _cpu_model():
    """The host CPU's model name, with its family / model / stepping numbers (a model name
    alone can be as short as the vendor's brand)."""
    info = {}
    try:
        for line in open("/proc/cpuinfo"):
            if ":" in line:
                k, v = line.split(":", 1)
                info.setdefault(k.strip(), v.strip())
    except Exception:
        return None
    name = info.get("model name")
    ids = [f"{k} {info[k]}" for k in ("cpu family", "model", "stepping") if k in info]
    return f"{name} ({', '.join(ids)})" if name else None


def cpu_baseline_prefill(pw, seconds, gpu_step_us):
    """The oracle (fp64 numpy) on rows of the prefill chunk: logits over every visible key,
    exact top-k, attention over the selected rows, one sampled row at a time for about
    `seconds`; the chunk's time is extrapolated from the per-row rate (labelled so)."""
    import numpy as np
    from oracle import indexer_logits, sparse_mla, topk_blocks
    from oracle import workload as ow
    from synth import bf16_to_f64
    threads = _host_threads()
    log("cpu baseline (prefill chunk): generating inputs")
    rng = np.random.default_rng(5)
    order = rng.permutation(len(pw.rows))
    ld = pw.rows[-1][1] // 4 + 1
    keys = ow.keys_of(pw, 0, 0, ld)
    reader = ow.rows_reader(pw, 0, 0)
    scale = 1.0 / math.sqrt(576.0)
    n, busy = 0, 0.0
    while busy < seconds and n < len(order):
        r = int(order[n])
        row = [pw.rows[r]]
        q_i = bf16_to_f64(pw.iq_bits(0, row))
        w_i = pw.weights(0, row).astype(np.float64)
        q_a = bf16_to_f64(pw.q_bits(0, row))
        t = row[0][1]
        t0 = time.perf_counter()
        lg = indexer_logits(q_i, w_i, [keys], [t], ld)
        blk = topk_blocks(lg, [min(t // 4 + 1, ld)], pw.k)
        sparse_mla(q_a, lambda _r, S: reader(S), blk, [t], scale)
        busy += time.perf_counter() - t0
        n += 1
    per_row = busy / n
    T = len(pw.rows)
    return {"value": round(1.0 / per_row, 3), "unit": "rows/s", "cores": threads["cores"], "kind": "oracle",
            "sample": f"{n} randomly chosen rows of the {T}-row chunk (logits over up to {ld} keys, exact "
                      f"top-{pw.k}, attention over the selected rows), {busy:.1f} s",
            "chunk_seconds_extrapolated": round(per_row * T, 2), "extrapolated": True,
            "gpu_chunk_us": gpu_step_us, "gpu_over_cpu": round(per_row * T / (gpu_step_us * 1e-6), 1),
            "blas_threads": threads["blas_threads"], "cpu_model": _cpu_model()}


# ---------------------------------------------------------------------- profile summaries
def _matches(name, p):
    """A kernel's short name belongs to a listed kernel name p: the same name, or p with
    template arguments (or a grid tag) appended."""
    n = name[5:] if name.startswith("void ") else name
    return n == p or n.startswith(p + " [") or (n.startswith(p + "<") if "<" not in p else n.startswith(p))


def _entry_of(name):
    for e, (prefixes, _) in ENTRIES.items():
        if any(_matches(name, p) for p in prefixes):
            return e
    return None


def _short(name):
    return name.split("(")[0].replace("void ", "")


def summarize_trace(db, label, command, bench_json=None):
    """Per-kernel durations from a rocprofv3 --kernel-trace database, written to
    profiles/<label>.txt, with the command that produced it; with `bench_json`, the
    HIP-event durations an unprofiled run of the same command measured beside them
    (the tracer itself lengthens the gaps between launches, not the kernels)."""
    c = sqlite3.connect(db)
    stats, grids = {}, {}
    rows = c.execute("select name, start, end, grid_x * grid_y * grid_z from kernels").fetchall()
    for name, _, _, g in rows:
        grids.setdefault(_short(name), set()).add(g)
    for name, start, end, g in rows:   # a kernel launched at several grid sizes gets a line per size
        n = _short(name)
        key = f"{n} [grid {g}]" if len(grids[n]) > 1 else n
        stats.setdefault(key, []).append((end - start) / 1000.0)
    lines = [f"# rocprofv3 kernel trace: {label}", f"# command: {command}", "",
             f"{'kernel':60s} {'calls':>6s} {'avg_us':>10s} {'min_us':>10s} {'max_us':>10s} {'total_us':>12s}"]
    per_entry = {}
    for n, v in sorted(stats.items(), key=lambda kv: -sum(kv[1])):
        lines.append(f"{n[:60]:60s} {len(v):6d} {sum(v) / len(v):10.2f} {min(v):10.2f} {max(v):10.2f} "
                     f"{sum(v):12.1f}")
        # entries may name a kernel with its grid: match on the name tagged with its grid
        # even where it was launched at one size only (and so printed without the tag)
        e = _entry_of(n if " [grid" in n else f"{n} [grid {next(iter(grids[n]))}]")
        if e is not None:
            per_entry.setdefault(e, []).append((n, len(v), sum(v) / len(v)))
    # an entry's kernel launched at several sizes: keep the size launched most often (the timed one)
    for e, ks in per_entry.items():
        best = {}
        for n, cnt, a in ks:
            base = n.split(" [grid")[0]
            if base not in best or cnt > best[base][1]:
                best[base] = (n, cnt, a)
        per_entry[e] = list(best.values())
    lines += ["", "# per entry point: sum of its kernels' average durations (one launch each per call)"]
    for e, ks in per_entry.items():
        lines.append(f"{e:16s} {sum(a for _, _, a in ks):10.2f} us  <- " + " + ".join(
            f"{n} ({a:.2f})" for n, _, a in ks))
    if bench_json:
        b = json.loads([ln for ln in open(bench_json) if ln.startswith("{")][-1])
        lines += ["", "# HIP events in an unprofiled run of the same command vs the kernels' own durations above"
                      " (decode calls: differences of intervals from the step's start, so no event's own dispatch"
                      " is counted; the prefill and dense calls: event to event, one dispatch included)"]
        ev = {n: d["us"] for n, d in b["kernels"].items()}
        if b.get("prefill_indexer"):
            ev["indexer_prefill"] = b["prefill_indexer"]["us"]
        for call, e in (("topk", "topk_prefill"), ("attention", "attention_prefill")):
            if b.get("prefill_step"):
                ev[e] = b["prefill_step"]["calls"][call]["us"]
        if b.get("dense_pass"):
            ev["attention_dense"] = b["dense_pass"]["us"]
        if b.get("prefill_step", {}).get("fused_indexer_topk"):
            ev["indexer_topk_fused"] = b["prefill_step"]["fused_indexer_topk"]["us"]
        for e, us in ev.items():
            k = sum(a for _, _, a in per_entry.get(e, []))
            lines.append(f"{e:16s} events {us:9.2f} us   kernels {k:9.2f} us   ratio {us / k if k else 0:.3f}")
        lines.append(f"dominant call: {b['roofline']['kernel']}  achieved {b['roofline']['achieved']} GB/s "
                     f"= {b['roofline']['alg_bytes_per_launch']} B / {b['roofline']['avg_launch_us']} us")
    os.makedirs(PROFILES, exist_ok=True)
    path = os.path.join(PROFILES, f"{label}.txt")
    open(path, "w").write("\n".join(lines) + "\n")
    print("\n".join(lines))


SIMDS = 256 * 4   # MI355X: 256 CUs of 4 SIMDs


def summarize_counters(db, label, command, prefixes):
    """Per-dispatch values of every counter a rocprofv3 --pmc pass collected, for the
    kernels whose names start with one of `prefixes` (grouped by kernel and grid size;
    averaged over dispatches), written to profiles/<label>.txt with the command that
    produced them. A counter comes as one value per hardware instance (shader engine,
    XCD); a dispatch's value is the sum over instances, except GRBM_GUI_ACTIVE, whose
    maximum is the dispatch's active cycles. Where the pass holds
    SQ_VALU_MFMA_BUSY_CYCLES, MFMA utilisation is reported as rocprofv3's MfmaUtil
    defines it: MFMA-busy cycles over all SIMDs / (active cycles x SIMDs)."""
    c = sqlite3.connect(db)
    per = {}
    for name, g, did, cn, v in c.execute("select p.name, k.grid_x * k.grid_y * k.grid_z, p.dispatch_id, p.counter_name, "
                                         "p.counter_value from pmc_events p join kernels k "
                                         "on p.dispatch_id = k.dispatch_id"):
        n = _short(name)
        if not any(n.startswith(x) or n.startswith("void " + x) for x in prefixes if x):
            continue
        d = per.setdefault((n, g), {}).setdefault(did, {})
        if cn == "GRBM_GUI_ACTIVE":
            d[cn] = max(d.get(cn, 0.0), float(v))
        else:
            d[cn] = d.get(cn, 0.0) + float(v)
    lines = [f"# rocprofv3 counters: {label}", f"# command: {command}", "",
             "# per dispatch: counters summed over hardware instances (GRBM_GUI_ACTIVE: their maximum), "
             "averaged over dispatches"]
    for (n, g), ds in sorted(per.items()):
        names = sorted({cn for d in ds.values() for cn in d})
        lines.append(f"{n} [grid {g}]  ({len(ds)} dispatches)")
        avg = {cn: sum(d.get(cn, 0.0) for d in ds.values()) / len(ds) for cn in names}
        for cn in names:
            lines.append(f"  {cn:36s} {avg[cn]:20.1f}")
        if "SQ_VALU_MFMA_BUSY_CYCLES" in avg and avg.get("GRBM_GUI_ACTIVE"):
            util = 100.0 * avg["SQ_VALU_MFMA_BUSY_CYCLES"] / (avg["GRBM_GUI_ACTIVE"] * SIMDS)
            lines.append(f"  {'MFMA utilisation (MfmaUtil)':36s} {util:19.1f}%")
        if "SQ_INSTS_VALU_MFMA_MOPS_BF16" in avg:
            lines.append(f"  {'bf16 MFMA flop (MOPS x 512)':36s} {avg['SQ_INSTS_VALU_MFMA_MOPS_BF16'] * 512:20.4g}")
    os.makedirs(PROFILES, exist_ok=True)
    open(os.path.join(PROFILES, f"{label}.txt"), "w").write("\n".join(lines) + "\n")
    print("\n".join(lines))


def _pmc(db, counter):
    """(kernel, grid size) -> counter values per dispatch."""
    c = sqlite3.connect(db)
    by = {}
    for name, g, v in c.execute("select p.name, k.grid_x * k.grid_y * k.grid_z, p.counter_value from pmc_events p "
                                "join kernels k on p.dispatch_id = k.dispatch_id where p.counter_name = ?",
                                (counter,)):
        by.setdefault((_short(name), g), []).append(float(v))
    return by


def _pick(by, pattern):
    """The (kernel, grid) of a listed kernel name: the grid it pins (" [grid N]"), else the
    grid launched most often."""
    base, _, g = pattern.partition(" [grid ")
    cands = [kg for kg in by if _matches(kg[0], base) and (not g or kg[1] == int(g.rstrip("]")))]
    return max(cands, key=lambda kg: len(by[kg])) if cands else None


def summarize_pmc(fetch_db, write_db, command, traffic_file=TRAFFIC_FILE):
    """HBM bytes per launch of each entry point from one FETCH_SIZE and one WRITE_SIZE
    pass (KiB per dispatch), each scaled by what the same counter reads for the
    calibration stream (CAL_BYTES read and CAL_BYTES written by one torch.neg)."""
    fetch, write = _pmc(fetch_db, "FETCH_SIZE"), _pmc(write_db, "WRITE_SIZE")
    cal = [kg for kg in fetch if CAL_KERNEL in kg[0]]
    if cal:
        cf = CAL_BYTES / (fetch[cal[0]][0] * 1024.0)
        cw = CAL_BYTES / (write[[kg for kg in write if CAL_KERNEL in kg[0]][0]][0] * 1024.0)
        calib = {"kernel": cal[0][0], "bytes_read": CAL_BYTES, "bytes_written": CAL_BYTES}
    else:   # a pass over a leg without the stream: the scales of the decode pass's file
        assert traffic_file != TRAFFIC_FILE, "the calibration kernel is missing from the FETCH_SIZE pass"
        prev = json.load(open(os.path.join(PROFILES, TRAFFIC_FILE)))["calibration"]
        cf, cw = prev["fetch_scale"], prev["write_scale"]
        calib = {"from": TRAFFIC_FILE, "kernel": prev["kernel"], "bytes_read": CAL_BYTES, "bytes_written": CAL_BYTES}
    entries = {}
    for e, (patterns, src) in ENTRIES.items():
        for p in patterns:
            kg = _pick(fetch, p)
            if kg is None:
                continue
            f_kib = sum(fetch[kg]) / len(fetch[kg])
            w = write.get(kg, [0.0])
            w_kib = sum(w) / max(1, len(w))
            d = entries.setdefault(e, {"kernels": {}, "source_sha256_16": source_hash(src)})
            d["kernels"][f"{kg[0]} [grid {kg[1]}]"] = {"fetch_kib": round(f_kib, 1), "write_kib": round(w_kib, 1),
                                                       "dispatches": len(fetch[kg])}
    for e, d in entries.items():
        fb = sum(k["fetch_kib"] for k in d["kernels"].values()) * 1024.0 * cf
        wb = sum(k["write_kib"] for k in d["kernels"].values()) * 1024.0 * cw
        d["fetch_bytes_per_launch"] = round(fb)
        d["write_bytes_per_launch"] = round(wb)
        d["hbm_bytes_per_launch"] = round(fb + wb)
    res = {"command": command, "calibration": dict(calib, fetch_scale=round(cf, 4), write_scale=round(cw, 4)),
           "entries": entries}
    os.makedirs(PROFILES, exist_ok=True)
    path = os.path.join(PROFILES, traffic_file)
    json.dump(res, open(path, "w"), indent=1)
    print(json.dumps(res, indent=1))


if __name__ == "__main__":
    main()
