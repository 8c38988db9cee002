#!/usr/bin/env python3
"""Benchmark of the paged-attention hot path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload c2|c3|c5|c4_h16_q1_bf16|c4_h128_q4_fp8q|sparse_mla_h16_bf16|long_decode_b1|...]

Default workload: the Llama-70B-like GQA decode (64 requests, q_len 1, 64 query
/ 8 KV heads, head_dim 128, bf16, page 16, KV lengths uniform in [512, 8192]).
A step is one call of the hot path over the whole batch (every kernel that call
launches).  Inputs are resident in HBM before the timed region; the timed region
is bracketed by torch.cuda.synchronize() on both sides.  Prints one JSON line.

Algorithmic bytes count each needed KV row once per KV head (a shared latent
row once; a broadcast KV batch once), the page ids, Q, O and LSE, and for split
runs the fp32 partial states written and read.  Flops count 2*Dqk + 2*Dvo per
(row, allowed token).
"""
from __future__ import annotations

import argparse
import dataclasses
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_HBM_GBS = 8000.0          # MI355X HBM3E, GB/s
PEAK_BF16_TFLOPS = 2516.6      # dense bf16/fp16 MFMA, TFLOP/s
PEAK_FP8_TFLOPS = 5033.2       # dense fp8 MFMA, TFLOP/s
METRIC = ("decode attn µs/step + achieved HBM GB/s (% peak); "
          "prefill TFLOP/s (% MFMA)")


def make_workload(name: str):
    from paged_kv_attention_prefill_amd import workloads as W
    if name == "c1":
        return W.config1(poison=False)
    if name == "c2":
        return W.config2(poison=False)
    if name == "c3":
        return W.config3(poison=False)
    if name == "c5":
        return W.config5(poison=False)
    if name == "long_decode_b1":
        # one request, 131072 KV tokens: all parallelism comes from splitting the KV
        w = W.config2(batch=1, min_len=131072, max_len=131072, dtype=W.DT_F16, page_size=128,
                      num_qo_heads=32, num_kv_heads=8, poison=False)
        return dataclasses.replace(w, name="long_decode_b1_131072_f16")
    if name.startswith("sparse"):
        # sparse_<mla|gqa>_h<heads>_<bf16|fp8>: top-2048 selected rows per query
        _, kind, h, dt = name.split("_")
        return W.config_sparse(num_heads=int(h[1:]), kv_dtype=W.DT_FP8 if dt == "fp8" else W.DT_BF16,
                               mla=kind == "mla", poison=False)
    if name.startswith("c4"):
        # c4_h<heads>_q<q_len>_<bf16|fp8|fp8q>; fp8q: fp8 queries over the fp8 cache
        _, h, q, dt = name.split("_")
        return W.config4(num_heads=int(h[1:]), q_len=int(q[1:]),
                         kv_dtype=W.DT_FP8 if dt.startswith("fp8") else W.DT_BF16,
                         q_dtype=W.DT_FP8 if dt == "fp8q" else W.DT_BF16, poison=False)
    raise SystemExit(f"unknown workload {name}")


def allowed_tokens(w) -> np.ndarray:
    """|J| per query token (all heads share it)."""
    out = np.empty(w.total_q, dtype=np.int64)
    for b in range(w.batch):
        kb = 0 if w.kv_broadcast else b
        L = int(w.kv_lens[kb])
        t0, t1 = int(w.qo_indptr[b]), int(w.qo_indptr[b + 1])
        qb = t1 - t0
        i = np.arange(qb)
        out[t0:t1] = np.clip(L - qb + i + 1, 0, L) if w.causal else L
    return out


def algorithmic_counts(w, num_states: int = 1):
    """(attention-kernel bytes, merge bytes, flops) of one step."""
    from paged_kv_attention_prefill_amd import workloads as W
    kvb = W.DT_BYTES[w.kv_dtype]
    qb = W.DT_BYTES[w.q_dtype]
    ob = 2 if w.q_dtype != W.DT_F32 else 4
    lens = w.kv_lens[:1] if w.kv_broadcast else w.kv_lens
    row_elems = w.head_dim_qk if w.shared_kv else (w.head_dim_qk + w.head_dim_vo)
    kv_bytes = int(lens.sum()) * w.num_kv_heads * row_elems * kvb
    table = int(w.kv_indptr[-1]) * 4 + (len(w.kv_indptr) + len(w.kv_last_page_len)) * 4
    rows = w.total_q * w.num_qo_heads
    q_bytes = rows * w.head_dim_qk * qb
    flops = int(allowed_tokens(w).sum()) * w.num_qo_heads * 2 * (w.head_dim_qk + w.head_dim_vo)
    if num_states > 1:
        part = num_states * rows * (w.head_dim_vo + 1) * 4
        attn = kv_bytes + table + q_bytes + part
        merge = part + rows * (w.head_dim_vo * ob + 4)
    else:
        attn = kv_bytes + table + q_bytes + rows * (w.head_dim_vo * ob + 4)
        merge = 0
    return attn, merge, flops


def cpu_model() -> str:
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    import platform
    return platform.processor() or "unknown"


def cpu_baseline(w, target_s: float = 15.0, threads: int = 0):
    """Time the oracle on a bounded sample of query batches (whole batches, all heads),
    scaled to the whole workload by the sample's share of (row x allowed token) work.
    threads = 0: every host core (OpenMP default); otherwise that many threads."""
    from oracle import oracle as OR
    work = allowed_tokens(w) * w.num_qo_heads
    per_batch = np.array([work[w.qo_indptr[b]:w.qo_indptr[b + 1]].sum() for b in range(w.batch)],
                         dtype=np.float64)
    order = np.argsort(-per_batch)
    # calibrate on the smallest batch first
    rows_of = lambda b: np.arange(w.qo_indptr[b] * w.num_qo_heads,
                                  w.qo_indptr[b + 1] * w.num_qo_heads, dtype=np.int64)
    t0 = time.perf_counter()
    b_small = int(order[-1])
    OR.attention(w, rows=rows_of(b_small), num_kv_splits=1, num_threads=threads)
    t_small = time.perf_counter() - t0
    rate = per_batch[b_small] / max(t_small, 1e-6)
    budget = rate * target_s
    chosen, acc = [], 0.0
    for b in order[::-1]:  # small to large, so the sample spans several batches
        if acc + per_batch[b] > budget and chosen:
            break
        chosen.append(int(b))
        acc += per_batch[b]
    rows = np.concatenate([rows_of(b) for b in chosen])
    # repeat a sample that finishes quickly so the timing covers ~min(10 s, target)
    reps, elapsed = 0, 0.0
    while reps == 0 or (elapsed < min(10.0, target_s) and reps < 20):
        t0 = time.perf_counter()
        OR.attention(w, rows=rows, num_kv_splits=1, num_threads=threads)
        elapsed += time.perf_counter() - t0
        reps += 1
    frac = acc / per_batch.sum()
    return elapsed / reps / frac, dict(batches=len(chosen), rows=int(rows.size),
                                       seconds=elapsed, reps=reps, fraction=frac,
                                       threads=threads if threads > 0 else OR.num_threads())


COPY_BYTES = 1 << 30  # calibration copy: reads and writes this many bytes per launch
COPY2_BYTES = 1 << 28  # second calibration kernel (a device-to-device copy)


def copy_calibration(steps: int) -> int:
    """Plain streaming kernels of known size for scaling HBM byte counters:
    torch's elementwise negate of a 1 GiB fp32 tensor (1 GiB read, 1 GiB written
    per launch) and a 256 MiB device-to-device tensor copy (the runtime's copy
    kernel: 256 MiB read, 256 MiB written), a second point for the scale."""
    import torch
    src = torch.ones(COPY_BYTES // 4, dtype=torch.float32, device="cuda:0")
    dst = torch.empty_like(src)
    for _ in range(steps):
        torch.neg(src, out=dst)
    src2 = src[: COPY2_BYTES // 4]
    dst2 = torch.empty_like(src2)
    for _ in range(steps):
        dst2.copy_(src2)
    torch.cuda.synchronize()
    print(json.dumps({"copy_calibration_bytes": COPY_BYTES, "copy2_calibration_bytes": COPY2_BYTES,
                      "launches": steps}))
    return 0


def recorded_traffic(workload: str):
    """HBM bytes per launch of the workload's attention kernel from
    profiles/traffic.json if it was measured with the current sources of that
    kernel, else None."""
    from paged_kv_attention_prefill_amd import profiling
    if not os.path.exists(profiling.TRAFFIC_JSON):
        return None
    rec = json.load(open(profiling.TRAFFIC_JSON)).get(workload)
    # the record names the kernel as the profiler does; its hash covers the
    # sources that build that kernel family
    if not rec or rec.get("source_hash") != profiling.kernel_source_hash(rec.get("kernel", "")):
        return None
    return int(rec["traffic_bytes"])


FLUSH_BYTES = 1 << 30  # read before every cold iteration: 4x the 256 MB MALL


def pct(xs):
    a = np.asarray(xs, dtype=np.float64)
    return {"median": round(float(np.median(a)), 2), "p10": round(float(np.percentile(a, 10)), 2),
            "p90": round(float(np.percentile(a, 90)), 2)}


def step_distribution(call, stream, iters: int):
    """Per-step µs over `iters` iterations, warm (back to back) and cold (an untimed
    read of a 1 GiB scratch buffer before every step, so KV, tables and Q come
    from HBM; a read rather than a write, so that no dirty lines of the flush are
    written back during the timed step).  Each step is bracketed by its own
    event pair on the stream it runs on."""
    import torch
    # fp32, so that the sum reads the buffer in place (an int32 sum would first
    # write an int64 copy of it)
    scratch = torch.ones(FLUSH_BYTES // 4, dtype=torch.float32, device="cuda:0")
    out = {}
    for mode in ("warm", "cold"):
        evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
               for _ in range(iters)]
        torch.cuda.synchronize()
        for i, (e0, e1) in enumerate(evs):
            if mode == "cold":
                scratch.sum()
            e0.record(stream)
            call()
            e1.record(stream)
        torch.cuda.synchronize()
        out[mode + "_us"] = pct([e0.elapsed_time(e1) * 1e3 for e0, e1 in evs])
    del scratch
    out["iters"] = iters
    out["flush_bytes"] = FLUSH_BYTES
    return out


# Warm-up of the side workloads: under back-to-back MFMA-heavy launches the
# shader clock takes some 30-40 calls to settle (config 3: ~450 us in the first
# calls, ~520 us a few calls later, ~430 us settled), so the timed steps start
# after that.
SIDE_WARMUP = 40


def side_workload(name: str, steps: int, warmup: int, iters: int):
    """Timing of a second workload in the same run (same protocol as the main one,
    with at least SIDE_WARMUP warm-up steps): step µs, the attention kernel's µs,
    and its rate against its binding roof."""
    import torch
    from paged_kv_attention_prefill_amd import runner as R
    w = make_workload(name)
    d = R.upload(w, "cuda:0")
    stream = torch.cuda.current_stream()
    call = R.prepare(d)
    for _ in range(max(warmup, SIDE_WARMUP)):
        call()
    torch.cuda.synchronize()
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    ev0.record(stream)
    for _ in range(steps):
        call()
    ev1.record(stream)
    torch.cuda.synchronize()
    ms = ev0.elapsed_time(ev1) / steps
    attn_ms = call.time_attention_kernel(steps)
    attn_bytes, merge_bytes, flops = algorithmic_counts(w, call.num_states)
    rec = {"workload": w.name, "kernel": call.attention_kernel_name,
           "us_per_step": round(ms * 1e3, 2), "kernel_us": round(attn_ms * 1e3, 2),
           "tflops": round(flops / (attn_ms * 1e-3) / 1e12, 2),
           "mfma_frac": round(flops / (attn_ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4),
           "hbm_gbs": round(attn_bytes / (attn_ms * 1e-3) / 1e9, 1),
           "hbm_frac": round(attn_bytes / (attn_ms * 1e-3) / 1e9 / PEAK_HBM_GBS, 4),
           "flops_per_launch": flops, "bytes_per_launch": attn_bytes}
    rec["timing"] = step_distribution(call, stream, iters)
    del call, d
    torch.cuda.empty_cache()
    return rec


def mfma_peak(w, kernel_name):
    """(peak TFLOP/s, dtype) of the attention kernel's matrix products: fp8
    queries over an fp8 cache with more than 64 rows per request run both
    products on the fp8 MFMA (P.V as two fp8 products, hi and lo parts of P);
    every other MLA, GQA and prefill kernel multiplies in bf16/fp16."""
    rows = (w.q_len or 0) * (w.num_qo_heads // w.num_kv_heads)
    if kernel_name == "mla_decode_mfma_fp8q" and rows > 64:
        return PEAK_FP8_TFLOPS, "fp8"
    return PEAK_BF16_TFLOPS, "bf16"


def main(argv=None):
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="c2")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=15.0)
    ap.add_argument("--iters", type=int, default=100,
                    help="iterations of the cold/warm per-step distribution")
    ap.add_argument("--no-side", action="store_true",
                    help="skip the prefill (c3) and tiny-decode (c1) side measurements")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="run only the HBM-counter calibration copy kernel")
    a = ap.parse_args(argv)
    if a.gpus != 1:
        print("bench.py measures one GPU only: the library has no multi-GPU path "
              f"(asked for --gpus {a.gpus}); run with --gpus 1", file=sys.stderr)
        return 2

    if a.copy_calibration:
        return copy_calibration(a.steps)

    import torch
    from paged_kv_attention_prefill_amd import binding as B
    from paged_kv_attention_prefill_amd import runner as R

    B.load_library()
    w = make_workload(a.workload)
    d = R.upload(w, "cuda:0")
    stream = torch.cuda.current_stream()
    call = R.prepare(d)

    for _ in range(a.warmup):
        call()
    torch.cuda.synchronize()
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    ev0.record(stream)
    for _ in range(a.steps):
        call()
    ev1.record(stream)
    torch.cuda.synchronize()
    ms = ev0.elapsed_time(ev1) / a.steps

    # the dominant (attention) kernel alone, same launch configuration, timed with
    # events on the stream it is launched on
    attn_ms = call.time_attention_kernel(a.steps)
    states = call.num_states
    attn_bytes, merge_bytes, flops = algorithmic_counts(w, states)
    step_bytes = attn_bytes + merge_bytes
    gbs = step_bytes / (ms * 1e-3) / 1e9
    tflops = flops / (ms * 1e-3) / 1e12
    decode_like = w.q_len is not None
    peak_mfma, mfma_dtype = mfma_peak(w, call.attention_kernel_name)
    bound_hbm = (attn_bytes / PEAK_HBM_GBS) >= (flops / peak_mfma / 1e3)
    if bound_hbm:
        ach = attn_bytes / (attn_ms * 1e-3) / 1e9
        roof = {"bound": "hbm", "achieved": round(ach, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                "frac": round(ach / PEAK_HBM_GBS, 4), "traffic": None}
    else:
        ach = flops / (attn_ms * 1e-3) / 1e12
        roof = {"bound": "mfma", "achieved": round(ach, 1), "peak": peak_mfma,
                "unit": "TFLOP/s", "frac": round(ach / peak_mfma, 4), "traffic": None,
                "mfma_dtype": mfma_dtype}
    roof["traffic"] = recorded_traffic(a.workload)
    roof["kernel"] = call.attention_kernel_name
    roof["kernel_ms"] = round(attn_ms, 5)
    roof["bytes_per_launch"] = attn_bytes
    roof["flops_per_launch"] = flops

    if decode_like:
        value, unit = gbs, "GB/s"
    else:
        value, unit = tflops, "TFLOP/s"
    from paged_kv_attention_prefill_amd import workloads as W
    line = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": unit,
        "n_gpus": 1,
        "steps": a.steps,
        "warmup": a.warmup,
        "ms_per_step": round(ms, 5),
        "us_per_step": round(ms * 1e3, 2),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": W.DT_NAMES[w.kv_dtype],
        "data": "synthetic: seeded N(0,1) values, seeded lengths and shuffled page table",
        "config": {"workload": w.name, **{k: v for k, v in w.manifest().items()
                                          if k not in ("name",)}},
        "achieved_hbm_gbs": round(gbs, 1),
        "hbm_frac": round(gbs / PEAK_HBM_GBS, 4),
        "achieved_tflops": round(tflops, 2),
        "mfma_frac": round(tflops / peak_mfma, 4),
        "roofline": roof,
    }
    line["timing"] = step_distribution(call, stream, a.iters)
    if not a.no_side and a.workload == "c2":
        # the prefill half of the metric (causal GPT-OSS-like prefill) and the
        # launch-latency-bound tiny decode, in the same run
        line["prefill_c3"] = side_workload("c3", max(5, a.steps // 2), a.warmup, a.iters)
        line["tiny_c1"] = side_workload("c1", a.steps, a.warmup, a.iters)
    if not a.no_cpu_baseline:
        full_s, info = cpu_baseline(w, a.cpu_seconds)
        one_s, info1 = cpu_baseline(w, a.cpu_seconds * 2 / 3, threads=1)
        rate = lambda s: (step_bytes / s / 1e9) if decode_like else (flops / s / 1e12)
        line["cpu_baseline"] = {"value": round(rate(full_s), 6), "unit": unit,
                                "cores": info["threads"], "kind": "oracle",
                                "sample": (f"{info['batches']} whole query batches "
                                           f"({info['rows']} rows, {info['fraction']:.3f} of the "
                                           f"work), {info['reps']} run(s) in "
                                           f"{info['seconds']:.1f} s, scaled to the full workload"),
                                "seconds_full_workload": round(full_s, 2),
                                "one_thread": {"value": round(rate(one_s), 6),
                                               "seconds_full_workload": round(one_s, 2),
                                               "sample": (f"{info1['batches']} whole query "
                                                          f"batches, {info1['fraction']:.3f} of "
                                                          f"the work, {info1['reps']} run(s)")},
                                "cpu_model": cpu_model(), "os_cpu_count": os.cpu_count()}
    print(json.dumps(line), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
