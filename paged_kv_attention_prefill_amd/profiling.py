"""Summaries of rocprofv3 output for the profiles/ directory.

    python -m paged_kv_attention_prefill_amd.profiling kernels <trace_dir> [--match NAME]
    python -m paged_kv_attention_prefill_amd.profiling counters <pmc_dir> [--match NAME]
    python -m paged_kv_attention_prefill_amd.profiling utilisation <pmc_dir> --match NAME
    python -m paged_kv_attention_prefill_amd.profiling traffic --workload W --kernel K \
        --fetch <pmc_dir> --write <pmc_dir> --copy-fetch <pmc_dir> --copy-write <pmc_dir> \
        --copy-bytes N

``kernels`` prints per-kernel dispatch counts and durations from a
``--kernel-trace`` run (CSV output, ``-f csv``); ``counters`` prints per-kernel
averages of the counters of a ``--pmc`` run; ``utilisation`` prints, for one
kernel of a ``--pmc`` run that collected rocprofv3's derived ``MfmaUtil`` and
``VALUBusy`` with ``GRBM_GUI_ACTIVE``, the matrix-core and vector-ALU busy
fractions and the shader clock (GUI-active cycles over the dispatch's
duration); ``traffic`` turns FETCH_SIZE and
WRITE_SIZE (KiB per dispatch) into HBM bytes per launch, each scaled by what the
same counter reads for a plain copy kernel of known size, and records them in
profiles/traffic.json together with a hash of the sources that build that
kernel (the bench reports the record only while they are unchanged).
"""
from __future__ import annotations

import argparse
import csv
import glob
import hashlib
import json
import os
import statistics
import sys
from collections import defaultdict

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
TRAFFIC_JSON = os.path.join(ROOT, "profiles", "traffic.json")


# the source file that holds each kernel family (matched by name prefix)
KERNEL_SOURCES = (("gqa_decode", "gqa_decode.hip"), ("flash_attn", "flash_attn.hip"),
                  ("mla_", "mla_decode.hip"), ("generic", "generic.hip"),
                  ("chunk_merge", "merge.hip"), ("merge", "merge.hip"))


def _with_includes(name: str, seen: set) -> None:
    """`name` and, transitively, the local headers it includes."""
    if name in seen:
        return
    seen.add(name)
    with open(os.path.join(PKG, "csrc", name)) as f:
        for line in f:
            line = line.strip()
            if line.startswith('#include "'):
                inc = line.split('"')[1]
                if os.path.exists(os.path.join(PKG, "csrc", inc)):
                    _with_includes(inc, seen)


def kernel_sources(kernel: str = "") -> list:
    """The csrc files that build `kernel`: its own file, the headers it includes,
    and api.cpp (the host plan that sets its grid, split and workspace).  With no
    kernel name, or one of no known family: every source."""
    for prefix, src in KERNEL_SOURCES:
        if kernel.startswith(prefix):
            seen: set = set()
            _with_includes(src, seen)
            _with_includes("api.cpp", seen)
            return sorted(seen)
    seen = set()
    for path in glob.glob(os.path.join(PKG, "csrc", "*")):
        _with_includes(os.path.basename(path), seen)
    return sorted(seen)


def kernel_source_hash(kernel: str = "") -> str:
    """sha256 over kernel_sources(kernel)."""
    h = hashlib.sha256()
    for name in kernel_sources(kernel):
        with open(os.path.join(PKG, "csrc", name), "rb") as f:
            h.update(name.encode())
            h.update(f.read())
    return h.hexdigest()[:16]


def _csv(dirname: str, suffix: str):
    files = sorted(glob.glob(os.path.join(dirname, "**", f"*{suffix}"), recursive=True))
    if not files:
        raise SystemExit(f"no *{suffix} under {dirname}")
    rows = []
    for fn in files:
        with open(fn, newline="") as f:
            rows.extend(csv.DictReader(f))
    return rows


def short(name: str) -> str:
    name = name.replace("(anonymous namespace)::", "")
    return name if len(name) < 110 else name[:107] + "..."


def kernel_stats(trace_dir: str, match: str = ""):
    rows = _csv(trace_dir, "kernel_trace.csv")
    agg = defaultdict(list)
    for r in rows:
        n = r.get("Kernel_Name", "")
        if match and match not in n:
            continue
        agg[n].append((int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3)
    out = []
    for n, ds in sorted(agg.items(), key=lambda kv: -sum(kv[1])):
        out.append(dict(kernel=short(n), calls=len(ds), avg_us=statistics.mean(ds),
                        median_us=statistics.median(ds), min_us=min(ds), max_us=max(ds),
                        total_us=sum(ds)))
    return out


def counter_stats(pmc_dir: str, match: str = ""):
    rows = _csv(pmc_dir, "counter_collection.csv")
    agg = defaultdict(lambda: defaultdict(list))
    for r in rows:
        n = r.get("Kernel_Name", "")
        if match and match not in n:
            continue
        agg[n][r["Counter_Name"]].append(float(r["Counter_Value"]))
    out = []
    for n, ctrs in agg.items():
        out.append(dict(kernel=short(n), dispatches=max(len(v) for v in ctrs.values()),
                        **{k: statistics.mean(v) for k, v in ctrs.items()}))
    return out


def utilisation(pmc_dir: str, match: str):
    """Matrix-core and VALU busy percentages and the shader clock of one kernel.

    Per dispatch: MfmaUtil and VALUBusy as rocprofv3 derives them (busy cycles
    over GUI-active cycles times the SIMD or CU count), and GRBM_GUI_ACTIVE
    divided by the dispatch's own start-to-end time.  Averages over dispatches.
    The CSV value of GRBM_GUI_ACTIVE is summed over the XCDs (one GRBM count per
    XCD), so the clock divides it by the GPU agent's Num_Xcc.
    """
    num_xcc = 1
    for r in _csv(pmc_dir, "agent_info.csv"):
        if r.get("Agent_Type") == "GPU":
            num_xcc = max(1, int(r["Num_Xcc"]))
    rows = [r for r in _csv(pmc_dir, "counter_collection.csv") if match in r.get("Kernel_Name", "")]
    if not rows:
        raise SystemExit(f"no dispatch of {match} in {pmc_dir}")
    per = defaultdict(dict)
    for r in rows:
        d = per[r["Dispatch_Id"]]
        d[r["Counter_Name"]] = float(r["Counter_Value"])
        d["us"] = (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3
        d["kernel"] = r["Kernel_Name"]
    out = dict(kernel=short(next(iter(per.values()))["kernel"]), dispatches=len(per),
               avg_us=statistics.mean(d["us"] for d in per.values()))
    for c in ("MfmaUtil", "VALUBusy", "LDSBankConflict"):
        vals = [d[c] for d in per.values() if c in d]
        if vals:
            out[c] = statistics.mean(vals)
    clk = [d["GRBM_GUI_ACTIVE"] / num_xcc / (d["us"] * 1e3) for d in per.values()
           if "GRBM_GUI_ACTIVE" in d]
    if clk:
        out["clock_ghz"] = statistics.mean(clk)
    for c in ("SQ_INSTS_MFMA", "SQ_INSTS_VALU", "SQ_INSTS_LDS"):
        vals = [d[c] for d in per.values() if c in d]
        if vals:
            out[c] = statistics.mean(vals)
    return out


def _one(stats, counter):
    vals = [s[counter] for s in stats if counter in s]
    if not vals:
        raise SystemExit(f"counter {counter} not found")
    return max(vals)


def main(argv=None):
    ap = argparse.ArgumentParser()
    sub = ap.add_subparsers(dest="cmd", required=True)
    k = sub.add_parser("kernels")
    k.add_argument("dir")
    k.add_argument("--match", default="")
    c = sub.add_parser("counters")
    c.add_argument("dir")
    c.add_argument("--match", default="")
    u = sub.add_parser("utilisation")
    u.add_argument("dir")
    u.add_argument("--match", required=True)
    t = sub.add_parser("traffic")
    for a in ("--workload", "--kernel", "--fetch", "--write", "--copy-fetch", "--copy-write"):
        t.add_argument(a, required=True)
    t.add_argument("--copy-bytes", type=int, required=True)
    t.add_argument("--algorithmic-bytes", type=int, default=0)
    a = ap.parse_args(argv)
    if a.cmd == "kernels":
        print("| kernel | calls | avg us | median us | min us | max us |")
        print("|---|---|---|---|---|---|")
        for s in kernel_stats(a.dir, a.match):
            print(f"| {s['kernel']} | {s['calls']} | {s['avg_us']:.2f} | {s['median_us']:.2f} | "
                  f"{s['min_us']:.2f} | {s['max_us']:.2f} |")
        return 0
    if a.cmd == "counters":
        for s in counter_stats(a.dir, a.match):
            print(json.dumps(s))
        return 0
    if a.cmd == "utilisation":
        print(json.dumps(utilisation(a.dir, a.match)))
        return 0
    fetch = _one(counter_stats(a.fetch, a.kernel), "FETCH_SIZE")
    write = _one(counter_stats(a.write, a.kernel), "WRITE_SIZE")
    cf = _one(counter_stats(a.copy_fetch, "neg_kernel"), "FETCH_SIZE")
    cw = _one(counter_stats(a.copy_write, "neg_kernel"), "WRITE_SIZE")
    f_scale = a.copy_bytes / (cf * 1024.0)
    w_scale = a.copy_bytes / (cw * 1024.0)
    rec = dict(workload=a.workload, kernel=a.kernel, source_hash=kernel_source_hash(a.kernel),
               fetch_kib=fetch, write_kib=write, copy_fetch_kib=cf, copy_write_kib=cw,
               copy_bytes=a.copy_bytes, fetch_scale=f_scale, write_scale=w_scale,
               fetch_bytes=fetch * 1024.0 * f_scale, write_bytes=write * 1024.0 * w_scale)
    rec["traffic_bytes"] = rec["fetch_bytes"] + rec["write_bytes"]
    if a.algorithmic_bytes:
        rec["algorithmic_bytes"] = a.algorithmic_bytes
        rec["traffic_over_algorithmic"] = rec["traffic_bytes"] / a.algorithmic_bytes
    data = {}
    if os.path.exists(TRAFFIC_JSON):
        data = json.load(open(TRAFFIC_JSON))
    data[a.workload] = rec
    os.makedirs(os.path.dirname(TRAFFIC_JSON), exist_ok=True)
    with open(TRAFFIC_JSON, "w") as f:
        json.dump(data, f, indent=1, sort_keys=True)
    print(json.dumps(rec, indent=1))
    return 0


if __name__ == "__main__":
    sys.exit(main())
