#!/usr/bin/env python3
"""rocprofv3 summaries of the stage-1 and merge kernels, per workload (the files in profiles/).

Two steps:
  python3 profile_stage1.py run c2 c4 ...        (on the GPU machine)
      For each workload, as child processes: one rocprofv3 --kernel-trace --stats run of
      bench.py (100 timed steps after 100 warm-up steps, 100 graph replays), then three
      rocprofv3 --pmc runs of 2 steps each, every counter pass in a run of its own:
      FETCH_SIZE, WRITE_SIZE (both with one 256 MiB device copy as a known-size
      reference), and SQ_VALU_MFMA_BUSY_CYCLES SQ_INSTS_MFMA SQ_WAVES GRBM_GUI_ACTIVE.
      Raw output goes to gpurun_out/prof/, with the SHA-256 of the kernel sources the run used.
  python3 profile_stage1.py summarize c2 c4 ...  (anywhere)
      Reads gpurun_out/prof/ and writes profiles/<kernel>_<workload>_kernel_trace.txt and
      profiles/<kernel>_<workload>_hbm_traffic.txt (the traffic file carries the digest that
      bench.py compares before it reports roofline.traffic).

The cache operations (bench.py --op kv_append / kv_quantize) the same way, named op:workload:
  python3 profile_stage1.py run-ops kv_append:c4 kv_quantize:c2 ...      (GPU machine)
  python3 profile_stage1.py summarize-ops kv_append:c4 kv_quantize:c2 ...
      writes profiles/<kernel>_<op>_<workload>_kernel_trace.txt and _hbm_traffic.txt (an
      op's time and traffic are the sums over the library kernels it launches per step).

This script itself never touches the GPU: rocprofv3 starts bench.py as its own child.
"""
from __future__ import annotations

import csv
import glob
import json
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)
PROF = os.path.join(ROOT, "gpurun_out", "prof")
PMC_PASSES = {"FETCH_SIZE": ["FETCH_SIZE"], "WRITE_SIZE": ["WRITE_SIZE"],
              "MFMA": ["SQ_VALU_MFMA_BUSY_CYCLES", "SQ_INSTS_MFMA", "SQ_WAVES", "GRBM_GUI_ACTIVE"]}
BENCH_TRACE_ARGS = ["--steps", "100", "--warmup", "100", "--graph-reps", "100", "--no-cpu-baseline",
                    "--no-per-config"]
BENCH_PMC_ARGS = ["--steps", "2", "--warmup", "1", "--graph-reps", "0", "--no-cpu-baseline", "--no-per-config"]
CACHE_TRACE_ARGS = ["--steps", "50", "--warmup", "20", "--no-cpu-baseline"]
CACHE_PMC_ARGS = ["--steps", "2", "--warmup", "1", "--no-cpu-baseline", "--calibrate-copy"]


def _kernel_of(cfg: str):
    import bench
    from paged_split_kv_stage1_amd.inputs import CONFIGS
    rope = CONFIGS[cfg].get("dv", CONFIGS[cfg]["d"]) != CONFIGS[cfg]["d"]
    return bench.stage1_kernel_of(bool(CONFIGS[cfg].get("latent", False)), rope)


def _run(cmd, log, timeout):
    print("+", " ".join(cmd), flush=True)
    with open(log, "w") as f:
        r = subprocess.run(cmd, stdout=f, stderr=subprocess.STDOUT, timeout=timeout, cwd="/tmp",
                           env=dict(os.environ, TMPDIR="/tmp"))
    if r.returncode != 0:
        print(open(log).read()[-3000:], flush=True)
        raise SystemExit(f"{cmd[0]} exited with {r.returncode}")


def _trim(d, keep):
    """Keep only the rows of the kernels the summary reads (the flush and set-up kernels
    of a run add megabytes of counter rows), and drop the per-dispatch kernel trace
    (the summary reads the per-kernel statistics)."""
    for f in glob.glob(os.path.join(d, "**", "run_counter_collection.csv"), recursive=True):
        with open(f, newline="") as fh:
            rows = list(csv.reader(fh))
        col = rows[0].index("Kernel_Name")
        kept = [rows[0]] + [r for r in rows[1:] if any(k in r[col] for k in keep)]
        with open(f, "w", newline="") as fh:
            csv.writer(fh).writerows(kept)
    for f in glob.glob(os.path.join(d, "**", "run_kernel_trace.csv"), recursive=True):
        os.remove(f)


def run(configs):
    import bench
    os.makedirs(PROF, exist_ok=True)
    py = sys.executable
    bench_py = os.path.join(ROOT, "bench.py")
    for cfg in configs:
        kernel, sources = _kernel_of(cfg)
        json.dump({"workload": cfg, "kernel": kernel, "kernel_source_sha256": bench.source_digest(sources)},
                  open(os.path.join(PROF, f"meta_{cfg}.json"), "w"))
        d = os.path.join(PROF, f"trace_{cfg}")
        _run(["rocprofv3", "--kernel-trace", "--stats", "-d", d, "-o", "run", "--output-format", "csv", "--",
              py, bench_py, "--config", cfg] + BENCH_TRACE_ARGS, d + ".log", 600)
        _trim(d, (kernel, "merge_kernel", "copyBuffer"))
        for tag, counters in PMC_PASSES.items():
            d = os.path.join(PROF, f"pmc_{tag}_{cfg}")
            extra = ["--calibrate-copy"] if tag in ("FETCH_SIZE", "WRITE_SIZE") else []
            _run(["timeout", "-s", "KILL", "200", "rocprofv3", "--pmc"] + counters +
                 ["-d", d, "-o", "run", "--output-format", "csv", "--", py, bench_py, "--config", cfg] +
                 BENCH_PMC_ARGS + extra, d + ".log", 260)
            _trim(d, (kernel, "merge_kernel", "copyBuffer"))
        print(f"profiled {cfg}", flush=True)


def _one(pattern):
    f = glob.glob(pattern, recursive=True)
    if len(f) != 1:
        raise SystemExit(f"expected one file for {pattern}, found {f}")
    return f[0]


def _bench_json(log):
    for line in reversed(open(log).read().splitlines()):
        if line.startswith("{"):
            return json.loads(line)
    raise SystemExit(f"no bench line in {log}")


def _counters(cfg, tag):
    out = {}
    for r in csv.DictReader(open(_one(f"{PROF}/pmc_{tag}_{cfg}/**/run_counter_collection.csv"))):
        k = (int(r["Dispatch_Id"]), r["Kernel_Name"])
        out.setdefault(k, {})
        out[k][r["Counter_Name"]] = out[k].get(r["Counter_Name"], 0.0) + float(r["Counter_Value"])
    return [(k[1], v) for k, v in sorted(out.items())]


def summarize(configs):
    import bench
    repo = "$REPO"
    for cfg in configs:
        meta = json.load(open(os.path.join(PROF, f"meta_{cfg}.json")))
        kernel = meta["kernel"]
        stats = list(csv.DictReader(open(_one(f"{PROF}/trace_{cfg}/**/run_kernel_stats.csv"))))
        bj = _bench_json(os.path.join(PROF, f"trace_{cfg}.log"))
        trace_cmd = (f"cd /tmp && export TMPDIR=/tmp && rocprofv3 --kernel-trace --stats -d "
                     f"{repo}/gpurun_out/prof/trace_{cfg} -o run --output-format csv -- python3 {repo}/bench.py "
                     f"--config {cfg} " + " ".join(BENCH_TRACE_ARGS))
        lines = [f"# {kernel} + merge_kernel, workload {cfg}: {bench.WORKLOAD_NAMES[cfg]}",
                 f"command: {trace_cmd}",
                 f"written by: python3 profile_stage1.py run {cfg} (GPU machine), then "
                 f"python3 profile_stage1.py summarize {cfg}",
                 "counters: the same bench arguments with " + " ".join(BENCH_PMC_ARGS) +
                 " under rocprofv3 --pmc " + " ".join(PMC_PASSES["MFMA"]),
                 f"kernel sources: SHA-256 {meta['kernel_source_sha256']} (comment-free text, as bench.py computes it)",
                 "", f"{'kernel':<72} {'calls':>6} {'avg_ns':>10} {'min_ns':>8} {'max_ns':>8}"]
        s1 = mg = None
        for r in sorted(stats, key=lambda r: -float(r["TotalDurationNs"])):
            name = r["Name"] if len(r["Name"]) <= 72 else r["Name"][:69] + "..."
            lines.append(f"{name:<72} {int(r['Calls']):>6} {float(r['AverageNs']):>10.0f} "
                         f"{float(r['MinNs']):>8.0f} {float(r['MaxNs']):>8.0f}")
            if kernel in r["Name"] and s1 is None:
                s1 = float(r["AverageNs"]) / 1e3
            if "merge_kernel" in r["Name"]:
                mg = float(r["AverageNs"]) / 1e3
        mg = mg or 0.0
        ab, af = bj["algorithmic_bytes_per_step"], bj["algorithmic_flops_per_step"]
        tot = s1 + mg
        g = bj.get("graph_replay") or {}
        lines += ["", f"work items {bj['config']['work_items']}, max splits {bj['config']['max_splits']}",
                  f"stage1 avg {s1:.1f} us + merge avg {mg:.1f} us = {tot:.1f} us per step (kernel trace)",
                  f"HIP events in the same run: stage1 {bj['stage1_us']:.1f} us, merge {bj['merge_us']:.1f} us; "
                  f"hipGraph replay of both: mean {g.get('us_per_step_mean', 0):.3f} us, IQM "
                  f"{g.get('us_per_step_iqm', 0):.3f} us over {g.get('reps', 0)} reps",
                  f"algorithmic bytes per step {ab} -> {ab / tot / 1e3:.1f} GB/s = {ab / tot / 1e3 / 80:.1f}% of "
                  f"8 TB/s (stage1 alone {ab / s1 / 1e3:.1f} GB/s)",
                  f"algorithmic flops per step {af} -> {af / tot / 1e6:.1f} TFLOP/s"]
        s1c = [v for k, v in _counters(cfg, "MFMA") if kernel in k]
        v = s1c[-1]
        util = v["SQ_VALU_MFMA_BUSY_CYCLES"] / (v["GRBM_GUI_ACTIVE"] / 8 * 1024)
        lines.append(f"MFMA utilisation ({kernel}) = SQ_VALU_MFMA_BUSY_CYCLES / (GRBM_GUI_ACTIVE/8 x 1024 SIMDs) = "
                     f"{100 * util:.1f}%  ({int(v['SQ_INSTS_MFMA'])} MFMA instructions); effective clock "
                     f"{v['GRBM_GUI_ACTIVE'] / 8 / (s1 * 1e3):.2f} GHz")
        open(os.path.join(ROOT, "profiles", f"{kernel}_{cfg}_kernel_trace.txt"), "w").write("\n".join(lines) + "\n")
        fe, wr = _counters(cfg, "FETCH_SIZE"), _counters(cfg, "WRITE_SIZE")

        def calib(c, key, ref_kib=262144.0):
            cp = [v[key] for k, v in c if "copyBuffer" in k]
            if not cp:
                raise SystemExit(f"{cfg}: no calibration copy in the {key} run")
            return cp[0], ref_kib / cp[0]
        fcal, fs = calib(fe, "FETCH_SIZE")
        wcal, ws = calib(wr, "WRITE_SIZE")
        f1 = [v["FETCH_SIZE"] for k, v in fe if kernel in k]
        w1 = [v["WRITE_SIZE"] for k, v in wr if kernel in k]
        fm = [v["FETCH_SIZE"] for k, v in fe if "merge_kernel" in k]
        wm = [v["WRITE_SIZE"] for k, v in wr if "merge_kernel" in k]
        traffic = int((f1[-1] * fs + w1[-1] * ws) * 1024)
        mtraffic = (fm[-1] * fs + wm[-1] * ws) * 1024 if fm else 0.0
        pmc_cmd = (f"cd /tmp && export TMPDIR=/tmp && timeout -s KILL 200 rocprofv3 --pmc FETCH_SIZE -d "
                   f"{repo}/gpurun_out/prof/pmc_FETCH_SIZE_{cfg} -o run --output-format csv -- python3 "
                   f"{repo}/bench.py --config {cfg} " + " ".join(BENCH_PMC_ARGS) + " --calibrate-copy")
        t = [f"# {kernel}, workload {cfg}: HBM traffic from FETCH_SIZE and WRITE_SIZE (two separate rocprofv3 --pmc runs)",
             f"command (fetch): {pmc_cmd}",
             f"command (write): the same with --pmc WRITE_SIZE -d {repo}/gpurun_out/prof/pmc_WRITE_SIZE_{cfg}",
             f"written by: python3 profile_stage1.py run {cfg}, then python3 profile_stage1.py summarize {cfg}", "",
             f"calibration (256 MiB device copy): FETCH_SIZE {fcal:.0f} KiB -> scale {fs:.4f}; "
             f"WRITE_SIZE {wcal:.0f} KiB -> scale {ws:.4f}",
             f"{kernel} per dispatch: FETCH_SIZE {', '.join(f'{x:.0f}' for x in f1)} KiB; "
             f"WRITE_SIZE {', '.join(f'{x:.0f}' for x in w1)} KiB",
             f"scaled stage-1 traffic per launch: {traffic / 1e6:.1f} MB (algorithmic {ab / 1e6:.1f} MB, ratio "
             f"{traffic / ab:.4f}; the excess is the partial O/LSE write of split requests)",
             f"merge_kernel traffic per launch: {mtraffic / 1e6:.1f} MB", "",
             f"workload_name: {cfg}",
             "digest: SHA-256 of the stage-1 kernel sources without comments and blank lines",
             f"kernel_source_sha256: {meta['kernel_source_sha256']}",
             f"traffic_bytes_per_launch: {traffic}"]
        open(os.path.join(ROOT, "profiles", f"{kernel}_{cfg}_hbm_traffic.txt"), "w").write("\n".join(t) + "\n")
        print(f"{cfg}: stage1 {s1:.1f} + merge {mg:.1f} = {tot:.1f} us, {ab / tot / 1e3:.0f} GB/s "
              f"({ab / tot / 1e3 / 80:.1f}%), MFMA {100 * util:.1f}%, traffic/alg {traffic / ab:.3f}")


def _cache_kernel(op: str, cfg: str) -> str:
    """The kernel an op's measurements are filed under (bench.py reports roofline.traffic for it)."""
    from paged_split_kv_stage1_amd.inputs import CONFIGS
    if op == "kv_append":
        return "append_kernel"
    return "quant_rows_kernel" if CONFIGS[cfg]["scale"] == "per_token_head" else "quant_tensor_kernel"


def _op_specs(specs):
    out = []
    for spec in specs:
        op, cfg = spec.split(":")
        if op not in ("kv_append", "kv_quantize"):
            raise SystemExit(f"unknown op {op}")
        out.append((op, cfg))
    return out


def _library_kernel(name: str) -> bool:
    return name.startswith("pa::") or name.startswith("void pa::")


def run_ops(specs):
    import bench
    os.makedirs(PROF, exist_ok=True)
    py = sys.executable
    bench_py = os.path.join(ROOT, "bench.py")
    for op, cfg in _op_specs(specs):
        tag = f"{op}_{cfg}"
        json.dump({"workload": tag, "kernel": _cache_kernel(op, cfg),
                   "kernel_source_sha256": bench.source_digest(bench.CACHE_OP_SOURCES)},
                  open(os.path.join(PROF, f"meta_{tag}.json"), "w"))
        keep = ("pa::", "copyBuffer")
        d = os.path.join(PROF, f"trace_{tag}")
        _run(["rocprofv3", "--kernel-trace", "--stats", "-d", d, "-o", "run", "--output-format", "csv", "--",
              py, bench_py, "--op", op, "--config", cfg] + CACHE_TRACE_ARGS, d + ".log", 600)
        _trim(d, keep)
        for counter in ("FETCH_SIZE", "WRITE_SIZE"):
            d = os.path.join(PROF, f"pmc_{counter}_{tag}")
            _run(["timeout", "-s", "KILL", "200", "rocprofv3", "--pmc", counter, "-d", d, "-o", "run",
                  "--output-format", "csv", "--", py, bench_py, "--op", op, "--config", cfg] + CACHE_PMC_ARGS,
                 d + ".log", 260)
            _trim(d, keep)
        print(f"profiled {tag}", flush=True)


def summarize_ops(specs):
    repo = "$REPO"
    for op, cfg in _op_specs(specs):
        tag = f"{op}_{cfg}"
        meta = json.load(open(os.path.join(PROF, f"meta_{tag}.json")))
        kernel = meta["kernel"]
        stats = [r for r in csv.DictReader(open(_one(f"{PROF}/trace_{tag}/**/run_kernel_stats.csv")))
                 if _library_kernel(r["Name"])]
        if not any(kernel in r["Name"] for r in stats):
            raise SystemExit(f"{tag}: no {kernel} in the kernel statistics")
        bj = _bench_json(os.path.join(PROF, f"trace_{tag}.log"))
        us = sum(float(r["AverageNs"]) for r in stats) / 1e3
        nbytes = bj["algorithmic_bytes_per_step"]
        names = ", ".join(r["Name"].split("(")[0].replace("void ", "") for r in stats)
        trace_cmd = (f"cd /tmp && export TMPDIR=/tmp && rocprofv3 --kernel-trace --stats -d {repo}/gpurun_out/prof/"
                     f"trace_{tag} -o run --output-format csv -- python3 {repo}/bench.py --op {op} --config {cfg} " +
                     " ".join(CACHE_TRACE_ARGS))
        lines = [f"# {op} ({names}), workload: {bj['config']['workload']}",
                 f"command: {trace_cmd}",
                 f"written by: python3 profile_stage1.py run-ops {op}:{cfg} (GPU machine), then "
                 f"python3 profile_stage1.py summarize-ops {op}:{cfg}",
                 f"kernel sources: SHA-256 {meta['kernel_source_sha256']} (comment-free text, as bench.py computes it)",
                 "", f"{'kernel':<72} {'calls':>6} {'avg_ns':>10} {'min_ns':>8} {'max_ns':>8}"]
        for r in sorted(stats, key=lambda r: -float(r["TotalDurationNs"])):
            name = r["Name"] if len(r["Name"]) <= 72 else r["Name"][:69] + "..."
            lines.append(f"{name:<72} {int(r['Calls']):>6} {float(r['AverageNs']):>10.0f} "
                         f"{float(r['MinNs']):>8.0f} {float(r['MaxNs']):>8.0f}")
        lines += ["", f"op avg {us:.1f} us per step (kernel trace, sum over the kernels above); HIP events in the "
                      f"same run {bj['us_per_step']:.1f} us",
                  f"algorithmic bytes per step {nbytes} -> {nbytes / us / 1e3:.1f} GB/s = "
                  f"{nbytes / us / 1e3 / 80:.1f}% of 8 TB/s"]
        open(os.path.join(ROOT, "profiles", f"{kernel}_{tag}_kernel_trace.txt"), "w").write("\n".join(lines) + "\n")
        fe, wr = _counters(tag, "FETCH_SIZE"), _counters(tag, "WRITE_SIZE")
        fc = [v["FETCH_SIZE"] for k, v in fe if "copyBuffer" in k]
        wc = [v["WRITE_SIZE"] for k, v in wr if "copyBuffer" in k]
        if not fc or not wc:
            raise SystemExit(f"{tag}: no calibration copy in the counter runs")
        fs, ws = 262144.0 / fc[0], 262144.0 / wc[0]
        per = []
        traffic = 0.0
        for r in stats:
            base = r["Name"]
            f1 = [v["FETCH_SIZE"] for k, v in fe if k == base]
            w1 = [v["WRITE_SIZE"] for k, v in wr if k == base]
            if f1 and w1:
                traffic += (f1[-1] * fs + w1[-1] * ws) * 1024     # the last step's dispatch of each kernel
                per.append(f"{base.split('(')[0].replace('void ', '')}: FETCH_SIZE "
                           f"{', '.join(f'{x:.0f}' for x in f1)} KiB; WRITE_SIZE {', '.join(f'{x:.0f}' for x in w1)} KiB")
        traffic = int(traffic)
        pmc_cmd = (f"cd /tmp && export TMPDIR=/tmp && timeout -s KILL 200 rocprofv3 --pmc FETCH_SIZE -d "
                   f"{repo}/gpurun_out/prof/pmc_FETCH_SIZE_{tag} -o run --output-format csv -- python3 "
                   f"{repo}/bench.py --op {op} --config {cfg} " + " ".join(CACHE_PMC_ARGS))
        t = [f"# {op} ({names}), workload: {bj['config']['workload']}: HBM traffic from FETCH_SIZE and "
             f"WRITE_SIZE (two separate rocprofv3 --pmc runs)",
             f"command (fetch): {pmc_cmd}",
             f"command (write): the same with --pmc WRITE_SIZE -d {repo}/gpurun_out/prof/pmc_WRITE_SIZE_{tag}",
             f"written by: python3 profile_stage1.py run-ops {op}:{cfg}, then python3 profile_stage1.py "
             f"summarize-ops {op}:{cfg}", "",
             f"calibration (256 MiB device copy): FETCH_SIZE {fc[0]:.0f} KiB -> scale {fs:.4f}; "
             f"WRITE_SIZE {wc[0]:.0f} KiB -> scale {ws:.4f}"] + per + [
             f"scaled traffic per step: {traffic / 1e6:.1f} MB (algorithmic {nbytes / 1e6:.1f} MB, ratio "
             f"{traffic / nbytes:.4f})", "",
             f"workload_name: {tag}",
             "digest: SHA-256 of the quantiser / append kernel sources without comments and blank lines",
             f"kernel_source_sha256: {meta['kernel_source_sha256']}",
             f"traffic_bytes_per_launch: {traffic}"]
        open(os.path.join(ROOT, "profiles", f"{kernel}_{tag}_hbm_traffic.txt"), "w").write("\n".join(t) + "\n")
        print(f"{tag}: {us:.1f} us, {nbytes / us / 1e3:.0f} GB/s, traffic/alg {traffic / nbytes:.3f}")


MODES = {"run": run, "summarize": summarize, "run-ops": run_ops, "summarize-ops": summarize_ops}

if __name__ == "__main__":
    if len(sys.argv) < 3 or sys.argv[1] not in MODES:
        raise SystemExit(__doc__)
    MODES[sys.argv[1]](sys.argv[2:])
