#!/usr/bin/env python3
"""Decode-attention benchmark: stage 1 + merge of paged split-KV decode on one MI355X.

Default workload: FP8 single-row decode, batch 128, 64 Q / 8 KV heads, head_dim 128,
KV 2048 tokens per request in pages of 64, Q/K/V e4m3 with per-tensor scales, bf16
output (the hpc-ops issue #4 benchmark shape).  A step is one stage-1 launch plus
one merge launch over the whole batch, with inputs resident in HBM; a 512 MiB write
before every step evicts L2 and the 256 MiB MALL (FreeToken PR #900 times its
kernels with the cache flushed before each rep).  Each step is timed with HIP
events on the stream the kernels run on.

Prints one JSON line.  value = algorithmic HBM bytes per step / time per step (GB/s).
"""
from __future__ import annotations

import argparse
import json
import os
import platform
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "decode-attention µs/step + achieved HBM GB/s (% of MI355X peak), 1 GPU"
HBM_PEAK_GBPS = 8000.0
WORKLOAD_NAMES = {
    "c1": "tiny decode B1 8/1 heads d128 ctx512 P16 bf16, fp32 out, 4 splits",
    "c2": "fp8 single-row decode B128 64/8 heads d128 ctx2048 P64, e4m3 Q/K/V per-tensor, bf16 out",
    "c2_ph": "fp8 single-row decode B128 64/8 heads d128 ctx2048 P64, e4m3 Q/K/V per-head scales, bf16 out",
    "c3": "MTP verify R4 B16 16/2 heads d256 ctx32768 P16 bf16 KV",
    "c3_b1": "MTP verify R4 B1 16/2 heads d256 ctx32768 P16 bf16 KV",
    "c3_r1": "single-row decode B16 16/2 heads d256 ctx32768 P16 bf16 KV",
    "c3_r8": "MTP verify R8 B16 16/2 heads d256 ctx32768 P16 bf16 KV",
    "c3_b1_r1": "single-row decode B1 16/2 heads d256 ctx32768 P16 bf16 KV",
    "c3_b1_r8": "MTP verify R8 B1 16/2 heads d256 ctx32768 P16 bf16 KV",
    "c4": "long-context R8 B16 16/2 heads d256 ctx131072 P16 e4m3 KV per-token-head",
    "c4_i8": "long-context R8 B16 16/2 heads d256 ctx131072 P16 int8 KV per-token-head",
    "c4_i8t": "long-context R8 B16 16/2 heads d256 ctx131072 P16 int8 KV per-tensor",
    "c4_b1": "long-context R8 B1 16/2 heads d256 ctx131072 P16 e4m3 KV per-token-head",
    "c4_r1": "long-context R1 B16 16/2 heads d256 ctx131072 P16 e4m3 KV per-token-head",
    "c4_b1_r1": "long-context R1 B1 16/2 heads d256 ctx131072 P16 e4m3 KV per-token-head",
    "c6": "head_dim 512 verify R8 B1 8/1 heads ctx131072 P16 bf16 KV",
    "c6_r4": "head_dim 512 verify R4 B1 8/1 heads ctx131072 P16 bf16 KV",
    "c6_f8": "head_dim 512 verify R8 B1 8/1 heads ctx131072 P16 e4m3 KV per-token-head",
    "c5": "ragged R1..8 B64 48/2 heads (group 24) d128 ctx loguniform 1K-64K, half window 64, P32 e4m3 per-token-head",
    "f3": "keys 192 / values 128, B32 R1 32/4 heads ctx8192 P16 bf16 KV",
    "f3_r4": "keys 192 / values 128, B32 R4 32/4 heads ctx8192 P16 bf16 KV",
    "mla": "MLA-style latent cache 576/512, B64 R1 16/1 heads ctx4096 P64, e4m3 latent per (token, 128 ch) + bf16 rope",
    "mla_r2": "MLA-style latent cache 576/512, B64 R2 16/1 heads ctx4096 P64, e4m3 latent per (token, 128 ch) + bf16 rope",
}


def _cpu_model() -> str:
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return platform.processor()


KERNEL_SOURCES = ("stage1.hip", "common.hpp", "fair_share.hpp", "row_store.hpp", "kv_addr.hpp", "pa_internal.hpp")
KR_SOURCES = ("stage1_kr.hip", "common.hpp", "fair_share.hpp", "kv_addr.hpp", "pa_internal.hpp")
MLA_SOURCES = ("stage1_mla.hip", "common.hpp", "fair_share.hpp", "row_store.hpp", "kv_addr.hpp", "pa_internal.hpp")


def stage1_kernel_of(latent: bool, rope: bool):
    """(kernel name, its source files) of the stage-1 kernel a workload runs: the latent-cache
    kernel, the rotary-key kernel (keys wider than values) or the equal-width kernel."""
    if latent:
        return "stage1_mla_kernel", MLA_SOURCES
    if rope:
        return "stage1_kr_kernel", KR_SOURCES
    return "stage1_kernel", KERNEL_SOURCES


def kernel_code(text: str) -> str:
    """Source text without comments and blank lines: what the digest of a kernel covers
    (a comment edit does not change the kernel the counters measured)."""
    import re

    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    lines = (re.sub(r"//.*$", "", line).rstrip() for line in text.splitlines())
    return "\n".join(line for line in lines if line.strip())


CACHE_OP_SOURCES = ("quant.hip", "common.hpp", "kv_append.hpp")


def source_digest(files) -> str:
    import hashlib

    h = hashlib.sha256()
    for f in files:
        with open(os.path.join(ROOT, "paged_split_kv_stage1_amd", "csrc", f)) as fh:
            h.update(kernel_code(fh.read()).encode())
    return h.hexdigest()


def measured_traffic(config: str, kernel: str = "stage1_kernel", sources=KERNEL_SOURCES):
    """HBM bytes per launch of ``kernel`` from the committed FETCH_SIZE/WRITE_SIZE summary of
    this workload, or None when there is none or the kernel sources changed since it was taken."""
    import glob

    digest = source_digest(sources)
    for path in glob.glob(os.path.join(ROOT, "profiles", f"{kernel}_{config}*_hbm_traffic.txt")):
        fields = {}
        for line in open(path):
            if ":" in line:
                k, v = line.split(":", 1)
                fields[k.strip()] = v.strip()
        if (fields.get("workload_name") == config and fields.get("kernel_source_sha256") == digest
                and "traffic_bytes_per_launch" in fields):
            return int(fields["traffic_bytes_per_launch"])
    return None


def measured_mfma_util(config: str, kernel: str = "stage1_kernel", sources=KERNEL_SOURCES):
    """MFMA utilisation of ``kernel`` on this workload (SQ_VALU_MFMA_BUSY_CYCLES over the
    SIMDs' cycles, rocprofv3 counters) from the committed kernel-trace summary, or None when
    there is none or the kernel sources changed since it was taken."""
    import re

    digest = source_digest(sources)
    path = os.path.join(ROOT, "profiles", f"{kernel}_{config}_kernel_trace.txt")
    if not os.path.exists(path):
        return None
    text = open(path).read()
    if f"SHA-256 {digest}" not in text:
        return None
    m = re.search(r"MFMA utilisation .*?= ([0-9.]+)%", text)
    return round(float(m.group(1)) / 100, 4) if m else None


def cpu_baseline(w, out_gpu: np.ndarray, budget_s: float, threads: int = 0):
    """Times the fp64 oracle on a bounded sample (whole requests, in order, until the
    time budget is spent) and compares the GPU output of those requests with it.
    threads > 0 limits torch and the BLAS pools to that many threads."""
    import contextlib

    import torch
    from threadpoolctl import threadpool_limits

    from oracle.attention import decode_attention
    from paged_split_kv_stage1_amd.accounting import step_accounting
    sys.path.insert(0, os.path.join(ROOT, "tests"))
    from tests.oracle_inputs import max_rel_err, oracle_inputs

    cores = threads if threads > 0 else len(os.sched_getaffinity(0))
    torch.set_num_threads(cores)
    t_setup = time.perf_counter()
    reqs = []
    elapsed = 0.0
    err = 0.0
    oi_all = None
    for b in range(w.batch):
        if oi_all is None or w.kv_scale_mode == "per_token_head":
            oi = oracle_inputs(w, requests=[b] if w.kv_scale_mode == "per_token_head" else None)
            if w.kv_scale_mode != "per_token_head":
                oi_all = oi
        else:
            oi = oi_all
        if b == 0:
            t_setup = time.perf_counter()      # the wall-clock guard starts after the first setup
        t0 = time.perf_counter()
        with threadpool_limits(limits=threads) if threads > 0 else contextlib.nullcontext():
            out, _ = decode_attention(oi["q64"], oi["k"], oi["v"], w.page_indices, w.kv_indptr, w.kv_len,
                                      w.qo_indptr, w.window, w.sm_scale, requests=[b])
        elapsed += time.perf_counter() - t0
        rows = slice(int(w.qo_indptr[b]), int(w.qo_indptr[b + 1]))
        err = max(err, max_rel_err(out_gpu[rows], out[rows]))
        reqs.append(b)
        if elapsed >= budget_s or time.perf_counter() - t_setup > 3 * budget_s:
            break
    sel = np.array(reqs)
    qo = np.concatenate([[0], np.cumsum(np.diff(w.qo_indptr)[sel])])
    acc = step_accounting(len(sel), qo, w.kv_len[sel], w.window[sel], w.page_size, w.num_q_heads, w.num_kv_heads,
                          w.head_dim, w.q_dtype, w.kv_dtype, w.kv_scale_mode, w.out_dtype)
    return {"value": round(acc["bytes"] / elapsed / 1e9, 4), "unit": "GB/s", "cores": cores, "kind": "oracle",
            "sample": f"{len(sel)} of {w.batch} requests (all rows, heads and visible tokens of each), "
                      f"{elapsed:.1f} s of fp64 numpy on {cores} threads, {_cpu_model()}",
            "seconds": round(elapsed, 3)}, err


def cache_op_bytes(op: str, n: int, hkv: int, d: int, kv: str, mode: str) -> int:
    """Algorithmic HBM bytes of one cache operation over n tokens of bf16 rows [n, Hkv, d].

    kv_append: per K or V row, read the bf16 row (2d), write the cache row (d codes or 2d
    bf16) and, per token and head, the fp32 scale; plus the int64 slot of each token.
    kv_quantize (one tensor of n*Hkv rows): per-row mode reads 2d and writes d + 4 per
    row; per-tensor mode reads the tensor twice (the amax must be known before encoding
    and the tensor does not fit on chip) and writes d per row."""
    cb = 1 if kv == "fp8" else 2
    pt = mode == "per_token_head"
    if op == "kv_append":
        return n * 8 + 2 * n * hkv * (2 * d + cb * d + (4 if pt else 0))
    rows = n * hkv
    return rows * (3 * d + 4) if pt else rows * 5 * d


def cache_op_cpu_baseline(op, hkv, d, P, kv, mode, budget_s):
    """Times the oracle's append / quantiser on growing samples of tokens until the
    budget is spent (single thread: the oracle loops over rows in Python)."""
    import torch
    from threadpoolctl import threadpool_limits

    from oracle.cache import append_kv
    from oracle.quantize import quantize_per_row, quantize_per_tensor

    kind = {"none": "bf16", "per_tensor": "fp8_per_tensor", "per_token_head": "fp8_per_token_head"}[mode]
    gen = torch.Generator().manual_seed(11)
    m, elapsed, done = 16, 0.0, 0
    with threadpool_limits(limits=1):
        while elapsed < budget_s:
            bits = torch.randn(m, hkv, d, generator=gen).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
            t0 = time.perf_counter()
            if op == "kv_append":
                pages = (m + P - 1) // P
                cache = np.zeros((pages, hkv, P, d), dtype=np.uint8 if kv == "fp8" else np.uint16)
                sc = np.zeros((pages, hkv, P), dtype=np.float32) if kind == "fp8_per_token_head" else None
                for _ in range(2):                                  # K and V
                    append_kv(cache, sc, bits, "bf16", np.arange(m), P, kind, tensor_scale=0.02)
            elif mode == "per_token_head":
                quantize_per_row(bits.reshape(m * hkv, d), "bf16")
            else:
                quantize_per_tensor(bits.reshape(m * hkv, d), "bf16")
            elapsed += time.perf_counter() - t0
            done += m
            # double the batch, but not past what the rest of the budget can take
            m = max(16, min(2 * m, int((budget_s - elapsed) * done / elapsed)))
    return {"value": round(cache_op_bytes(op, done, hkv, d, kv, mode) / elapsed / 1e9, 5), "unit": "GB/s",
            "cores": 1, "kind": "oracle",
            "sample": f"{done} tokens x {hkv} KV heads in growing batches, {elapsed:.1f} s of numpy on 1 thread, "
                      f"{_cpu_model()}", "seconds": round(elapsed, 3)}


def bench_cache_op(args):
    """KV append (new tokens' bf16 K/V rows into random pages of the paged cache) or the
    standalone quantiser, on one workload's cache geometry and dtypes."""
    import torch

    from paged_split_kv_stage1_amd import pa_kv_append, pa_kv_quantize_fp8
    from paged_split_kv_stage1_amd.inputs import CONFIGS

    cfg = CONFIGS[args.config]
    hkv, d, P, kv, mode = cfg["hkv"], cfg["d"], cfg["page"], cfg["kv"], cfg["scale"]
    if args.op == "kv_quantize" and kv != "fp8":
        raise SystemExit(f"{args.config} keeps a bf16 cache: nothing to quantise")
    n = args.tokens
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    gen = torch.Generator().manual_seed(7)
    k_new = torch.randn(n, hkv, d, generator=gen).to(torch.bfloat16).to(dev)
    v_new = (torch.randn(n, hkv, d, generator=gen) * 2).to(torch.bfloat16).to(dev)
    stream = torch.cuda.current_stream()
    pt = mode == "per_token_head"
    if args.op == "kv_append":
        pages = (n + P - 1) // P + 64
        perm = np.random.default_rng(7).permutation(pages)
        slots = torch.from_numpy((perm[np.arange(n) // P] * P + np.arange(n) % P).astype(np.int64)).to(dev)
        dt = torch.uint8 if kv == "fp8" else torch.bfloat16
        kc = torch.zeros(pages, hkv, P, d, dtype=dt, device=dev)
        vc = torch.zeros_like(kc)
        layout = (hkv * P * d, P * d, d)
        ks = vs = sl = None
        if pt:
            ks = torch.zeros(pages, hkv, P, dtype=torch.float32, device=dev)
            vs = torch.zeros_like(ks)
            sl = (hkv * P, P, 1)
        elif mode == "per_tensor":
            ks = torch.full((1,), 0.02, dtype=torch.float32, device=dev)
            vs = torch.full((1,), 0.04, dtype=torch.float32, device=dev)

        def run():
            pa_kv_append(k_new, v_new, "bf16", n, hkv, d, P, slots, kc, vc, kv, mode, layout, ks, vs, sl,
                         stream=stream)
        kernel = "append_kernel"
    else:
        codes = torch.empty(n, hkv, d, dtype=torch.uint8, device=dev)
        scale = torch.empty(n * hkv if pt else 1, dtype=torch.float32, device=dev)

        def run():
            pa_kv_quantize_fp8(k_new, "bf16", n * hkv, d, mode, codes, scale, stream=stream)
        kernel = "quant_rows_kernel" if pt else "quant_tensor_kernel"
    flush = torch.empty(512 * 1024 * 1024 // 4, dtype=torch.float32, device=dev)
    _spin_up(flush)
    for _ in range(args.warmup):
        flush.fill_(1.0)
        run()
    torch.cuda.synchronize()
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(args.steps)]
    for i in range(args.steps):
        flush.fill_(1.0)
        ev[i][0].record(stream)
        run()
        ev[i][1].record(stream)
    torch.cuda.synchronize()
    us = float(np.mean([e[0].elapsed_time(e[1]) for e in ev])) * 1e3
    nbytes = cache_op_bytes(args.op, n, hkv, d, kv, mode)
    gbps = nbytes / (us * 1e-6) / 1e9
    what = {"kv_append": f"append {n} tokens into random pages", "kv_quantize": f"quantise {n * hkv} rows"}[args.op]
    result = {
        "metric": f"{args.op} achieved HBM GB/s, 1 GPU", "value": round(gbps, 2), "unit": "GB/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(us / 1e3, 6), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "bf16 -> " + ("bf16" if kv == "bf16" else "fp8-e4m3"),
        "data": "synthetic (seeded N(0,1) bf16 rows)",
        "config": {"workload": f"{what}, {hkv} KV heads d{d} P{P} {kv} cache, scales {mode}", "op": args.op,
                   "name": args.config, "tokens": n, "num_kv_heads": hkv, "head_dim": d, "page_size": P,
                   "kv_dtype": kv, "kv_scale_mode": mode, "cache_flush_between_steps": True},
        "us_per_step": round(us, 3), "algorithmic_bytes_per_step": nbytes,
        "roofline": {"bound": "hbm", "achieved": round(gbps, 2), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                     "frac": round(gbps / HBM_PEAK_GBPS, 4),
                     "traffic": measured_traffic(f"{args.op}_{args.config}", kernel, CACHE_OP_SOURCES),
                     "kernel": kernel, "bytes_per_launch": nbytes},
    }
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cache_op_cpu_baseline(args.op, hkv, d, P, kv, mode, args.cpu_budget)
    print(json.dumps(result), flush=True)


def _spin_up(flush, seconds: float = 0.5):
    """Streams the flush buffer for ``seconds`` before the warm-up steps: a few dozen steps
    of tens of microseconds do not bring the clocks up, so without this the warm-up and the
    first timed steps (and a profiler's per-call average over all of them) run slower."""
    import torch

    t_end = time.perf_counter() + seconds
    while time.perf_counter() < t_end:
        for _ in range(10):
            flush.fill_(1.0)
        torch.cuda.synchronize()


def _calibrate_copy():
    """One 256 MiB device-to-device copy: a known-size reference for the HBM counters."""
    import torch

    src = torch.ones(256 * 1024 * 1024 // 4, dtype=torch.float32, device="cuda:0")
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    dst.copy_(src)
    torch.cuda.synchronize()
    del src, dst


def iqm(x):
    x = np.sort(x)
    n = len(x)
    return float(np.mean(x[n // 4: n - n // 4])) if n >= 4 else float(np.mean(x))


def time_steps(pd, step, merge, flush, stream, steps, warmup, do_flush):
    """Warm-up steps, then ``steps`` timed steps, each after a cache-evicting write of the
    flush buffer, with HIP events on the launch stream around each step (stage 1 + merge
    launched back to back, nothing between them).  When the plan has a merge, a second
    pass of ``steps`` steps puts a third event between the two launches to split the time
    into stage 1 and merge; that marker itself delays the merge launch by a few µs, so the
    step time comes from the first pass.
    Returns (step us, stage-1 us, merge us, wall seconds of the first timed pass); arrays
    with one entry per step."""
    import torch

    for _ in range(warmup):
        if do_flush:
            flush.fill_(1.0)
        step()
        merge()
    torch.cuda.synchronize()
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(steps):
        if do_flush:
            flush.fill_(1.0)
        ev[i][0].record(stream)
        step()
        merge()
        ev[i][1].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    tot = np.array([e[0].elapsed_time(e[1]) for e in ev]) * 1e3      # us
    if not pd.info.needs_merge:          # no merge launch: the step is stage 1
        return tot, tot.copy(), np.zeros_like(tot), wall
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(steps)]
    for i in range(steps):
        if do_flush:
            flush.fill_(1.0)
        ev[i][0].record(stream)
        step()
        ev[i][1].record(stream)
        merge()
        ev[i][2].record(stream)
    torch.cuda.synchronize()
    s1 = np.array([e[0].elapsed_time(e[1]) for e in ev]) * 1e3
    mg = np.array([e[1].elapsed_time(e[2]) for e in ev]) * 1e3
    return tot, s1, mg, wall


# Every configuration of the benchmark target, timed in the default run after the
# headline: the five workloads, the batch-1 and row-count variants the R8/R1 bar compares.
PER_CONFIG = ("c1", "c3", "c3_r1", "c3_r8", "c3_b1", "c3_b1_r1", "c3_b1_r8", "c4", "c4_r1", "c4_b1", "c4_b1_r1",
              "c5", "f3", "mla")
MEMORY_BOUND = {"c2", "c3", "c3_r1", "c3_r8", "c3_b1", "c3_b1_r1", "c3_b1_r8", "c4", "c4_r1", "c4_b1", "c4_b1_r1",
                "c5"}
R8_R1 = (("c3_r8", "c3_r1"), ("c3_b1_r8", "c3_b1_r1"), ("c4", "c4_r1"), ("c4_b1", "c4_b1_r1"))


def arithmetic(w, variant: int) -> str:
    """What the stage-1 kernel of this plan multiplies in, from the tile configuration."""
    if (variant >> 16) & 1:
        return arithmetic(w, variant & ~(1 << 16)) + "; query rows on the MFMA M axis (S = Q K^T, O = P V, P " \
            "transposed through LDS)"
    if (variant >> 14) & 1:
        if (variant >> 15) & 1:
            return ("bf16 MFMA on the e4m3 latent codes upconverted exactly: q.k per 128-channel block times both "
                    "scales plus the bf16 rotary part; P.V with P times the token's block scale (one bf16 term)")
        return "bf16 MFMA for q.k (192 channels) and P.V (128 channels, P as two bf16 terms)"
    qf8, kvf8, pt = (variant >> 1) & 1, (variant >> 2) & 1, (variant >> 3) & 1
    wq, nqb, i8 = (variant >> 4) & 15, (variant >> 8) & 15, (variant >> 12) & 1
    one_block_waves = wq == 4 and nqb == 1
    if not kvf8:
        return "bf16 MFMA for q.k and P.V (P as two bf16 terms)"
    if qf8:
        return "e4m3 MFMA for q.k (exact products) and P.V (P as two e4m3 terms)"
    if i8:
        qk = ("int8 MFMA on the raw K codes, bf16 query as two int8 terms" if one_block_waves
              else "bf16 MFMA on K converted to bf16")
        return f"q.k: {qk}; P.V: bf16 MFMA on V converted to bf16 (P one bf16 term, v_scale folded)"
    if pt and one_block_waves:
        qk = "e4m3 16x16x128 MFMA on the raw K codes, bf16 query as two e4m3 terms under a per-row scale"
    else:
        qk = "bf16 MFMA on K upconverted exactly from e4m3"
    pv = ("bf16 MFMA on V upconverted exactly from e4m3 (P one bf16 term, v_scale folded)" if pt
          else "e4m3 MFMA (P as two e4m3 terms)")
    return f"q.k: {qk}; P.V: {pv}"


def stage1_call(pd, di, w, out, stream):
    """Stage 1 of the plan: the equal-width kernel, or the one for keys wider than values."""
    if pd.rope:
        pd.stage1_rope(di, w.sm_scale, out, w.out_dtype, stream=stream)
    else:
        pd.stage1(di.q, di.q_scale, di.k, di.v, di.kv_layout, di.k_scale, di.v_scale, di.scale_layout,
                  di.page_indices, w.sm_scale, out, w.out_dtype, stream=stream)


def per_config(args, flush, stream):
    """Stage-1 and merge times of every configuration in PER_CONFIG (same flush and events as
    the headline; at least 20 timed and 50 warm-up steps each), with achieved GB/s against
    8 TB/s and the R8/R1 ratios."""
    import torch

    from paged_split_kv_stage1_amd.accounting import workload_accounting
    from paged_split_kv_stage1_amd.decode import PagedDecode
    from paged_split_kv_stage1_amd.device_inputs import to_device
    from paged_split_kv_stage1_amd.inputs import make_workload

    res = {}
    for name in PER_CONFIG:
        w = make_workload(name)
        di = to_device(w, "cuda:0")
        acc = workload_accounting(w)
        pd = PagedDecode(w.qo_indptr, w.kv_indptr, w.kv_len, w.window, w.max_q_len, w.page_size, w.num_q_heads,
                         w.num_kv_heads, w.head_dim, w.q_dtype, w.kv_dtype, w.kv_scale_mode, di.q.device,
                         force_splits=w.forced_splits, head_dim_v=w.head_dim_v)
        out = torch.empty(w.total_rows, w.num_q_heads, w.dv,
                          dtype=torch.float32 if w.out_dtype == "fp32" else torch.bfloat16, device=di.q.device)

        def step():
            stage1_call(pd, di, w, out, stream)

        def merge():
            pd.merge(out, w.out_dtype, stream=stream)

        # at least 50 warm-up steps: the compute-heavy shapes need that many back-to-back
        # steps before the clocks settle, whatever the headline's own warm-up count is
        st, s1, mg, _ = time_steps(pd, step, merge, flush, stream, max(args.steps, 20), max(args.warmup, 50),
                                   not args.no_flush)
        tot = float(np.mean(st))
        gbps = acc["bytes"] / (tot * 1e-6) / 1e9
        res[name] = {"workload": WORKLOAD_NAMES[name], "stage1_us": round(float(np.mean(s1)), 2),
                     "merge_us": round(float(np.mean(mg)), 2), "us_per_step": round(tot, 2),
                     "algorithmic_bytes": acc["bytes"], "gbps": round(gbps, 1),
                     "frac_of_8tbs": round(gbps / HBM_PEAK_GBPS, 4), "work_items": pd.num_items,
                     "max_splits": pd.max_splits, "arithmetic": arithmetic(w, int(pd.info.variant)),
                     "mfma_util": measured_mfma_util(name, *stage1_kernel_of(w.latent, pd.rope))}
        if name in MEMORY_BOUND:
            res[name]["meets_70pct"] = bool(gbps >= 0.7 * HBM_PEAK_GBPS)
        del di, out, pd
        torch.cuda.empty_cache()
    ratios = {f"{r8}/{r1}": round(res[r8]["us_per_step"] / res[r1]["us_per_step"], 3)
              for r8, r1 in R8_R1 if r8 in res and r1 in res}
    return res, ratios


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    # compute-heavy workloads need ~50 back-to-back steps before the clocks settle
    ap.add_argument("--warmup", type=int, default=100)
    ap.add_argument("--config", default="c2", choices=sorted(WORKLOAD_NAMES))
    ap.add_argument("--no-flush", action="store_true", help="skip the cache-evicting write between steps")
    ap.add_argument("--cpu-budget", type=float, default=15.0, help="seconds of oracle work for cpu_baseline")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--force-splits", type=int, default=None)
    ap.add_argument("--orientation", default="kv_on_m", choices=["kv_on_m", "q_on_m"],
                    help="stage 1 with the key tokens (default) or the query rows on the MFMA M axis")
    ap.add_argument("--graph-reps", type=int, default=100,
                    help="also time this many replays of stage 1 + merge captured in one hipGraph (0: skip)")
    ap.add_argument("--op", default="decode", choices=["decode", "kv_append", "kv_quantize"],
                    help="decode (stage 1 + merge), or the cache-side append / quantiser on the workload's geometry")
    ap.add_argument("--tokens", type=int, default=131072, help="tokens appended or quantised per step (cache ops)")
    ap.add_argument("--no-per-config", action="store_true",
                    help="time only the headline workload (skip the per_config object of every configuration)")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="run one 256 MiB device-to-device copy first, as a known-size reference for HBM counters")
    args = ap.parse_args()
    if args.gpus != 1:
        print(json.dumps({"error": "the library and this benchmark run on one GPU; run with --gpus 1"}))
        sys.exit(2)
    if args.calibrate_copy:
        _calibrate_copy()
    if args.op != "decode":
        return bench_cache_op(args)

    import torch

    from paged_split_kv_stage1_amd.accounting import workload_accounting
    from paged_split_kv_stage1_amd.decode import PagedDecode
    from paged_split_kv_stage1_amd.device_inputs import to_device
    from paged_split_kv_stage1_amd.inputs import make_workload

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    w = make_workload(args.config)
    di = to_device(w, dev)
    acc = workload_accounting(w)
    pd = PagedDecode(w.qo_indptr, w.kv_indptr, w.kv_len, w.window, w.max_q_len, w.page_size, w.num_q_heads,
                     w.num_kv_heads, w.head_dim, w.q_dtype, w.kv_dtype, w.kv_scale_mode, dev,
                     force_splits=w.forced_splits if args.force_splits is None else args.force_splits,
                     head_dim_v=w.head_dim_v, orientation=args.orientation)
    out = torch.empty(w.total_rows, w.num_q_heads, w.dv,
                      dtype=torch.float32 if w.out_dtype == "fp32" else torch.bfloat16, device=dev)
    flush = torch.empty(512 * 1024 * 1024 // 4, dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream()

    def step():
        stage1_call(pd, di, w, out, stream)

    def merge():
        pd.merge(out, w.out_dtype, stream=stream)

    def step_on(st):
        stage1_call(pd, di, w, out, st)
        pd.merge(out, w.out_dtype, stream=st)

    _spin_up(flush)
    tot, s1, mg, wall = time_steps(pd, step, merge, flush, stream, args.steps, args.warmup, not args.no_flush)

    graph = None
    if args.graph_reps > 0:
        # the same two launches captured once and replayed; flush stays outside the graph
        g = torch.cuda.CUDAGraph()
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            step_on(side)
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        with torch.cuda.graph(g):
            step_on(torch.cuda.current_stream())
        for _ in range(3):
            g.replay()
        gev = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(args.graph_reps)]
        for i in range(args.graph_reps):
            if not args.no_flush:
                flush.fill_(1.0)
            gev[i][0].record()
            g.replay()
            gev[i][1].record()
        torch.cuda.synchronize()
        gt = np.array([e[0].elapsed_time(e[1]) for e in gev]) * 1e3
        graph = {"reps": args.graph_reps, "us_per_step_mean": round(float(np.mean(gt)), 3),
                 "us_per_step_iqm": round(iqm(gt), 3)}

    us_step = float(np.mean(tot))
    gbps = acc["bytes"] / (us_step * 1e-6) / 1e9
    s1_us = float(np.mean(s1))
    s1_bytes = acc["bytes"]
    roof_achieved = s1_bytes / (s1_us * 1e-6) / 1e9
    result = {
        "metric": METRIC, "value": round(gbps, 2), "unit": "GB/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(us_step / 1e3, 6), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": ("bf16" if w.kv_dtype == "bf16" else "int8" if w.kv_dtype == "int8" else "fp8-e4m3"),
        "arithmetic": arithmetic(w, int(pd.info.variant)),
        "data": "synthetic (seeded N(0,1), random page permutation)",
        "config": {"workload": WORKLOAD_NAMES[args.config], "name": args.config, "batch": w.batch,
                   "total_rows": w.total_rows, "num_q_heads": w.num_q_heads, "num_kv_heads": w.num_kv_heads,
                   "head_dim": w.head_dim, "page_size": w.page_size, "kv_dtype": w.kv_dtype,
                   "kv_scale_mode": w.kv_scale_mode, "work_items": pd.num_items, "max_splits": pd.max_splits,
                   "orientation": args.orientation, "cache_flush_between_steps": not args.no_flush},
        "us_per_step": round(us_step, 3), "us_per_step_iqm": round(iqm(tot), 3),
        "stage1_us": round(s1_us, 3), "merge_us": round(float(np.mean(mg)), 3), "graph_replay": graph,
        "pct_of_hbm_peak": round(100.0 * gbps / HBM_PEAK_GBPS, 2),
        "algorithmic_bytes_per_step": acc["bytes"], "algorithmic_flops_per_step": acc["flops"],
        "tflops": round(acc["flops"] / (us_step * 1e-6) / 1e12, 3),
        "wall_ms_per_step_incl_flush": round(wall / args.steps * 1e3, 4),
        "roofline": {"bound": "hbm", "achieved": round(roof_achieved, 2), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                     "frac": round(roof_achieved / HBM_PEAK_GBPS, 4),
                     "traffic": (measured_traffic(args.config, *stage1_kernel_of(w.latent, pd.rope))
                                 if args.orientation == "kv_on_m" else None),
                     "kernel": stage1_kernel_of(w.latent, pd.rope)[0], "bytes_per_launch": s1_bytes,
                     "mfma_util": (measured_mfma_util(args.config, *stage1_kernel_of(w.latent, pd.rope))
                                   if args.orientation == "kv_on_m" else None)},
    }
    if not args.no_per_config and args.config == "c2" and args.orientation == "kv_on_m":
        result["per_config"], result["r8_over_r1"] = per_config(args, flush, stream)
    if not args.no_cpu_baseline:
        out_np = out.float().cpu().numpy().astype(np.float64)
        cb, err = cpu_baseline(w, out_np, args.cpu_budget)
        result["cpu_baseline"] = cb
        result["sampled_parity_maxrel"] = err
        cb1, _ = cpu_baseline(w, out_np, min(3.0, args.cpu_budget), threads=1)
        result["cpu_baseline_1core"] = {k: cb1[k] for k in ("value", "unit", "cores", "sample")}
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
