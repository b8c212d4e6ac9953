"""Parity at the workloads' full sizes, in the launch configuration bench.py times
(planner-chosen splits, the workload's own output dtype): every row and head of one whole
request (the one with the most rows, ties to the shortest context), plus sampled outputs
of other requests that the oracle computes one (row, head) at a time."""
import numpy as np
import pytest
import torch

from oracle.attention import decode_attention, decode_attention_one
from paged_split_kv_stage1_amd.device_inputs import to_device
from paged_split_kv_stage1_amd.inputs import make_workload
from tests.gpu_run import run_decode
from tests.oracle_inputs import max_rel_err, oracle_inputs

pytestmark = pytest.mark.gpu

BAR = {"bf16": 2e-3, "fp8": 2e-2, "int8": 2e-2}
OUT_EXTRA = {"bf16": 2.0 ** -8, "fp32": 0.0}      # bf16 output rounding on top of the bar


def _samples(w, rng, n=6):
    """(row t, query head h) pairs: the first and last row of the batch, the last row of
    the longest request, and random ones."""
    T, Hq = w.total_rows, w.num_q_heads
    longest = int(np.argmax(w.kv_len))
    picks = [(0, 0), (T - 1, Hq - 1), (int(w.qo_indptr[longest + 1]) - 1, Hq // 2)]
    while len(picks) < n:
        picks.append((int(rng.integers(T)), int(rng.integers(Hq))))
    return picks


@pytest.mark.parametrize("name", ["c2", "c2_ph", "c3", "c3_b1", "c3_r1", "c3_r8", "c4", "c4_r1", "c4_b1", "c4_b1_r1",
                                  "c4_i8", "c5", "c6", "c6_f8", "f3", "f3_r4", "mla", "mla_r2"])
def test_full_size_whole_request_and_samples(name):
    print(f"[full-size] {name}", flush=True)
    w = make_workload(name)
    di = to_device(w)
    o, pd, _ = run_decode(w, di)
    print(f"  items={pd.num_items} S_max={pd.max_splits}", flush=True)
    assert not np.isnan(o).any()
    rows = np.diff(w.qo_indptr)
    whole = int(min(range(w.batch), key=lambda b: (-int(rows[b]), int(w.kv_len[b]))))
    picks = _samples(w, np.random.default_rng(11))
    reqs = sorted({int(np.searchsorted(w.qo_indptr, t, side="right") - 1) for t, _ in picks} | {whole})
    oi = oracle_inputs(w, requests=reqs if w.kv_scale_mode == "per_token_head" else None)
    bar = BAR[w.kv_dtype] + OUT_EXTRA[w.out_dtype]
    ref, _ = decode_attention(oi["q64"], oi["k"], oi["v"], w.page_indices, w.kv_indptr, w.kv_len, w.qo_indptr,
                              w.window, w.sm_scale, requests=[whole])
    sl = slice(int(w.qo_indptr[whole]), int(w.qo_indptr[whole + 1]))
    err_whole = max_rel_err(o[sl], ref[sl])
    assert err_whole <= bar, (whole, err_whole)
    worst = 0.0
    for t, h in picks:
        ref1, _ = decode_attention_one(oi["q64"][t, h], oi["k"], oi["v"], w.page_indices, w.kv_indptr, w.kv_len,
                                       w.qo_indptr, w.window, w.sm_scale, t, h, w.num_kv_heads, w.num_q_heads)
        err = max_rel_err(o[t, h][None], ref1[None])
        worst = max(worst, err)
        assert err <= bar, (t, h, err)
    print(f"  request {whole} ({rows[whole]} rows x {w.num_q_heads} heads, ctx {w.kv_len[whole]}) "
          f"maxrel={err_whole:.3e}; sampled maxrel={worst:.3e} (bar {bar:.3e})", flush=True)
