"""Every stage-1 tile configuration the library instantiates, in every KV format and query
dtype it supports, run once against the oracle on a small problem.  The (rows x group)
of each case selects the tile shape: 16 rows -> one query block, 32 -> two (two waves
per block), 64 -> four waves of one block, 128 -> two blocks per wave, 192 -> three
(head_dim 512: one block per wave, and 128 or 192 rows x heads split into two or three
work items per KV split)."""
import numpy as np
import pytest

from oracle.attention import decode_attention
from paged_split_kv_stage1_amd.device_inputs import to_device
from paged_split_kv_stage1_amd.inputs import make_workload
from tests.gpu_run import run_decode
from tests.oracle_inputs import max_rel_err, oracle_inputs

pytestmark = pytest.mark.gpu

BAR = {"bf16": 2e-3, "fp8": 2e-2, "int8": 2e-2}
MODES = {                         # (q dtype, kv dtype, scale mode)
    "bf16": ("bf16", "bf16", "none"),
    "fp8_tensor": ("bf16", "fp8", "per_tensor"),
    "fp8_tensor_q8": ("fp8", "fp8", "per_tensor"),
    "fp8_head": ("bf16", "fp8", "per_head"),
    "fp8_head_q8": ("fp8", "fp8", "per_head"),
    "fp8_token": ("bf16", "fp8", "per_token_head"),
    "fp8_token_q8": ("fp8", "fp8", "per_token_head"),
    "int8_token": ("bf16", "int8", "per_token_head"),
    "int8_tensor": ("bf16", "int8", "per_tensor"),
}
SHAPES = {16: (8, 2), 32: (8, 4), 64: (8, 8), 128: (16, 8), 192: (24, 8)}   # rows x group -> (G, R)


def _supported(d, mode, m):
    q, kv, scale = MODES[mode]
    if d == 512:                  # bf16 or per-token-head FP8 KV, bf16 queries, one block per wave
        return kv == "bf16" or (kv == "fp8" and scale == "per_token_head" and q == "bf16")
    per_tensor_v = kv == "fp8" and scale != "per_token_head"    # fp8 P.V keeps a second accumulator
    if d == 128:
        return m <= (128 if per_tensor_v else 192)
    return m <= (64 if per_tensor_v else 128)


CASES = [(d, mode, m) for d in (128, 256, 512) for mode in MODES for m in SHAPES if _supported(d, mode, m)]


@pytest.mark.parametrize("d,mode,m", CASES)
def test_every_tile_configuration(d, mode, m):
    q, kv, scale = MODES[mode]
    G, R = SHAPES[m]
    print(f"[coverage] d={d} {mode} rows x group={m}", flush=True)
    w = make_workload("c3", batch=2, ctx=[700, R + 37], rows=R, out_dtype="fp32",
                      overrides=dict(hq=2 * G, hkv=2, d=d, q=q, kv=kv, scale=scale))
    di = to_device(w)
    o, pd, _ = run_decode(w, di)
    oi = oracle_inputs(w)
    ref, _ = decode_attention(oi["q64"], oi["k"], oi["v"], w.page_indices, w.kv_indptr, w.kv_len, w.qo_indptr,
                              w.window, w.sm_scale)
    err = max_rel_err(o, ref)
    print(f"  variant={pd.info.variant:#x} items={pd.num_items} maxrel={err:.3e}", flush=True)
    assert not np.isnan(o).any()
    assert err <= BAR[kv], err
