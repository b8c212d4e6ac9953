"""GPU test of the allocation-free decode entry point (pa_decode_noalloc): its output and
LSE must equal, bit for bit, those of stage 1 + merge with caller workspace on the same
plan and inputs (the same kernels run; only where the split partials live differs), on
two calls in a row, the second with a smaller input, and stay within the oracle's bar."""
import numpy as np
import pytest
import torch

from oracle.attention import decode_attention
from paged_split_kv_stage1_amd import pa_decode_noalloc
from paged_split_kv_stage1_amd.decode import PagedDecode
from paged_split_kv_stage1_amd.device_inputs import to_device
from paged_split_kv_stage1_amd.inputs import make_workload
from tests.oracle_inputs import max_rel_err, oracle_inputs

pytestmark = pytest.mark.gpu

BAR = {"bf16": 2e-3, "fp8": 2e-2, "int8": 2e-2}


def _both(name, shape, force):
    w = make_workload(name, **shape, out_dtype="fp32")
    di = to_device(w)
    pd = PagedDecode(w.qo_indptr, w.kv_indptr, w.kv_len, w.window, w.max_q_len, w.page_size, w.num_q_heads,
                     w.num_kv_heads, w.head_dim, w.q_dtype, w.kv_dtype, w.kv_scale_mode, di.q.device,
                     force_splits=force)
    shape_o = (w.total_rows, w.num_q_heads, w.head_dim)
    out_ws = torch.full(shape_o, float("nan"), dtype=torch.float32, device="cuda")
    lse_ws = torch.full(shape_o[:2], float("nan"), dtype=torch.float32, device="cuda")
    out_na = torch.full_like(out_ws, float("nan"))
    lse_na = torch.full_like(lse_ws, float("nan"))
    pd.run(di.q, di.q_scale, di.k, di.v, di.kv_layout, di.k_scale, di.v_scale, di.scale_layout, di.page_indices,
           w.sm_scale, out_ws, "fp32", out_lse=lse_ws)
    pa_decode_noalloc(pd.info, pd.plan, di.q, di.q_scale, di.k, di.v, di.kv_layout, di.k_scale, di.v_scale,
                      di.scale_layout, di.page_indices, w.sm_scale, out_na, "fp32", lse_na)
    torch.cuda.synchronize()
    return w, pd, out_ws.cpu().numpy(), lse_ws.cpu().numpy(), out_na.cpu().numpy(), lse_na.cpu().numpy()


def test_noalloc_equals_workspace_path_on_two_calls_second_smaller():
    cases = [("c4", dict(batch=2, ctx=[2500, 700]), 9),        # FP8 per-token-head, bf16 partials
             ("c3", dict(batch=1, ctx=[517]), 3)]               # bf16, float32 partials; smaller plan
    sizes = []
    for name, shape, force in cases:
        print(f"[noalloc] {name} {shape} splits {force}", flush=True)
        w, pd, o_ws, l_ws, o_na, l_na = _both(name, shape, force)
        assert pd.info.needs_merge
        sizes.append(int(pd.info.partial_o_bytes))
        assert not np.isnan(o_na).any() and not np.isnan(l_na).any()
        assert np.array_equal(o_na.view(np.uint32), o_ws.view(np.uint32))
        assert np.array_equal(l_na.view(np.uint32), l_ws.view(np.uint32))
        oi = oracle_inputs(w)
        ref, _ = decode_attention(oi["q64"], oi["k"], oi["v"], w.page_indices, w.kv_indptr, w.kv_len, w.qo_indptr,
                                  w.window, w.sm_scale)
        assert max_rel_err(o_na.astype(np.float64), ref) <= BAR[w.kv_dtype]
    assert sizes[1] < sizes[0]


def test_noalloc_single_split_plan():
    # no split partials at all: stage 1 writes the output and LSE directly
    w, pd, o_ws, l_ws, o_na, l_na = _both("c2", dict(batch=3, ctx=[300, 77, 1000]), 1)
    assert not pd.info.needs_merge
    assert np.array_equal(o_na.view(np.uint32), o_ws.view(np.uint32))
    assert np.array_equal(l_na.view(np.uint32), l_ws.view(np.uint32))
