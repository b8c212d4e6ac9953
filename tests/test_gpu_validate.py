"""GPU tests of the page-table check (pa_validate_page_indices and PA_VALIDATE=1): a
table whose entries all lie inside the caches passes; entries outside them are reported
(count and first position) before stage 1 is launched, so the kernel never reads them."""
import pytest
import torch

from paged_split_kv_stage1_amd import PaError, pa_validate_page_indices
from paged_split_kv_stage1_amd._lib import PA_ERR_INVALID_ARGUMENT
from paged_split_kv_stage1_amd.decode import PagedDecode
from paged_split_kv_stage1_amd.device_inputs import to_device
from paged_split_kv_stage1_amd.inputs import make_workload

pytestmark = pytest.mark.gpu


def _setup():
    w = make_workload("c3", batch=3, ctx=[3001, 517, 4], out_dtype="fp32")
    di = to_device(w)
    pd = PagedDecode(w.qo_indptr, w.kv_indptr, w.kv_len, w.window, w.max_q_len, w.page_size, w.num_q_heads,
                     w.num_kv_heads, w.head_dim, w.q_dtype, w.kv_dtype, w.kv_scale_mode, di.q.device,
                     force_splits=3)
    return w, di, pd


def test_validate_accepts_a_good_table_and_reports_bad_entries():
    w, di, pd = _setup()
    npages = di.k.shape[0]
    pa_validate_page_indices(pd.info, pd.plan, di.page_indices, npages)
    bad = di.page_indices.clone()
    bad[5] = npages + 7
    bad[190] = -1                       # request 1's first page (request 0 has 188)
    with pytest.raises(PaError) as e:
        pa_validate_page_indices(pd.info, pd.plan, bad, npages)
    assert e.value.status == PA_ERR_INVALID_ARGUMENT
    # each entry is read by the items of both KV heads: 2 bad entries, 4 reads
    assert "4 reads" in str(e.value) and "page_indices[5]" in str(e.value)
    with pytest.raises(PaError):        # one page fewer in the caches: the largest entry is out
        pa_validate_page_indices(pd.info, pd.plan, di.page_indices, int(di.page_indices.max().item()))


def test_pa_validate_environment_stops_stage1(monkeypatch):
    w, di, pd = _setup()
    bad = di.page_indices.clone()
    bad[0] = 1 << 30
    out = torch.full((w.total_rows, w.num_q_heads, w.head_dim), float("nan"), device="cuda")
    monkeypatch.setenv("PA_VALIDATE", "1")
    with pytest.raises(PaError):
        pd.run(di.q, di.q_scale, di.k, di.v, di.kv_layout, di.k_scale, di.v_scale, di.scale_layout, bad,
               w.sm_scale, out, "fp32")
    torch.cuda.synchronize()
    assert torch.isnan(out).all()       # nothing was launched
    pd.run(di.q, di.q_scale, di.k, di.v, di.kv_layout, di.k_scale, di.v_scale, di.scale_layout, di.page_indices,
           w.sm_scale, out, "fp32")
    torch.cuda.synchronize()
    assert not torch.isnan(out).any()
