"""Helpers for the GPU tests: run one decode step through the C ABI."""
import numpy as np
import torch

from paged_split_kv_stage1_amd.decode import PagedDecode


def run_decode(w, di, force_splits=None, out_dtype=None, max_splits=0, num_cus=0, out_lse=False,
               orientation="kv_on_m"):
    out_dtype = out_dtype or w.out_dtype
    fs = w.forced_splits if force_splits is None else force_splits
    pd = PagedDecode(w.qo_indptr, w.kv_indptr, w.kv_len, w.window, w.max_q_len, w.page_size, w.num_q_heads,
                     w.num_kv_heads, w.head_dim, w.q_dtype, w.kv_dtype, w.kv_scale_mode, di.q.device,
                     num_cus=num_cus, max_splits=max_splits, force_splits=fs, head_dim_v=w.head_dim_v,
                     orientation=orientation)
    T = w.total_rows
    out = torch.full((T, w.num_q_heads, w.dv), float("nan"),
                     dtype=torch.float32 if out_dtype == "fp32" else torch.bfloat16, device=di.q.device)
    lse = torch.full((T, w.num_q_heads), float("nan"), dtype=torch.float32, device=di.q.device) if out_lse else None
    pd.run_inputs(di, w.sm_scale, out, out_dtype, out_lse=lse)
    torch.cuda.synchronize()
    o = out.float().cpu().numpy().astype(np.float64)
    return (o, pd, lse.cpu().numpy() if out_lse else None)
