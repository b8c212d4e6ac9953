"""One decode step = plan (host) + stage 1 + merge, with torch providing device memory."""
from __future__ import annotations

import os
from typing import Optional, Sequence

import numpy as np
import torch

from ._lib import (pa_decode_merge, pa_decode_stage1, pa_decode_stage1_rope, pa_plan_splits,
                   pa_validate_page_indices)


class PagedDecode:
    """Plans a batch once and launches stage 1 + merge for it.

    The plan (work list) and the split scratch are device tensors owned by this
    object; the launches never allocate, so ``run`` can be captured in a HIP graph.
    """

    def __init__(self, qo_indptr, kv_indptr, kv_len, window, max_q_len: int, page_size: int, num_q_heads: int,
                 num_kv_heads: int, head_dim: int, q_dtype: str, kv_dtype: str, kv_scale_mode: str,
                 device: torch.device, num_cus: int = 0, max_splits: int = 0, force_splits: int = 0,
                 head_dim_v: int = 0, orientation: str = "kv_on_m"):
        self.info, plan = pa_plan_splits(qo_indptr, kv_indptr, kv_len, window, max_q_len, page_size, num_q_heads,
                                         num_kv_heads, head_dim, q_dtype, kv_dtype, kv_scale_mode, num_cus=num_cus,
                                         max_splits=max_splits, force_splits=force_splits, head_dim_v=head_dim_v,
                                         orientation=orientation)
        self.rope = head_dim_v not in (0, head_dim)
        self.plan_host = plan
        self.plan = torch.from_numpy(plan).to(device)
        n_o = max(1, int(self.info.partial_o_bytes) // 4)
        n_l = max(1, int(self.info.partial_lse_bytes) // 4)
        self.partial_o = torch.empty(n_o, dtype=torch.float32, device=device)
        self.partial_lse = torch.empty(n_l, dtype=torch.float32, device=device)

    @property
    def num_items(self) -> int:
        return int(self.info.num_items)

    @property
    def max_splits(self) -> int:
        return int(self.info.max_splits)

    def stage1(self, q, q_scale, k_cache, v_cache, kv_layout: Sequence[int], k_scale, v_scale,
               scale_layout: Optional[Sequence[int]], page_indices, sm_scale: float, out, out_dtype: str,
               out_lse=None, stream=None):
        if os.environ.get("PA_VALIDATE") == "1":         # page numbers must lie inside the caches
            pa_validate_page_indices(self.info, self.plan, page_indices, k_cache.shape[0], stream)
        pa_decode_stage1(self.info, self.plan, q, q_scale, k_cache, v_cache, kv_layout, k_scale, v_scale, scale_layout,
                         page_indices, sm_scale, self.partial_o, self.partial_lse, out, out_dtype, out_lse, stream)

    def stage1_rope(self, di, sm_scale: float, out, out_dtype: str, out_lse=None, stream=None):
        """Stage 1 of a plan whose keys are wider than their values, from DeviceInputs."""
        if os.environ.get("PA_VALIDATE") == "1":
            pa_validate_page_indices(self.info, self.plan, di.page_indices, di.k.shape[0], stream)
        pa_decode_stage1_rope(self.info, self.plan, di.q, di.q_scale, di.q_rope, di.k, di.kv_layout, di.k_rope,
                              di.rope_layout, di.k_scale, di.scale_layout, di.v, di.v_layout, di.page_indices,
                              sm_scale, self.partial_o, self.partial_lse, out, out_dtype, out_lse, stream)

    def run_inputs(self, di, sm_scale: float, out, out_dtype: str, out_lse=None, stream=None):
        """One decode step (stage 1 + merge) from DeviceInputs, for either kind of plan."""
        if self.rope:
            self.stage1_rope(di, sm_scale, out, out_dtype, out_lse, stream)
        else:
            self.stage1(di.q, di.q_scale, di.k, di.v, di.kv_layout, di.k_scale, di.v_scale, di.scale_layout,
                        di.page_indices, sm_scale, out, out_dtype, out_lse, stream)
        self.merge(out, out_dtype, out_lse, stream)

    def merge(self, out, out_dtype: str, out_lse=None, stream=None):
        pa_decode_merge(self.info, self.plan, self.partial_o, self.partial_lse, out, out_dtype, out_lse, stream)

    def run(self, q, q_scale, k_cache, v_cache, kv_layout, k_scale, v_scale, scale_layout, page_indices,
            sm_scale: float, out, out_dtype: str, out_lse=None, stream=None):
        self.stage1(q, q_scale, k_cache, v_cache, kv_layout, k_scale, v_scale, scale_layout, page_indices, sm_scale,
                    out, out_dtype, out_lse, stream)
        self.merge(out, out_dtype, out_lse, stream)

    def row_nsplit(self) -> np.ndarray:
        off = self.num_items * 64
        return self.plan_host[off:].view(np.int32)

    def items(self) -> np.ndarray:
        """Work items as an int32 [num_items, 16] array (host copy)."""
        return self.plan_host[: self.num_items * 64].view(np.int32).reshape(-1, 16)
