"""MI355X (gfx950) paged split-KV decode attention: HIP kernels behind a C ABI.

The binding functions keep the C names of include/pa.h (pa_plan_splits,
pa_decode_stage1, pa_decode_merge, pa_kv_quantize_fp8, pa_kv_quantize_fp8_per_head,
pa_kv_quantize_int8, pa_kv_append, pa_debug_gather, pa_decode_noalloc,
pa_validate_page_indices);
``PagedDecode`` strings them together for one decode step with torch-owned buffers.
"""
from ._lib import (PaError, pa_debug_gather, pa_decode_merge, pa_decode_noalloc, pa_decode_stage1,  # noqa: F401
                   pa_decode_stage1_rope, pa_kv_append, pa_validate_page_indices,
                   pa_kv_quantize_fp8, pa_kv_quantize_fp8_per_head, pa_kv_quantize_int8, pa_plan_splits, pa_version,
                   PlanInfo)
from .decode import PagedDecode  # noqa: F401
