"""Appending new tokens' K and V to the paged cache -- oracle, test infrastructure.

What is computed: a serving step writes the keys and values of the tokens it adds
into the paged cache before decode attention reads them.  With the per-token-head
FP8 KV cache (FreeToken PR #900, end-to-end table row "fp8_per_token_head") every
(token, KV head) row is quantised with its own scale as it is written; with a
per-tensor FP8 cache the rows are encoded with the cache's given scale (FlashMLA
PR #54, symmetric per-tensor scales) or with its head's given scale (per-head scales,
FlashInfer PR #869).

Readings where the pages are silent:
  * token t goes to physical slot slot_mapping[t] = page * P + slot, the slot that
    the decode page table addresses (token j of a request lives in page
    page_indices[kv_indptr[b] + j // P] at slot j % P); a negative slot skips the
    token (padding);
  * a bf16 cache stores bf16 sources unchanged and float32 sources rounded to the
    nearest bf16 (ties to even);
  * FP8 and INT8 codes follow oracle.quantize (RNE of the clamped fp32 quotient).
"""
from __future__ import annotations

import numpy as np

from .formats import f32_to_bf16_bits_rne
from .quantize import _as_f32, _encode, _encode_int8, quantize_int8_per_row, quantize_per_row


def _row_view(cache: np.ndarray, layout: str, page: int, head: int, slot: int):
    """Index tuple of cache element row (page, KV head, slot, :) for HPD
    ([pages, Hkv, P, d]) or PHD ([pages, P, Hkv, d]) caches."""
    return (page, head, slot) if layout == "HPD" else (page, slot, head)


def append_kv(cache: np.ndarray, scales, rows: np.ndarray, src_dtype: str, slot_mapping,
              page_size: int, kind: str, layout: str = "HPD", tensor_scale=None):
    """Writes rows [n, Hkv, d] (bf16 bit patterns or float32) into a copy of ``cache``
    and returns (cache, scales).

    kind: "bf16" (cache holds bf16 bit patterns), "fp8_per_tensor" (codes, encoded with
    ``tensor_scale``), "fp8_per_head" (codes, KV head h encoded with
    ``tensor_scale[h]``), "fp8_per_token_head" (codes, and ``scales`` [pages, Hkv, P]
    or [pages, P, Hkv] receives each row's scale), "int8_per_tensor" and
    "int8_per_token_head" (the same with int8 codes; the cache holds their bytes)."""
    cache = cache.copy()
    scales = None if scales is None else scales.copy()
    n, hkv, _ = rows.shape
    x32 = _as_f32(rows, src_dtype)
    for t in range(n):
        s = int(slot_mapping[t])
        if s < 0:
            continue
        page, slot = s // page_size, s % page_size
        for h in range(hkv):
            idx = _row_view(cache, layout, page, h, slot)
            if kind == "bf16":
                cache[idx] = rows[t, h] if src_dtype == "bf16" else f32_to_bf16_bits_rne(x32[t, h])
            elif kind == "fp8_per_tensor":
                cache[idx] = _encode(x32[t, h], np.float32(tensor_scale))
            elif kind == "fp8_per_head":
                cache[idx] = _encode(x32[t, h], np.float32(np.asarray(tensor_scale, dtype=np.float32)[h]))
            elif kind == "int8_per_tensor":
                cache[idx] = _encode_int8(x32[t, h], np.float32(tensor_scale)).view(cache.dtype)
            elif kind == "int8_per_token_head":
                codes, sc = quantize_int8_per_row(rows[t, h][None], src_dtype)
                cache[idx] = codes[0].view(cache.dtype)
                scales[idx] = sc[0]
            elif kind == "fp8_per_token_head":
                codes, sc = quantize_per_row(rows[t, h][None], src_dtype)
                cache[idx] = codes[0]
                scales[idx] = sc[0]
            else:
                raise ValueError(kind)
    return cache, scales
