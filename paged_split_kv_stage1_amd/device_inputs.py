"""Puts a synthetic workload on the GPU in the layouts the kernels read.

bf16 caches are uploaded as they are; FP8 / INT8 caches and FP8 queries are produced
on the device by the library's own quantisers.  Slots that hold no
token (the tail of each request's last page) are then overwritten with NaN bit
patterns, together with their per-token scales, so that any read of them shows.
"""
from __future__ import annotations

import dataclasses
from typing import Optional

import numpy as np
import torch

from ._lib import pa_kv_quantize_fp8, pa_kv_quantize_fp8_per_head, pa_kv_quantize_int8
from .inputs import BF16_NAN_BITS, E4M3_NAN_CODE, INT8_POISON_CODE, Workload


@dataclasses.dataclass
class DeviceInputs:
    q: torch.Tensor                  # bf16 [T, Hq, d] or uint8 codes
    q_scale: Optional[torch.Tensor]  # float32 [1] for FP8 queries ([Hq] with per-head scales)
    k: torch.Tensor                  # bf16 or uint8, layout HPD [pages, Hkv, P, d] or PHD [pages, P, Hkv, d]
    v: torch.Tensor
    k_scale: Optional[torch.Tensor]  # float32 [1] (per tensor), [Hkv] (per head) or [pages, Hkv, P] / [pages, P, Hkv]
    v_scale: Optional[torch.Tensor]
    page_indices: torch.Tensor       # int32
    layout: str
    kv_layout: tuple                 # element strides (page, head, slot)
    scale_layout: Optional[tuple]
    v_layout: Optional[tuple] = None        # value strides when values are narrower than keys
    k_rope: Optional[torch.Tensor] = None   # latent cache: bf16 rotary rows [pages, Hkv, P, 64]
    rope_layout: Optional[tuple] = None
    q_rope: Optional[torch.Tensor] = None   # latent cache: bf16 [T, Hq, 64]


def _strides(layout: str, Hkv: int, P: int, d: int):
    if layout == "HPD":
        return (Hkv * P * d, P * d, d), (Hkv * P, P, 1)
    return (P * Hkv * d, d, Hkv * d), (P * Hkv, 1, Hkv)


def _quantize_heads(src_bf16: torch.Tensor, head_axis: int, device):
    """Per-head codes and scales [H] of a tensor whose head axis is ``head_axis``: the
    quantiser takes token-major rows [tokens, H, d], so other layouts go through a
    transposed copy."""
    x = src_bf16.movedim(head_axis, -2).contiguous()
    H, d = x.shape[-2], x.shape[-1]
    codes = torch.empty(x.shape, dtype=torch.uint8, device=device)
    scale = torch.empty(H, dtype=torch.float32, device=device)
    pa_kv_quantize_fp8_per_head(x, "bf16", x.numel() // (H * d), H, d, codes, scale)
    return codes.movedim(-2, head_axis).contiguous(), scale


def _quantize(src_bf16: torch.Tensor, mode: str, d: int, device, int8: bool = False):
    """FP8 (or INT8) codes, as bytes, and the scales of a bf16 tensor of rows of d."""
    n_rows = src_bf16.numel() // d
    codes = torch.empty(src_bf16.shape, dtype=torch.uint8, device=device)
    scale = torch.empty(1 if mode == "per_tensor" else n_rows, dtype=torch.float32, device=device)
    (pa_kv_quantize_int8 if int8 else pa_kv_quantize_fp8)(src_bf16, "bf16", n_rows, d, mode, codes, scale)
    if mode == "per_token_head":
        scale = scale.view(src_bf16.shape[:-1])
    return codes, scale


def _to_device_rope(w: Workload, device) -> DeviceInputs:
    """Keys wider than values ([pages, Hkv, P, d] layout): bf16 192/128 caches, or the
    MLA-style latent cache (latent codes with a scale per (token, 128 channels) from the
    library's quantiser over 128-channel rows, bf16 rotary rows; queries likewise)."""
    d, dv, P, Hkv = w.head_dim, w.dv, w.page_size, w.num_kv_heads
    unused = torch.from_numpy(w.unused_slots).to(device)
    m4 = unused[:, None, :, None]
    if not w.latent:
        k = w.k.to(device)
        v = w.v.to(device)
        k.view(torch.int16).masked_fill_(m4.expand(k.shape), BF16_NAN_BITS)
        v.view(torch.int16).masked_fill_(m4.expand(v.shape), BF16_NAN_BITS)
        return DeviceInputs(q=w.q.to(device), q_scale=None, k=k, v=v, k_scale=None, v_scale=None,
                            page_indices=torch.from_numpy(np.ascontiguousarray(w.page_indices)).to(device),
                            layout="HPD", kv_layout=(Hkv * P * d, P * d, d), scale_layout=None,
                            v_layout=(Hkv * P * dv, P * dv, dv))
    src = w.k.to(device)
    lat = src[..., :dv].contiguous()
    codes, scale = _quantize(lat.view(*lat.shape[:-1], dv // 128, 128), "per_token_head", 128, device)
    codes = codes.view(lat.shape)
    rope = src[..., dv:].contiguous()
    codes.masked_fill_(m4.expand(codes.shape), E4M3_NAN_CODE)
    scale.masked_fill_(m4.expand(scale.shape), float("nan"))
    rope.view(torch.int16).masked_fill_(m4.expand(rope.shape), BF16_NAN_BITS)
    qsrc = w.q.to(device)
    qn = qsrc[..., :dv].contiguous()
    qc, qs = _quantize(qn.view(*qn.shape[:-1], dv // 128, 128), "per_token_head", 128, device)
    dr = d - dv
    return DeviceInputs(q=qc.view(qn.shape), q_scale=qs, k=codes, v=None, k_scale=scale, v_scale=None,
                        page_indices=torch.from_numpy(np.ascontiguousarray(w.page_indices)).to(device),
                        layout="HPD", kv_layout=(Hkv * P * dv, P * dv, dv),
                        scale_layout=(Hkv * P * (dv // 128), P * (dv // 128), dv // 128),
                        k_rope=rope, rope_layout=(Hkv * P * dr, P * dr, dr), q_rope=qsrc[..., dv:].contiguous())


def to_device(w: Workload, device="cuda", layout: str = "HPD") -> DeviceInputs:
    if w.dv != w.head_dim:
        assert layout == "HPD", "keys wider than values: [pages, Hkv, P, d] caches"
        return _to_device_rope(w, device)
    d, P, Hkv = w.head_dim, w.page_size, w.num_kv_heads
    kv_layout, sc_layout = _strides(layout, Hkv, P, d)
    k_src, v_src = w.k, w.v
    if layout == "PHD":
        k_src = k_src.permute(0, 2, 1, 3).contiguous()
        v_src = v_src.permute(0, 2, 1, 3).contiguous()
    unused = torch.from_numpy(w.unused_slots).to(device)
    m4 = unused[:, None, :, None] if layout == "HPD" else unused[:, :, None, None]
    m3 = unused[:, None, :] if layout == "HPD" else unused[:, :, None]
    k_scale = v_scale = None
    if w.kv_dtype == "bf16":
        k = k_src.to(device)
        v = v_src.to(device)
        k.view(torch.int16).masked_fill_(m4.expand(k.shape), BF16_NAN_BITS)
        v.view(torch.int16).masked_fill_(m4.expand(v.shape), BF16_NAN_BITS)
    elif w.kv_dtype == "int8":
        k, k_scale = _quantize(k_src.to(device), w.kv_scale_mode, d, device, int8=True)
        v, v_scale = _quantize(v_src.to(device), w.kv_scale_mode, d, device, int8=True)
        k.masked_fill_(m4.expand(k.shape), INT8_POISON_CODE)
        v.masked_fill_(m4.expand(v.shape), INT8_POISON_CODE)
        if w.kv_scale_mode == "per_token_head":
            k_scale.masked_fill_(m3.expand(k_scale.shape), float("nan"))
            v_scale.masked_fill_(m3.expand(v_scale.shape), float("nan"))
    elif w.kv_scale_mode == "per_head":
        axis = 1 if layout == "HPD" else 2
        k, k_scale = _quantize_heads(k_src.to(device), axis, device)
        v, v_scale = _quantize_heads(v_src.to(device), axis, device)
        k.masked_fill_(m4.expand(k.shape), E4M3_NAN_CODE)
        v.masked_fill_(m4.expand(v.shape), E4M3_NAN_CODE)
    else:
        k, k_scale = _quantize(k_src.to(device), w.kv_scale_mode, d, device)
        v, v_scale = _quantize(v_src.to(device), w.kv_scale_mode, d, device)
        k.masked_fill_(m4.expand(k.shape), E4M3_NAN_CODE)
        v.masked_fill_(m4.expand(v.shape), E4M3_NAN_CODE)
        if w.kv_scale_mode == "per_token_head":
            k_scale.masked_fill_(m3.expand(k_scale.shape), float("nan"))
            v_scale.masked_fill_(m3.expand(v_scale.shape), float("nan"))
    q_scale = None
    if w.q_dtype == "fp8" and w.kv_scale_mode == "per_head":
        q, q_scale = _quantize_heads(w.q.to(device), 1, device)     # one scale per query head
    elif w.q_dtype == "fp8":
        q, q_scale = _quantize(w.q.to(device), "per_tensor", d, device)
    else:
        q = w.q.to(device)
    return DeviceInputs(q=q, q_scale=q_scale, k=k, v=v, k_scale=k_scale, v_scale=v_scale,
                        page_indices=torch.from_numpy(np.ascontiguousarray(w.page_indices)).to(device),
                        layout=layout, kv_layout=kv_layout,
                        scale_layout=sc_layout if w.kv_scale_mode == "per_token_head" else None)
