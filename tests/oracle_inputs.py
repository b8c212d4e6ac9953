"""Oracle-side view of a synthetic workload (CPU, numpy): quantised with the
oracle's own quantiser and poisoned exactly like the device copy."""
import numpy as np
import torch

from oracle.attention import LatentKV, PagedKV, dequant_q, dequant_q_latent
from oracle.quantize import (quantize_int8_per_row, quantize_int8_per_tensor, quantize_per_head, quantize_per_row,
                             quantize_per_tensor)
from paged_split_kv_stage1_amd.inputs import BF16_NAN_BITS, E4M3_NAN_CODE, INT8_POISON_CODE


def _bits(t: torch.Tensor) -> np.ndarray:
    return t.view(torch.int16).numpy().astype(np.uint16)


def oracle_inputs(w, layout="HPD", requests=None):
    """Returns dict(q64, k, v, q_codes, q_scale) for the oracle.  With ``requests``
    given (per-token-head scales only), only those requests' pages are quantised."""
    k_src, v_src = w.k, w.v
    unused = w.unused_slots
    if layout == "PHD":
        k_src = k_src.permute(0, 2, 1, 3).contiguous()
        v_src = v_src.permute(0, 2, 1, 3).contiguous()
    kb, vb = _bits(k_src), _bits(v_src)
    m4 = unused[:, None, :, None] if layout == "HPD" else unused[:, :, None, None]
    m3 = unused[:, None, :] if layout == "HPD" else unused[:, :, None]
    out = {}
    if w.latent:
        # MLA-style latent cache: latent channels quantised per (token, 128 channels), the
        # rotary channels kept in bf16; queries the same way
        dv = w.dv
        assert layout == "HPD"
        lat = kb[..., :dv]
        codes, scale = quantize_per_row(np.ascontiguousarray(lat).reshape(*lat.shape[:-1], dv // 128, 128), "bf16")
        codes = codes.reshape(lat.shape)
        rope = np.ascontiguousarray(kb[..., dv:])
        codes = np.where(np.broadcast_to(m4, codes.shape), np.uint8(E4M3_NAN_CODE), codes)
        scale = np.where(np.broadcast_to(m4, scale.shape), np.float32(np.nan), scale)
        rope = np.where(np.broadcast_to(m4, rope.shape), np.uint16(BF16_NAN_BITS), rope)
        lkv = LatentKV(codes, scale, rope)
        out["latent"], out["k"], out["v"] = lkv, lkv.key_view(), lkv.value_view()
        qb = _bits(w.q)
        qn = np.ascontiguousarray(qb[..., :dv])
        qc, qs = quantize_per_row(qn.reshape(*qn.shape[:-1], dv // 128, 128), "bf16")
        out["q_codes"], out["q_scale"], out["q_rope"] = qc.reshape(qn.shape), qs, np.ascontiguousarray(qb[..., dv:])
        out["q64"] = dequant_q_latent(out["q_codes"], qs, out["q_rope"])
        return out
    if w.kv_dtype == "bf16":
        kb = np.where(np.broadcast_to(m4, kb.shape), np.uint16(BF16_NAN_BITS), kb)
        vb = np.where(np.broadcast_to(m4, vb.shape), np.uint16(BF16_NAN_BITS), vb)
        out["k"] = PagedKV(kb, "bf16", layout)
        out["v"] = PagedKV(vb, "bf16", layout)
    elif w.kv_dtype == "int8":
        if w.kv_scale_mode == "per_tensor":
            kc, ks = quantize_int8_per_tensor(kb, "bf16")
            vc, vs = quantize_int8_per_tensor(vb, "bf16")
        else:
            pages = (np.concatenate([w.page_indices[w.kv_indptr[b]:w.kv_indptr[b + 1]] for b in requests])
                     if requests is not None else np.arange(kb.shape[0]))
            kc = np.zeros(kb.shape, np.int8); vc = np.zeros(vb.shape, np.int8)
            ks = np.zeros(kb.shape[:-1], np.float32); vs = np.zeros(vb.shape[:-1], np.float32)
            kc[pages], ks[pages] = quantize_int8_per_row(kb[pages], "bf16")
            vc[pages], vs[pages] = quantize_int8_per_row(vb[pages], "bf16")
            ks = np.where(m3, np.float32(np.nan), ks)
            vs = np.where(m3, np.float32(np.nan), vs)
        kc = np.where(np.broadcast_to(m4, kc.shape), np.uint8(INT8_POISON_CODE), kc.view(np.uint8))
        vc = np.where(np.broadcast_to(m4, vc.shape), np.uint8(INT8_POISON_CODE), vc.view(np.uint8))
        out["k"] = PagedKV(kc, "int8", layout, w.kv_scale_mode, ks)
        out["v"] = PagedKV(vc, "int8", layout, w.kv_scale_mode, vs)
    elif w.kv_scale_mode == "per_tensor":
        kc, ks = quantize_per_tensor(kb, "bf16")
        vc, vs = quantize_per_tensor(vb, "bf16")
        kc = np.where(np.broadcast_to(m4, kc.shape), np.uint8(E4M3_NAN_CODE), kc)
        vc = np.where(np.broadcast_to(m4, vc.shape), np.uint8(E4M3_NAN_CODE), vc)
        out["k"] = PagedKV(kc, "fp8", layout, "per_tensor", ks)
        out["v"] = PagedKV(vc, "fp8", layout, "per_tensor", vs)
    elif w.kv_scale_mode == "per_head":
        axis = 1 if layout == "HPD" else 2
        kc, ks = quantize_per_head(kb, "bf16", axis)
        vc, vs = quantize_per_head(vb, "bf16", axis)
        kc = np.where(np.broadcast_to(m4, kc.shape), np.uint8(E4M3_NAN_CODE), kc)
        vc = np.where(np.broadcast_to(m4, vc.shape), np.uint8(E4M3_NAN_CODE), vc)
        out["k"] = PagedKV(kc, "fp8", layout, "per_head", ks)
        out["v"] = PagedKV(vc, "fp8", layout, "per_head", vs)
    else:
        if requests is not None:
            pages = np.concatenate([w.page_indices[w.kv_indptr[b]:w.kv_indptr[b + 1]] for b in requests])
        else:
            pages = np.arange(kb.shape[0])
        kc = np.zeros(kb.shape, np.uint8); vc = np.zeros(vb.shape, np.uint8)
        ks = np.zeros(kb.shape[:-1], np.float32); vs = np.zeros(vb.shape[:-1], np.float32)
        kc[pages], ks[pages] = quantize_per_row(kb[pages], "bf16")
        vc[pages], vs[pages] = quantize_per_row(vb[pages], "bf16")
        kc = np.where(np.broadcast_to(m4, kc.shape), np.uint8(E4M3_NAN_CODE), kc)
        vc = np.where(np.broadcast_to(m4, vc.shape), np.uint8(E4M3_NAN_CODE), vc)
        ks = np.where(m3, np.float32(np.nan), ks)
        vs = np.where(m3, np.float32(np.nan), vs)
        out["k"] = PagedKV(kc, "fp8", layout, "per_token_head", ks)
        out["v"] = PagedKV(vc, "fp8", layout, "per_token_head", vs)
    qb = _bits(w.q)
    if w.q_dtype == "fp8":
        if w.kv_scale_mode == "per_head":
            qc, qs = quantize_per_head(qb, "bf16", 1)          # one scale per query head
        else:
            qc, qs = quantize_per_tensor(qb, "bf16")
        out["q_codes"], out["q_scale"] = qc, qs
        out["q64"] = dequant_q(qc, "fp8", qs)
    else:
        out["q64"] = dequant_q(qb, "bf16")
    return out


def max_rel_err(o: np.ndarray, r: np.ndarray) -> float:
    """max over (row, head) of ||o - r||_inf / ||r||_inf."""
    num = np.max(np.abs(o - r), axis=-1)
    den = np.max(np.abs(r), axis=-1)
    return float(np.max(num / den))
