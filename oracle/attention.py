"""Paged split-KV decode attention in float64 -- oracle, test infrastructure.

What is computed (FreeToken PR #900, "Changes", first item; hpc-ops issue #4 for
the paged, block-size-64 FP8 decode it extends):
  * a request b owns n_b = qo_indptr[b+1] - qo_indptr[b] query rows (at most 8)
    and kv_len[b] cached tokens, the last n_b of which are the new rows' own keys;
  * each row is limited to its own position and to its window;
  * query head h reads KV head h // G with G = Hq / Hkv (grouped-query attention; the
    same PR makes the query heads of one program lie inside a single GQA group);
  * the output is softmax(sm_scale * q K^T) V over the visible tokens, with the
    K/V values dequantised first (FP8 dequantisation folded into the scores and
    into the final normaliser is the same arithmetic, FlashInfer PR #869 item 3);
  * split-KV: stage 1 produces, per KV split, the normalised partial output and
    its log-sum-exp; stage 2 merges the splits of each row;
  * keys and values may have different widths (FlashInfer PR #869, "Remaining Work":
    separate head_dim_qk and head_dim_v): the scores use the key width, the output has
    the value width; the MLA-style latent cache (LatentKV) is one such case.

Readings (where the pages are silent):
  * row r of request b sits at position p = kv_len - n_b + r;
  * a window W > 0 keeps keys j with p - W + 1 <= j <= p (W keys including self);
    W = 0 means no window;
  * the page table is a CSR: request b's pages are
    page_indices[kv_indptr[b] : kv_indptr[b+1]] and logical token t lives in
    page page_indices[kv_indptr[b] + t // P] at slot t % P;
  * LSE uses the natural logarithm of the scaled scores; an empty split has
    LSE = -inf and a zero partial output.
"""
from __future__ import annotations

import dataclasses
from typing import Iterable, Optional, Sequence

import numpy as np

from .formats import bf16_bits_to_f64, e4m3_code_to_f64


def gather_slots(kv_indptr, page_indices, kv_len, page_size: int, b: int) -> np.ndarray:
    """Physical token index page * P + slot of every logical token of request b
    (int64, length kv_len[b]).  This is the page-gather the GPU must match bit-exactly."""
    L = int(kv_len[b])
    t = np.arange(L, dtype=np.int64)
    pages = np.asarray(page_indices, dtype=np.int64)[int(kv_indptr[b]) + t // page_size]
    return pages * page_size + t % page_size


def visible_range(kv_len_b: int, n_rows_b: int, r: int, window_b: int):
    """Inclusive [lo, p] of keys that row r of a request may attend to."""
    p = int(kv_len_b) - int(n_rows_b) + int(r)
    lo = max(0, p - int(window_b) + 1) if window_b > 0 else 0
    return lo, p


@dataclasses.dataclass
class PagedKV:
    """One paged cache (K or V) as the GPU stores it.

    data: bf16 bit patterns (uint16), e4m3 codes (uint8) or int8 codes (int8 or their
          bytes as uint8), shape
          [pages, Hkv, P, d] for layout "HPD" or [pages, P, Hkv, d] for "PHD".
    scale: None; a float32 scalar (per tensor); float32 [Hkv] (per head); or float32
           [pages, Hkv, P] ("HPD") / [pages, P, Hkv] ("PHD") for per-(token, KV head)
           scales.
    """
    data: np.ndarray
    dtype: str
    layout: str = "HPD"
    scale_mode: str = "none"
    scale: Optional[object] = None

    @property
    def page_size(self) -> int:
        return self.data.shape[2] if self.layout == "HPD" else self.data.shape[1]

    def tokens(self, slots: np.ndarray, g: int) -> np.ndarray:
        """Dequantised float64 [len(slots), d] values of KV head g at physical slots."""
        P = self.page_size
        page, slot = slots // P, slots % P
        if self.layout == "HPD":
            raw = self.data[page, g, slot, :]
        else:
            raw = self.data[page, slot, g, :]
        if self.dtype == "bf16":
            val = bf16_bits_to_f64(raw)
        elif self.dtype == "fp8":
            val = e4m3_code_to_f64(raw)
        elif self.dtype == "int8":
            val = np.asarray(raw).view(np.int8).astype(np.float64)
        else:
            raise ValueError(self.dtype)
        if self.scale_mode == "per_tensor":
            val = val * np.float64(np.float32(self.scale))
        elif self.scale_mode == "per_head":
            val = val * np.float64(np.asarray(self.scale, dtype=np.float32)[g])
        elif self.scale_mode == "per_token_head":
            sc = self.scale[page, g, slot] if self.layout == "HPD" else self.scale[page, slot, g]
            val = val * np.asarray(sc, dtype=np.float32).astype(np.float64)[:, None]
        return val


@dataclasses.dataclass
class LatentKV:
    """MLA-style paged cache (FlashMLA PR #54, review thread: the no-position ("nope")
    part in 8 bits with one scale per token and 128 channels, the rotary part kept in
    16 bits): per (page, KV head, slot) a latent row of e4m3 codes with one float32 scale
    per 128 channels, plus a bf16 rotary row.  The key is [latent, rotary] and the value
    is the latent alone (the absorbed form of multi-head latent attention).

    codes: uint8 [pages, Hkv, P, dv]; scale: float32 [pages, Hkv, P, dv / 128];
    rope: bf16 bits [pages, Hkv, P, dr]."""
    codes: np.ndarray
    scale: np.ndarray
    rope: np.ndarray

    def latent(self, slots: np.ndarray, g: int) -> np.ndarray:
        """Dequantised float64 [len(slots), dv]: code times its 128-channel block's scale."""
        P = self.codes.shape[2]
        page, slot = slots // P, slots % P
        codes = e4m3_code_to_f64(self.codes[page, g, slot, :])
        sc = np.asarray(self.scale[page, g, slot, :], dtype=np.float32).astype(np.float64)
        return (codes.reshape(len(slots), -1, 128) * sc[:, :, None]).reshape(len(slots), -1)

    def key_view(self):
        return _LatentView(self, with_rope=True)

    def value_view(self):
        return _LatentView(self, with_rope=False)


class _LatentView:
    """Key ([latent, rotary]) or value (latent) side of a LatentKV, with the interface of
    PagedKV that decode_attention uses (tokens, data shape [pages, Hkv, P, ...], page_size)."""

    def __init__(self, kv: LatentKV, with_rope: bool):
        self.kv, self.with_rope = kv, with_rope
        self.data, self.layout = kv.codes, "HPD"

    @property
    def page_size(self) -> int:
        return self.kv.codes.shape[2]

    def tokens(self, slots: np.ndarray, g: int) -> np.ndarray:
        lat = self.kv.latent(slots, g)
        if not self.with_rope:
            return lat
        P = self.page_size
        rope = bf16_bits_to_f64(self.kv.rope[slots // P, g, slots % P, :])
        return np.concatenate([lat, rope], axis=1)


def dequant_q_latent(codes: np.ndarray, scale: np.ndarray, rope_bits: np.ndarray) -> np.ndarray:
    """MLA query [T, Hq, dv + dr] in float64: e4m3 codes [T, Hq, dv] times the scale of
    their 128-channel block ([T, Hq, dv / 128]), followed by the bf16 rotary part."""
    T, H, dv = codes.shape
    lat = e4m3_code_to_f64(codes).reshape(T, H, dv // 128, 128) * \
        np.asarray(scale, dtype=np.float32).astype(np.float64)[..., None]
    return np.concatenate([lat.reshape(T, H, dv), bf16_bits_to_f64(rope_bits)], axis=2)


def dequant_q(q_raw: np.ndarray, q_dtype: str, q_scale=None) -> np.ndarray:
    """Query [T, Hq, d] -> float64: bf16 bits, or e4m3 codes times a per-tensor scale
    (a scalar) or per-query-head scales ([Hq])."""
    if q_dtype == "bf16":
        return bf16_bits_to_f64(q_raw)
    if q_dtype == "fp8":
        qs = np.asarray(q_scale, dtype=np.float32).astype(np.float64)
        if qs.ndim == 1:
            qs = qs[None, :, None]
        return e4m3_code_to_f64(q_raw) * qs
    raise ValueError(q_dtype)


def attend(q_rows: np.ndarray, k: np.ndarray, v: np.ndarray, sm_scale: float):
    """softmax(sm_scale * q k^T) v for q_rows [m, d] against k, v [n, d] (n >= 1).
    Returns (o [m, d], lse [m]) in float64; lse = natural log-sum-exp of the scores."""
    s = np.float64(sm_scale) * (q_rows @ k.T)
    m = np.max(s, axis=1, keepdims=True)
    e = np.exp(s - m)
    l = np.sum(e, axis=1, keepdims=True)
    o = (e @ v) / l
    return o, (m + np.log(l))[:, 0]


def decode_attention(q64: np.ndarray, kc: PagedKV, vc: PagedKV, page_indices, kv_indptr, kv_len,
                     qo_indptr, window, sm_scale: float, requests: Optional[Iterable[int]] = None):
    """Full decode attention.  q64: float64 [T, Hq, d].  Returns (out [T, Hq, d], lse [T, Hq])
    float64; rows of requests not listed in ``requests`` are left as NaN."""
    T, Hq, d = q64.shape
    Hkv = kc.data.shape[1] if kc.layout == "HPD" else kc.data.shape[2]
    G = Hq // Hkv
    P = kc.page_size
    dv = vc.data.shape[-1]                     # value width (may differ from the key width d)
    out = np.full((T, Hq, dv), np.nan)
    lse = np.full((T, Hq), np.nan)
    B = len(kv_len)
    window = np.zeros(B, dtype=np.int64) if window is None else window
    for b in (range(B) if requests is None else requests):
        slots = gather_slots(kv_indptr, page_indices, kv_len, P, b)
        t0, n = int(qo_indptr[b]), int(qo_indptr[b + 1] - qo_indptr[b])
        for g in range(Hkv):
            K = kc.tokens(slots, g)
            V = vc.tokens(slots, g)
            for r in range(n):
                lo, p = visible_range(kv_len[b], n, r, int(window[b]))
                heads = slice(g * G, (g + 1) * G)
                o, l = attend(q64[t0 + r, heads, :], K[lo:p + 1], V[lo:p + 1], sm_scale)
                out[t0 + r, heads, :] = o
                lse[t0 + r, heads] = l
    return out, lse


def decode_attention_one(q64_vec: np.ndarray, kc: PagedKV, vc: PagedKV, page_indices, kv_indptr,
                         kv_len, qo_indptr, window, sm_scale: float, t: int, h: int, num_kv_heads: int,
                         num_q_heads: int):
    """One output vector (row t, query head h), for sampled checks at full size."""
    b = int(np.searchsorted(np.asarray(qo_indptr), t, side="right") - 1)
    n = int(qo_indptr[b + 1] - qo_indptr[b])
    r = t - int(qo_indptr[b])
    g = h // (num_q_heads // num_kv_heads)
    w = 0 if window is None else int(window[b])
    lo, p = visible_range(kv_len[b], n, r, w)
    slots = gather_slots(kv_indptr, page_indices, kv_len, kc.page_size, b)[lo:p + 1]
    o, l = attend(q64_vec[None, :], kc.tokens(slots, g), vc.tokens(slots, g), sm_scale)
    return o[0], l[0]


def split_partials(q64: np.ndarray, kc: PagedKV, vc: PagedKV, page_indices, kv_indptr, kv_len,
                   qo_indptr, window, sm_scale: float, b: int, splits: Sequence[tuple]):
    """Stage-1 quantities of request b for KV splits given as token ranges [a, e).
    Returns (o [n_rows, Hq, S, d], lse [n_rows, Hq, S]); an empty intersection of a
    split with a row's visible range gives o = 0, lse = -inf."""
    T, Hq, d = q64.shape
    Hkv = kc.data.shape[1] if kc.layout == "HPD" else kc.data.shape[2]
    G = Hq // Hkv
    slots = gather_slots(kv_indptr, page_indices, kv_len, kc.page_size, b)
    t0, n = int(qo_indptr[b]), int(qo_indptr[b + 1] - qo_indptr[b])
    S = len(splits)
    o_out = np.zeros((n, Hq, S, vc.data.shape[-1]))
    l_out = np.full((n, Hq, S), -np.inf)
    w = 0 if window is None else int(window[b])
    for g in range(Hkv):
        K = kc.tokens(slots, g)
        V = vc.tokens(slots, g)
        for r in range(n):
            lo, p = visible_range(kv_len[b], n, r, w)
            heads = slice(g * G, (g + 1) * G)
            for s, (a, e) in enumerate(splits):
                j0, j1 = max(lo, a), min(p + 1, e)
                if j1 <= j0:
                    continue
                o, l = attend(q64[t0 + r, heads, :], K[j0:j1], V[j0:j1], sm_scale)
                o_out[r, heads, s, :] = o
                l_out[r, heads, s] = l
    return o_out, l_out


def merge_partials(o_parts: np.ndarray, lse_parts: np.ndarray):
    """Stage-2 merge over the split axis (second to last of o, last of lse):
    out = sum_s e^{lse_s - M} o_s / sum_s e^{lse_s - M}, M = max_s lse_s;
    merged lse = M + ln sum_s e^{lse_s - M}."""
    M = np.max(lse_parts, axis=-1, keepdims=True)
    w = np.exp(lse_parts - M)
    w = np.where(np.isneginf(lse_parts), 0.0, w)
    den = np.sum(w, axis=-1, keepdims=True)
    out = np.sum(w[..., None] * o_parts, axis=-2) / den
    return out, (M + np.log(den))[..., 0]
