"""FP8 (E4M3FN) quantisation of K/V (and per-tensor Q) -- oracle, test infrastructure.

What the pages fix:
  * symmetric per-tensor scales for Q/K/V (FlashMLA PR #54, "Functionality");
  * a per-token-head FP8 KV cache, i.e. one scale per (token, KV head)
    (FreeToken PR #900, end-to-end table row "fp8_per_token_head");
  * per-head scales, one per head over all of that head's values (FlashInfer PR
    #869, title: per-head quantization);
  * scale = amax / 448 over the quantised group (the workloads' statement).
Readings where the pages are silent: the scale is computed in float32 as
fl32(amax / 448); a value is encoded as RNE_e4m3(clamp(fl32(x / scale), -448, 448))
with an IEEE float32 division; a group whose amax is 0 gets scale 1 (all codes 0).

INT8 codes (the pages name int8 KV caches -- FreeToken PR #900, "Tested on", the
register-spill check over bf16/fp8/int8 kernels -- but define no format): symmetric,
scale = fl32(amax / 127) (1 when amax is 0), code = round-half-even(clamp(fl32(x /
scale), -127, 127)) as a signed byte, value = code * scale; per (token, KV head) or per
tensor, like the FP8 scales.

Inputs are rows of d values (bf16 bit patterns, or float32); for per-token-head
scales a row is one (token, KV head) vector, for per-tensor scales all rows share
one scale, for per-head scales all rows of one head share one.
"""
from __future__ import annotations

import numpy as np

from .formats import E4M3_MAX, bf16_bits_to_f64, f64_to_e4m3_rne


def _as_f32(src: np.ndarray, src_dtype: str) -> np.ndarray:
    if src_dtype == "bf16":
        return bf16_bits_to_f64(src).astype(np.float32)      # exact
    if src_dtype == "fp32":
        return np.asarray(src, dtype=np.float32)
    raise ValueError(src_dtype)


def _encode(x32: np.ndarray, scale32: np.ndarray) -> np.ndarray:
    q = (x32 / scale32).astype(np.float32)                     # IEEE fp32 divide, RNE
    q = np.clip(q.astype(np.float64), -E4M3_MAX, E4M3_MAX)
    return f64_to_e4m3_rne(q)


def _scale_from_amax(amax32: np.ndarray) -> np.ndarray:
    amax32 = np.asarray(amax32, dtype=np.float32)
    s = (amax32 / np.float32(E4M3_MAX)).astype(np.float32)
    return np.where(amax32 == 0, np.float32(1.0), s).astype(np.float32)


def quantize_per_tensor(src: np.ndarray, src_dtype: str):
    """Returns (codes uint8 with src's shape, scale float32 scalar)."""
    x = _as_f32(src, src_dtype)
    amax = np.float32(np.max(np.abs(x))) if x.size else np.float32(0)
    scale = _scale_from_amax(amax)
    return _encode(x, scale), np.float32(scale)


def quantize_per_row(src: np.ndarray, src_dtype: str):
    """Per-(token, KV head) scales: src [..., d]; one scale per leading index.
    Returns (codes uint8 [..., d], scales float32 [...])."""
    x = _as_f32(src, src_dtype)
    amax = np.max(np.abs(x), axis=-1).astype(np.float32)
    scale = _scale_from_amax(amax)
    return _encode(x, scale[..., None]), scale


def quantize_per_head(src: np.ndarray, src_dtype: str, head_axis: int):
    """Per-head scales: one scale per index of ``head_axis`` over every value of that
    head (all tokens and all d).  Returns (codes uint8 with src's shape, scales
    float32 [H])."""
    x = _as_f32(src, src_dtype)
    xh = np.moveaxis(x, head_axis, 0)
    amax = np.max(np.abs(xh.reshape(xh.shape[0], -1)), axis=1).astype(np.float32) if x.size else \
        np.zeros(x.shape[head_axis], np.float32)
    scale = _scale_from_amax(amax)
    shape = [1] * x.ndim
    shape[head_axis] = -1
    return _encode(x, scale.reshape(shape)), scale


INT8_MAX = 127.0


def _encode_int8(x32: np.ndarray, scale32: np.ndarray) -> np.ndarray:
    q = (x32 / scale32).astype(np.float32)                     # IEEE fp32 divide, RNE
    q = np.clip(q.astype(np.float64), -INT8_MAX, INT8_MAX)
    return np.rint(q).astype(np.int8)                          # ties to even


def _int8_scale_from_amax(amax32: np.ndarray) -> np.ndarray:
    amax32 = np.asarray(amax32, dtype=np.float32)
    s = (amax32 / np.float32(INT8_MAX)).astype(np.float32)
    return np.where(amax32 == 0, np.float32(1.0), s).astype(np.float32)


def quantize_int8_per_row(src: np.ndarray, src_dtype: str):
    """INT8 with per-(token, KV head) scales: src [..., d]; one scale per leading index.
    Returns (codes int8 [..., d], scales float32 [...])."""
    x = _as_f32(src, src_dtype)
    scale = _int8_scale_from_amax(np.max(np.abs(x), axis=-1).astype(np.float32))
    return _encode_int8(x, scale[..., None]), scale


def quantize_int8_per_tensor(src: np.ndarray, src_dtype: str):
    """INT8 with one scale for the whole tensor.  Returns (codes int8, scale float32)."""
    x = _as_f32(src, src_dtype)
    amax = np.float32(np.max(np.abs(x))) if x.size else np.float32(0)
    scale = _int8_scale_from_amax(amax)
    return _encode_int8(x, scale), np.float32(scale)
