"""ctypes binding of the C ABI in include/pa.h (argument marshalling only).

The functions keep the C names.  Tensor arguments may be torch tensors (their
data_ptr() is passed), plain integers (device addresses) or None (NULL).  Every
non-zero status raises PaError with the library's message.  The library is never
emulated: if libpa_gfx950.so is missing, calls raise instead of falling back.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libpa_gfx950.so")

PA_OK, PA_ERR_INVALID_ARGUMENT, PA_ERR_UNSUPPORTED, PA_ERR_INSUFFICIENT_WORKSPACE, PA_ERR_HIP = range(5)
PA_DTYPE_BF16, PA_DTYPE_FP32, PA_DTYPE_FP8_E4M3, PA_DTYPE_INT8 = 0, 1, 2, 3
PA_SCALE_NONE, PA_SCALE_PER_TENSOR, PA_SCALE_PER_TOKEN_HEAD, PA_SCALE_PER_HEAD, PA_SCALE_PER_TOKEN_BLOCK128 = 0, 1, 2, 3, 4

DTYPES = {"bf16": PA_DTYPE_BF16, "fp32": PA_DTYPE_FP32, "fp8": PA_DTYPE_FP8_E4M3, "int8": PA_DTYPE_INT8}
SCALE_MODES = {"none": PA_SCALE_NONE, "per_tensor": PA_SCALE_PER_TENSOR, "per_token_head": PA_SCALE_PER_TOKEN_HEAD,
               "per_head": PA_SCALE_PER_HEAD, "per_token_block128": PA_SCALE_PER_TOKEN_BLOCK128}

_p = ctypes.c_void_p
_i32p = ctypes.POINTER(ctypes.c_int32)


class PlanArgs(ctypes.Structure):
    _fields_ = [("batch", ctypes.c_int32), ("qo_indptr", _i32p), ("kv_indptr", _i32p), ("kv_len", _i32p),
                ("window", _i32p), ("max_q_len", ctypes.c_int32), ("page_size", ctypes.c_int32),
                ("num_q_heads", ctypes.c_int32), ("num_kv_heads", ctypes.c_int32), ("head_dim", ctypes.c_int32),
                ("q_dtype", ctypes.c_int), ("kv_dtype", ctypes.c_int), ("kv_scale_mode", ctypes.c_int),
                ("num_cus", ctypes.c_int32), ("max_splits", ctypes.c_int32), ("force_splits", ctypes.c_int32),
                ("head_dim_v", ctypes.c_int32), ("orientation", ctypes.c_int32)]


PA_ORIENT_KV_ON_M, PA_ORIENT_Q_ON_M = 0, 1
_ORIENT = {"kv_on_m": PA_ORIENT_KV_ON_M, "q_on_m": PA_ORIENT_Q_ON_M}


def _orient(x) -> int:
    return _ORIENT[x] if isinstance(x, str) else int(x)


class PlanInfo(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in
                ("batch", "total_rows", "num_q_heads", "num_kv_heads", "head_dim", "page_size", "max_q_len",
                 "q_dtype", "kv_dtype", "kv_scale_mode", "num_items", "max_splits", "needs_merge", "num_cus",
                 "variant", "head_dim_v")] + \
               [("plan_bytes", ctypes.c_int64), ("partial_o_bytes", ctypes.c_int64),
                ("partial_lse_bytes", ctypes.c_int64), ("max_item_tokens", ctypes.c_int64),
                ("reserved", ctypes.c_int64 * 3)]


class KVLayout(ctypes.Structure):
    _fields_ = [("page", ctypes.c_int64), ("head", ctypes.c_int64), ("slot", ctypes.c_int64)]


class ScaleLayout(ctypes.Structure):
    _fields_ = [("page", ctypes.c_int64), ("head", ctypes.c_int64), ("slot", ctypes.c_int64)]


class PaError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"[pa status {status}] {message}")
        self.status = status


_lib = None


def lib() -> ctypes.CDLL:
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is not built; run paged_split_kv_stage1_amd/build.py "
                               f"(hipcc --offload-arch=gfx950) first")
        L = ctypes.CDLL(LIB_PATH)
        L.pa_plan_splits.argtypes = [ctypes.POINTER(PlanArgs), _p, ctypes.c_size_t, ctypes.POINTER(PlanInfo)]
        L.pa_decode_stage1.argtypes = [ctypes.POINTER(PlanInfo), _p, _p, _p, _p, _p, ctypes.POINTER(KVLayout), _p, _p,
                                       ctypes.POINTER(ScaleLayout), _p, ctypes.c_float, _p, _p, _p, ctypes.c_int, _p,
                                       _p]
        L.pa_decode_stage1_rope.argtypes = [ctypes.POINTER(PlanInfo), _p, _p, _p, _p, _p, ctypes.POINTER(KVLayout),
                                            _p, ctypes.POINTER(KVLayout), _p, ctypes.POINTER(KVLayout), _p,
                                            ctypes.POINTER(KVLayout), _p, ctypes.c_float, _p, _p, _p, ctypes.c_int,
                                            _p, _p]
        L.pa_decode_stage1_rope.restype = ctypes.c_int
        L.pa_decode_merge.argtypes = [ctypes.POINTER(PlanInfo), _p, _p, _p, _p, ctypes.c_int, _p, _p]
        L.pa_kv_quantize_fp8.argtypes = [_p, ctypes.c_int, ctypes.c_int64, ctypes.c_int32, ctypes.c_int, _p, _p, _p]
        L.pa_kv_quantize_int8.argtypes = [_p, ctypes.c_int, ctypes.c_int64, ctypes.c_int32, ctypes.c_int, _p, _p, _p]
        L.pa_kv_quantize_fp8_per_head.argtypes = [_p, ctypes.c_int, ctypes.c_int64, ctypes.c_int32, ctypes.c_int32,
                                                  _p, _p, _p]
        L.pa_kv_append.argtypes = [_p, _p, ctypes.c_int, ctypes.c_int64, ctypes.c_int32, ctypes.c_int32,
                                   ctypes.c_int32, _p, _p, _p, ctypes.c_int, ctypes.c_int, ctypes.POINTER(KVLayout),
                                   _p, _p, ctypes.POINTER(ScaleLayout), _p]
        L.pa_debug_gather.argtypes = [ctypes.POINTER(PlanInfo), _p, _p, ctypes.POINTER(KVLayout),
                                      ctypes.POINTER(ScaleLayout), _p, _p, _p]
        L.pa_debug_gather_rope.argtypes = [ctypes.POINTER(PlanInfo), _p, _p, ctypes.POINTER(KVLayout),
                                           ctypes.POINTER(KVLayout), ctypes.POINTER(KVLayout),
                                           ctypes.POINTER(ScaleLayout), _p, _p]
        L.pa_validate_page_indices.argtypes = [ctypes.POINTER(PlanInfo), _p, _p, ctypes.c_int64, _p]
        L.pa_validate_page_indices.restype = ctypes.c_int
        L.pa_decode_noalloc.argtypes = [ctypes.POINTER(PlanInfo), _p, _p, _p, _p, _p, ctypes.POINTER(KVLayout), _p,
                                        _p, ctypes.POINTER(ScaleLayout), _p, ctypes.c_float, _p, ctypes.c_int, _p,
                                        _p]
        for f in ("pa_plan_splits", "pa_decode_stage1", "pa_decode_merge", "pa_decode_noalloc", "pa_kv_quantize_fp8",
                  "pa_kv_quantize_fp8_per_head", "pa_kv_quantize_int8", "pa_kv_append", "pa_debug_gather",
                  "pa_debug_gather_rope"):
            getattr(L, f).restype = ctypes.c_int
        L.pa_last_error.restype = ctypes.c_char_p
        L.pa_version.restype = ctypes.c_char_p
        _lib = L
    return _lib


def _check(status: int):
    if status != PA_OK:
        raise PaError(status, lib().pa_last_error().decode())


def _ptr(x) -> Optional[int]:
    if x is None:
        return None
    if isinstance(x, int):
        return x
    return x.data_ptr()


def _stream(stream) -> Optional[int]:
    if stream is not None:
        return stream if isinstance(stream, int) else stream.cuda_stream
    import torch
    if torch.cuda.is_available() and torch.cuda.is_initialized():
        return torch.cuda.current_stream().cuda_stream
    return None


def _dt(x) -> int:
    return DTYPES[x] if isinstance(x, str) else int(x)


def _sm(x) -> int:
    return SCALE_MODES[x] if isinstance(x, str) else int(x)


def pa_version() -> str:
    return lib().pa_version().decode()


def pa_plan_splits(qo_indptr, kv_indptr, kv_len, window, max_q_len, page_size, num_q_heads, num_kv_heads, head_dim,
                   q_dtype, kv_dtype, kv_scale_mode, num_cus=0, max_splits=0, force_splits=0, query_only=False,
                   head_dim_v=0, orientation="kv_on_m"):
    """Returns (PlanInfo, plan bytes as a numpy uint8 array, or None with query_only)."""
    arrs = [np.ascontiguousarray(np.asarray(x, dtype=np.int32)) for x in (qo_indptr, kv_indptr, kv_len)]
    win = None if window is None else np.ascontiguousarray(np.asarray(window, dtype=np.int32))
    B = len(arrs[2])
    a = PlanArgs(B, arrs[0].ctypes.data_as(_i32p), arrs[1].ctypes.data_as(_i32p), arrs[2].ctypes.data_as(_i32p),
                 None if win is None else win.ctypes.data_as(_i32p), int(max_q_len), int(page_size),
                 int(num_q_heads), int(num_kv_heads), int(head_dim), _dt(q_dtype), _dt(kv_dtype),
                 _sm(kv_scale_mode), int(num_cus), int(max_splits), int(force_splits), int(head_dim_v),
                 _orient(orientation))
    info = PlanInfo()
    _check(lib().pa_plan_splits(ctypes.byref(a), None, 0, ctypes.byref(info)))
    if query_only:
        return info, None
    buf = np.zeros(int(info.plan_bytes), dtype=np.uint8)
    _check(lib().pa_plan_splits(ctypes.byref(a), buf.ctypes.data, buf.nbytes, ctypes.byref(info)))
    return info, buf


def pa_decode_stage1(info, plan_dev, q, q_scale, k_cache, v_cache, kv_layout, k_scale, v_scale, scale_layout,
                     page_indices, sm_scale, partial_o, partial_lse, out, out_dtype, out_lse=None, stream=None):
    kvl = KVLayout(*kv_layout)
    scl = None if scale_layout is None else ScaleLayout(*scale_layout)
    _check(lib().pa_decode_stage1(ctypes.byref(info), _ptr(plan_dev), _ptr(q), _ptr(q_scale), _ptr(k_cache),
                                  _ptr(v_cache), ctypes.byref(kvl), _ptr(k_scale), _ptr(v_scale),
                                  None if scl is None else ctypes.byref(scl), _ptr(page_indices),
                                  ctypes.c_float(sm_scale), _ptr(partial_o), _ptr(partial_lse), _ptr(out),
                                  _dt(out_dtype), _ptr(out_lse), _stream(stream)))


def pa_validate_page_indices(info, plan_dev, page_indices, num_pages, stream=None):
    _check(lib().pa_validate_page_indices(ctypes.byref(info), _ptr(plan_dev), _ptr(page_indices),
                                          ctypes.c_int64(int(num_pages)), _stream(stream)))


def pa_decode_noalloc(info, plan_dev, q, q_scale, k_cache, v_cache, kv_layout, k_scale, v_scale, scale_layout,
                      page_indices, sm_scale, out, out_dtype, out_lse=None, stream=None):
    kvl = KVLayout(*kv_layout)
    scl = None if scale_layout is None else ScaleLayout(*scale_layout)
    _check(lib().pa_decode_noalloc(ctypes.byref(info), _ptr(plan_dev), _ptr(q), _ptr(q_scale), _ptr(k_cache),
                                   _ptr(v_cache), ctypes.byref(kvl), _ptr(k_scale), _ptr(v_scale),
                                   None if scl is None else ctypes.byref(scl), _ptr(page_indices),
                                   ctypes.c_float(sm_scale), _ptr(out), _dt(out_dtype), _ptr(out_lse),
                                   _stream(stream)))


def _layout(x):
    return None if x is None else ctypes.byref(KVLayout(*x))


def pa_debug_gather_rope(info, plan_dev, page_indices, k_layout, k_rope_layout, v_layout, k_scale_layout, off_out,
                         stream=None):
    scl = None if k_scale_layout is None else ctypes.byref(ScaleLayout(*k_scale_layout))
    _check(lib().pa_debug_gather_rope(ctypes.byref(info), _ptr(plan_dev), _ptr(page_indices), _layout(k_layout),
                                      _layout(k_rope_layout), _layout(v_layout), scl, _ptr(off_out),
                                      _stream(stream)))


def pa_decode_stage1_rope(info, plan_dev, q, q_scale, q_rope, k_cache, k_layout, k_rope, k_rope_layout, k_scale,
                          k_scale_layout, v_cache, v_layout, page_indices, sm_scale, partial_o, partial_lse, out,
                          out_dtype, out_lse=None, stream=None):
    _check(lib().pa_decode_stage1_rope(ctypes.byref(info), _ptr(plan_dev), _ptr(q), _ptr(q_scale), _ptr(q_rope),
                                       _ptr(k_cache), _layout(k_layout), _ptr(k_rope), _layout(k_rope_layout),
                                       _ptr(k_scale), _layout(k_scale_layout), _ptr(v_cache), _layout(v_layout),
                                       _ptr(page_indices), ctypes.c_float(sm_scale), _ptr(partial_o),
                                       _ptr(partial_lse), _ptr(out), _dt(out_dtype), _ptr(out_lse), _stream(stream)))


def pa_decode_merge(info, plan_dev, partial_o, partial_lse, out, out_dtype, out_lse=None, stream=None):
    _check(lib().pa_decode_merge(ctypes.byref(info), _ptr(plan_dev), _ptr(partial_o), _ptr(partial_lse), _ptr(out),
                                 _dt(out_dtype), _ptr(out_lse), _stream(stream)))


def pa_kv_quantize_fp8(src, src_dtype, n_rows, head_dim, mode, dst, scale, stream=None):
    _check(lib().pa_kv_quantize_fp8(_ptr(src), _dt(src_dtype), int(n_rows), int(head_dim), _sm(mode), _ptr(dst),
                                    _ptr(scale), _stream(stream)))


def pa_kv_quantize_int8(src, src_dtype, n_rows, head_dim, mode, dst, scale, stream=None):
    _check(lib().pa_kv_quantize_int8(_ptr(src), _dt(src_dtype), int(n_rows), int(head_dim), _sm(mode), _ptr(dst),
                                     _ptr(scale), _stream(stream)))


def pa_kv_quantize_fp8_per_head(src, src_dtype, n_tokens, num_heads, head_dim, dst, scale, stream=None):
    _check(lib().pa_kv_quantize_fp8_per_head(_ptr(src), _dt(src_dtype), ctypes.c_int64(int(n_tokens)), int(num_heads),
                                             int(head_dim), _ptr(dst), _ptr(scale), _stream(stream)))


def pa_kv_append(k_new, v_new, src_dtype, n_tokens, num_kv_heads, head_dim, page_size, slot_mapping, k_cache,
                 v_cache, kv_dtype, mode, kv_layout, k_scale=None, v_scale=None, scale_layout=None, stream=None):
    kvl = KVLayout(*kv_layout)
    scl = None if scale_layout is None else ScaleLayout(*scale_layout)
    _check(lib().pa_kv_append(_ptr(k_new), _ptr(v_new), _dt(src_dtype), ctypes.c_int64(int(n_tokens)),
                              int(num_kv_heads), int(head_dim), int(page_size), _ptr(slot_mapping), _ptr(k_cache),
                              _ptr(v_cache), _dt(kv_dtype), _sm(mode), ctypes.byref(kvl), _ptr(k_scale),
                              _ptr(v_scale), None if scl is None else ctypes.byref(scl), _stream(stream)))


def pa_debug_gather(info, plan_dev, page_indices, kv_layout, scale_layout, kv_off_out, scale_off_out=None,
                    stream=None):
    kvl = KVLayout(*kv_layout)
    scl = None if scale_layout is None else ScaleLayout(*scale_layout)
    _check(lib().pa_debug_gather(ctypes.byref(info), _ptr(plan_dev), _ptr(page_indices), ctypes.byref(kvl),
                                 None if scl is None else ctypes.byref(scl), _ptr(kv_off_out), _ptr(scale_off_out),
                                 _stream(stream)))
