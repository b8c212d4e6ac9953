"""Algorithmic bytes and flops of one decode step (what the method must move).

Convention (the hpc-ops issue #4 benchmark printout reproduces exactly with it):
bytes = K+V values of every visible (token, KV head) + Q + output, each at its
storage width; flops = 4 * d per visible (query row, query head, token)
(2*d for q.k and 2*d for p.v).  For B=128, q_len 1, KV 2048, 64/8 heads,
d=128, FP8 Q/K/V and bf16 output this gives 540,016,640 B and 8,589,934,592
flop; at the printed 6800.0 iter/s that is 3672.1 GB/s and 58.41 TFLOPS.

Added here beyond that printout and reported separately: per-(token, KV head)
float32 scales (8 B per token per KV head for K and V), per-tensor scalars,
and the int32 page indices of the pages that hold visible tokens.
Split scratch (partial O / LSE) is overhead, not algorithmic traffic.
"""
from __future__ import annotations

import numpy as np

_SIZE = {"bf16": 2, "fp8": 1, "int8": 1, "fp32": 4}


def step_accounting(batch, qo_indptr, kv_len, window, page_size, num_q_heads, num_kv_heads,
                    head_dim, q_dtype, kv_dtype, kv_scale_mode, out_dtype, head_dim_v=0, latent=False) -> dict:
    """Keys of head_dim channels and values of head_dim_v (0 = head_dim); with ``latent``
    (MLA-style cache) each (token, KV head) stores head_dim_v e4m3 latent codes, one
    float32 scale per 128 of them and head_dim - head_dim_v bf16 rotary channels, read
    once for both products, and the queries likewise (codes, scales, bf16 rotary part)."""
    qo_indptr = np.asarray(qo_indptr, dtype=np.int64)
    kv_len = np.asarray(kv_len, dtype=np.int64)
    window = np.zeros(batch, dtype=np.int64) if window is None else np.asarray(window, dtype=np.int64)
    G = num_q_heads // num_kv_heads
    d = head_dim
    kv_tok = 0          # visible (token, request) pairs: union over the request's rows
    pages = 0
    row_tokens = 0      # visible (row, token) pairs
    for b in range(batch):
        n = int(qo_indptr[b + 1] - qo_indptr[b])
        L = int(kv_len[b])
        p0 = L - n
        lo0 = max(0, p0 - int(window[b]) + 1) if window[b] > 0 else 0
        kv_tok += L - lo0
        pages += (L - 1) // page_size - lo0 // page_size + 1
        for r in range(n):
            p = p0 + r
            lo = max(0, p - int(window[b]) + 1) if window[b] > 0 else 0
            row_tokens += p - lo + 1
    T = int(qo_indptr[batch])
    dv = head_dim_v or d
    if latent or dv != d:
        dr = d - dv
        if latent:
            per_tok = dv + 4 * (dv // 128) + 2 * dr
            q_bytes = T * num_q_heads * (dv + 4 * (dv // 128) + 2 * dr)
        else:
            per_tok = (d + dv) * _SIZE[kv_dtype]
            q_bytes = T * num_q_heads * d * _SIZE[q_dtype]
        out = {"kv": kv_tok * num_kv_heads * per_tok, "kv_scales": 0, "q": q_bytes,
               "out": T * num_q_heads * dv * _SIZE[out_dtype], "page_table": pages * 4,
               "flops": 2 * (d + dv) * row_tokens * G * num_kv_heads}
        out["bytes"] = out["kv"] + out["q"] + out["out"] + out["page_table"]
        return out
    out = {
        "kv": kv_tok * num_kv_heads * 2 * d * _SIZE[kv_dtype],
        "kv_scales": kv_tok * num_kv_heads * 8 if kv_scale_mode == "per_token_head" else
                     (8 if kv_scale_mode == "per_tensor" else
                      (8 * num_kv_heads if kv_scale_mode == "per_head" else 0)),
        "q": T * num_q_heads * d * _SIZE[q_dtype] +
             ((4 * num_q_heads if kv_scale_mode == "per_head" else 4) if q_dtype == "fp8" else 0),
        "out": T * num_q_heads * d * _SIZE[out_dtype],
        "page_table": pages * 4,
        "flops": 4 * d * row_tokens * G * num_kv_heads,
    }
    out["bytes"] = out["kv"] + out["kv_scales"] + out["q"] + out["out"] + out["page_table"]
    return out


def workload_accounting(w) -> dict:
    """step_accounting for an inputs.Workload."""
    return step_accounting(w.batch, w.qo_indptr, w.kv_len, w.window, w.page_size, w.num_q_heads,
                           w.num_kv_heads, w.head_dim, w.q_dtype, w.kv_dtype, w.kv_scale_mode,
                           w.out_dtype, head_dim_v=w.head_dim_v, latent=w.latent)
