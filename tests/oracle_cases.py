"""Tiny paged problems for the oracle's own tests (CPU)."""
import numpy as np
import torch

from oracle.attention import PagedKV


def bf16_bits(x: np.ndarray) -> np.ndarray:
    return torch.from_numpy(np.asarray(x, dtype=np.float32)).to(torch.bfloat16).view(torch.int16).numpy().astype(np.uint16)


def tiny_problem(seed, B=2, rows=(2, 3), kv_len=(13, 21), window=(0, 5), P=4, Hq=4, Hkv=2, d=8,
                 layout="HPD"):
    rng = np.random.default_rng(seed)
    rows = np.asarray(rows, dtype=np.int64)
    kv_len = np.asarray(kv_len, dtype=np.int64)
    window = np.asarray(window, dtype=np.int64)
    pages_b = (kv_len + P - 1) // P
    kv_indptr = np.concatenate([[0], np.cumsum(pages_b)])
    qo_indptr = np.concatenate([[0], np.cumsum(rows)])
    npages = int(pages_b.sum()) + 3                       # 3 pages nobody uses
    page_indices = rng.permutation(npages)[: int(pages_b.sum())].astype(np.int32)
    T = int(qo_indptr[-1])
    q = bf16_bits(rng.standard_normal((T, Hq, d)))
    shape = (npages, Hkv, P, d) if layout == "HPD" else (npages, P, Hkv, d)
    k = bf16_bits(rng.standard_normal(shape))
    v = bf16_bits(rng.standard_normal(shape))
    return dict(q=q, k=PagedKV(k, "bf16", layout), v=PagedKV(v, "bf16", layout),
                page_indices=page_indices, kv_indptr=kv_indptr, kv_len=kv_len, qo_indptr=qo_indptr,
                window=window, P=P, Hq=Hq, Hkv=Hkv, d=d, sm_scale=float(np.float32(1 / np.sqrt(d))))
