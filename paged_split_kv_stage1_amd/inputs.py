"""Seeded synthetic workloads for paged split-KV decode.

This module is the only code shared by the GPU path's tests/bench and by the
CPU oracle.  It draws random numbers and builds index structures; it holds none
of the method's arithmetic (no attention, no FP8 quantisation).  bf16 values are
produced with torch's own float32 -> bfloat16 cast (round to nearest even).

Shapes follow the workloads named on the pages:
  * FP8 single-row decode, batch 128, 64 Q / 8 KV heads, head_dim 128, KV 2048,
    page/block size 64 (hpc-ops issue #4, benchmark printout);
  * multi-row verify, 16 Q / 2 KV heads, head_dim 256, contexts 32K/128K
    (FreeToken PR #900, "Kernel time" table);
  * up to 8 query rows per request with per-row position and window, groups
    that are not a multiple of 16 such as 48/2 (FreeToken PR #900, "Changes").

Layouts produced here:
  * K/V source values: bf16, shape [num_pages, Hkv, page_size, d] (one page of one
    KV head is contiguous); the FP8 configs quantise these with the library's
    quantiser (GPU side) or the oracle's quantiser (CPU side).
  * page_indices: a seeded permutation of exactly sum(ceil(kv_len/P)) pages.
  * unused slots (the tail of each request's last page) are marked in
    ``unused_slots`` so that callers can poison them with NaN patterns.
"""
from __future__ import annotations

import dataclasses
import math
from typing import Optional

import numpy as np
import torch

__all__ = ["Workload", "CONFIGS", "make_workload", "poison_unused"]


@dataclasses.dataclass
class Workload:
    name: str
    seed: int
    batch: int
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    page_size: int
    qo_indptr: np.ndarray      # int32 [B+1]
    kv_len: np.ndarray         # int32 [B]
    window: np.ndarray         # int32 [B], 0 = no window
    kv_indptr: np.ndarray      # int32 [B+1], CSR over page_indices
    page_indices: np.ndarray   # int32 [num_pages]
    q: torch.Tensor            # bf16 [T, Hq, d] (CPU)
    k: torch.Tensor            # bf16 [num_pages, Hkv, P, d] (CPU)
    v: torch.Tensor            # bf16 [num_pages, Hkv, P, d] (CPU)
    unused_slots: np.ndarray   # bool [num_pages, P]: slot holds no token
    q_dtype: str               # "bf16" | "fp8"   (fp8: quantise q per tensor)
    kv_dtype: str              # "bf16" | "fp8" | "int8"
    kv_scale_mode: str         # "none" | "per_tensor" | "per_head" | "per_token_head"
    out_dtype: str             # "fp32" | "bf16"
    sm_scale: float            # float32 value of 1/sqrt(d)
    forced_splits: int = 0     # 0 = planner decides
    head_dim_v: int = 0        # value width when it differs from head_dim (the key width); 0 = same
    latent: bool = False       # MLA-style cache: k holds [latent (head_dim_v), rotary]; v is the latent

    @property
    def dv(self) -> int:
        return self.head_dim_v or self.head_dim

    @property
    def total_rows(self) -> int:
        return int(self.qo_indptr[-1])

    @property
    def num_pages(self) -> int:
        return int(self.page_indices.shape[0])

    @property
    def max_q_len(self) -> int:
        return int(np.max(np.diff(self.qo_indptr))) if self.batch else 0


# Named workloads.  "c1".."c5" are the five measured configurations; the other
# names are the same shapes at another batch or row count.
CONFIGS = {
    "c1": dict(batch=1, rows=1, hq=8, hkv=1, d=128, ctx=512, page=16, q="bf16", kv="bf16",
               scale="none", out="fp32", splits=4),
    "c2": dict(batch=128, rows=1, hq=64, hkv=8, d=128, ctx=2048, page=64, q="fp8", kv="fp8",
               scale="per_tensor", out="bf16"),
    "c2_ph": dict(batch=128, rows=1, hq=64, hkv=8, d=128, ctx=2048, page=64, q="fp8", kv="fp8",
                  scale="per_head", out="bf16"),
    "c3": dict(batch=16, rows=4, hq=16, hkv=2, d=256, ctx=32768, page=16, q="bf16", kv="bf16",
               scale="none", out="bf16"),
    "c3_b1": dict(batch=1, rows=4, hq=16, hkv=2, d=256, ctx=32768, page=16, q="bf16", kv="bf16",
                  scale="none", out="bf16"),
    "c3_r1": dict(batch=16, rows=1, hq=16, hkv=2, d=256, ctx=32768, page=16, q="bf16", kv="bf16",
                  scale="none", out="bf16"),
    "c3_b1_r1": dict(batch=1, rows=1, hq=16, hkv=2, d=256, ctx=32768, page=16, q="bf16", kv="bf16",
                     scale="none", out="bf16"),
    "c3_b1_r8": dict(batch=1, rows=8, hq=16, hkv=2, d=256, ctx=32768, page=16, q="bf16", kv="bf16",
                     scale="none", out="bf16"),
    "c3_r8": dict(batch=16, rows=8, hq=16, hkv=2, d=256, ctx=32768, page=16, q="bf16", kv="bf16",
                  scale="none", out="bf16"),
    "c4": dict(batch=16, rows=8, hq=16, hkv=2, d=256, ctx=131072, page=16, q="bf16", kv="fp8",
               scale="per_token_head", out="bf16"),
    "c4_i8": dict(batch=16, rows=8, hq=16, hkv=2, d=256, ctx=131072, page=16, q="bf16", kv="int8",
                  scale="per_token_head", out="bf16"),
    "c4_i8t": dict(batch=16, rows=8, hq=16, hkv=2, d=256, ctx=131072, page=16, q="bf16", kv="int8",
                   scale="per_tensor", out="bf16"),
    "c4_b1": dict(batch=1, rows=8, hq=16, hkv=2, d=256, ctx=131072, page=16, q="bf16", kv="fp8",
                  scale="per_token_head", out="bf16"),
    "c4_r1": dict(batch=16, rows=1, hq=16, hkv=2, d=256, ctx=131072, page=16, q="bf16", kv="fp8",
                  scale="per_token_head", out="bf16"),
    "c4_b1_r1": dict(batch=1, rows=1, hq=16, hkv=2, d=256, ctx=131072, page=16, q="bf16", kv="fp8",
                     scale="per_token_head", out="bf16"),
    # head_dim 512 with one KV head (the Gemma-4 full-attention layers of FreeToken PR #900,
    # "Gemma-4 MTP at long context": batch 1, k+1 = 4 or 8 verify rows, 128K context, bf16);
    # the page gives no query-head count: 8 query heads, so that 8 rows fill one 64-row tile
    "c6": dict(batch=1, rows=8, hq=8, hkv=1, d=512, ctx=131072, page=16, q="bf16", kv="bf16",
               scale="none", out="bf16"),
    "c6_r4": dict(batch=1, rows=4, hq=8, hkv=1, d=512, ctx=131072, page=16, q="bf16", kv="bf16",
                  scale="none", out="bf16"),
    # the same shape with an FP8 cache ("quantized head_dim 512" in the same PR's launch
    # notes): per-token-head e4m3 K/V, bf16 queries
    "c6_f8": dict(batch=1, rows=8, hq=8, hkv=1, d=512, ctx=131072, page=16, q="bf16", kv="fp8",
                  scale="per_token_head", out="bf16"),
    "c5": dict(batch=64, rows="ragged", hq=48, hkv=2, d=128, ctx="loguniform", page=32, q="bf16",
               kv="fp8", scale="per_token_head", out="bf16", windowed=True, window=64),
    # keys wider than values (FlashInfer PR #869, "Remaining Work"): 192-channel keys (128 +
    # a 64-channel rotary part, the split the pages' MLA model family uses) and 128-channel
    # values, bf16, grouped query heads
    "f3": dict(batch=32, rows=1, hq=32, hkv=4, d=192, dv=128, ctx=8192, page=16, q="bf16", kv="bf16",
               scale="none", out="bf16"),
    "f3_r4": dict(batch=32, rows=4, hq=32, hkv=4, d=192, dv=128, ctx=8192, page=16, q="bf16", kv="bf16",
                  scale="none", out="bf16"),
    # MLA-style decode (FlashMLA PR #54): one latent KV head of 512 e4m3 channels with a scale
    # per (token, 128 channels) plus 64 bf16 rotary channels; queries likewise (nope part
    # e4m3 per 128 channels, rotary bf16); 16 query heads; block size 64; values = latent
    "mla": dict(batch=64, rows=1, hq=16, hkv=1, d=576, dv=512, ctx=4096, page=64, q="fp8", kv="fp8",
                scale="per_token_block128", out="bf16", latent=True),
    "mla_r2": dict(batch=64, rows=2, hq=16, hkv=1, d=576, dv=512, ctx=4096, page=64, q="fp8", kv="fp8",
                   scale="per_token_block128", out="bf16", latent=True),
}

SEEDS = {"c1": 1, "c2": 2, "c3": 3, "c4": 4, "c5": 5, "c6": 6, "f3": 7, "mla": 8}


def _seed_for(name: str) -> int:
    base = SEEDS[name.split("_")[0]]
    return base + (100 if "_b1" in name else 0) + (10 if "_r" in name else 0)


def make_workload(name: str, seed: Optional[int] = None, *, batch: Optional[int] = None,
                  ctx: Optional[int] = None, ctx_range: Optional[tuple] = None,
                  rows: Optional[object] = None, out_dtype: Optional[str] = None,
                  page: Optional[int] = None, kv_layout_note: str = "HPD",
                  overrides: Optional[dict] = None) -> Workload:
    """Build the named workload, optionally shrunk (batch/ctx/rows overrides), with
    another page size (``page``), or with other configuration keys (``overrides``, the
    keys of CONFIGS: hq, hkv, d, q, kv, scale, ...).

    ``rows`` may be an int (every request), a list (per request) or "ragged"
    (uniform 1..8).  ``ctx`` may be an int or a list; ``ctx_range`` replaces the
    log-uniform range of the ragged workload.
    """
    cfg = dict(CONFIGS[name])
    cfg.update(overrides or {})          # e.g. other head counts, head_dim or dtypes
    seed = _seed_for(name) if seed is None else seed
    gen = torch.Generator().manual_seed(seed)
    rng = np.random.default_rng(seed)
    B = cfg["batch"] if batch is None else batch
    P = cfg["page"] if page is None else page
    hq, hkv, d = cfg["hq"], cfg["hkv"], cfg["d"]

    # rows per request
    r = cfg["rows"] if rows is None else rows
    if isinstance(r, str):
        assert r == "ragged"
        rows_b = rng.integers(1, 9, size=B)
    elif isinstance(r, (list, tuple, np.ndarray)):
        rows_b = np.asarray(r, dtype=np.int64)
        assert rows_b.shape == (B,)
    else:
        rows_b = np.full(B, int(r))

    # context lengths (tokens, including the new rows)
    c = cfg["ctx"] if ctx is None else ctx
    if isinstance(c, str) or ctx_range is not None:
        lo, hi = (1024, 65536) if ctx_range is None else ctx_range
        u = rng.uniform(math.log(lo), math.log(hi), size=B)
        kv_len = np.floor(np.exp(u)).astype(np.int64)
    elif isinstance(c, (list, tuple, np.ndarray)):
        kv_len = np.asarray(c, dtype=np.int64)
        assert kv_len.shape == (B,)
    else:
        kv_len = np.full(B, int(c))
    kv_len = np.maximum(kv_len, rows_b)

    window = np.zeros(B, dtype=np.int64)
    if cfg.get("windowed"):
        # half of the requests carry the sliding window
        chosen = rng.permutation(B)[:B // 2]
        window[chosen] = cfg["window"]

    pages_b = (kv_len + P - 1) // P
    num_pages = int(pages_b.sum())
    kv_indptr = np.zeros(B + 1, dtype=np.int64)
    kv_indptr[1:] = np.cumsum(pages_b)
    qo_indptr = np.zeros(B + 1, dtype=np.int64)
    qo_indptr[1:] = np.cumsum(rows_b)
    perm = torch.randperm(num_pages, generator=gen).numpy()
    page_indices = perm.astype(np.int32)

    T = int(qo_indptr[-1])
    dv = cfg.get("dv", d)
    q = torch.randn(T, hq, d, generator=gen, dtype=torch.float32).to(torch.bfloat16)
    k = torch.randn(num_pages, hkv, P, d, generator=gen, dtype=torch.float32).to(torch.bfloat16)
    if cfg.get("latent"):
        v = k[..., :dv]                  # the value is the key's latent part
    else:
        v = torch.randn(num_pages, hkv, P, dv, generator=gen, dtype=torch.float32).to(torch.bfloat16)

    unused = np.zeros((num_pages, P), dtype=bool)
    for b in range(B):
        last = int(kv_len[b] - 1) // P
        used_in_last = int(kv_len[b]) - last * P
        phys = page_indices[kv_indptr[b] + last]
        unused[phys, used_in_last:] = True

    return Workload(
        name=name, seed=seed, batch=B, num_q_heads=hq, num_kv_heads=hkv, head_dim=d,
        page_size=P, qo_indptr=qo_indptr.astype(np.int32), kv_len=kv_len.astype(np.int32),
        window=window.astype(np.int32), kv_indptr=kv_indptr.astype(np.int32),
        page_indices=page_indices, q=q, k=k, v=v, unused_slots=unused,
        q_dtype=cfg["q"], kv_dtype=cfg["kv"], kv_scale_mode=cfg["scale"],
        out_dtype=cfg["out"] if out_dtype is None else out_dtype,
        sm_scale=float(np.float32(1.0) / np.sqrt(np.float32(d))),
        forced_splits=cfg.get("splits", 0), head_dim_v=dv if dv != d else 0, latent=bool(cfg.get("latent")))


# Byte patterns used to poison slots that hold no token: a NaN in each format, and for
# INT8 codes (which have no NaN) -128, a code the quantiser never writes (the per-token
# scales of those slots are NaN).
BF16_NAN_BITS = 0x7FC1
E4M3_NAN_CODE = 0x7F
INT8_POISON_CODE = 0x80


def poison_unused(cache: torch.Tensor, unused_slots: np.ndarray, layout: str = "HPD") -> torch.Tensor:
    """Overwrite unused slots of a [pages, Hkv, P, d] (HPD) or [pages, P, Hkv, d]
    (PHD) cache with a NaN bit pattern of its storage format.  Returns the cache.
    Works on bf16 tensors and on uint8 (e4m3 code) tensors."""
    mask = torch.from_numpy(unused_slots)
    if layout == "HPD":
        m = mask[:, None, :, None].expand(cache.shape)
    else:
        m = mask[:, :, None, None].expand(cache.shape)
    if cache.dtype == torch.bfloat16:
        cache.view(torch.int16)[m] = BF16_NAN_BITS
    elif cache.dtype == torch.uint8:
        cache[m] = E4M3_NAN_CODE
    else:
        raise TypeError(cache.dtype)
    return cache
