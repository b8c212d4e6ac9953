"""CPU oracle for paged split-KV decode attention -- test infrastructure only.

Plain, slow, float64 reference implementations of what the GPU library computes.
Only the tests, the smoke check and the benchmark's CPU-baseline leg may import
this package; the library itself never does, and this package imports nothing
from the library (it shares only the seeded input generator module).

Modules:
  formats   -- exact decoders for bf16 and OCP E4M3FN, and an RNE encoder into E4M3FN
  quantize  -- FP8 KV quantisation (per-tensor and per-(token, KV head) scales)
  attention -- page gather, per-row visible range, softmax attention in fp64,
               per-split partials and their log-sum-exp merge
"""
from . import formats, quantize, attention  # noqa: F401
