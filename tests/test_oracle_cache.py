"""Pins of oracle.cache (KV append) and of the float32 -> bf16 encoder it uses."""
import numpy as np
import pytest
import torch

from oracle.cache import append_kv
from oracle.formats import bf16_bits_to_f64, e4m3_code_to_f64, f32_to_bf16_bits_rne
from oracle.quantize import quantize_per_row


def test_f32_to_bf16_matches_torch_cast():
    # ties (lower 16 bits exactly 0x8000) and their neighbours, both signs, plus
    # random values, overflow to infinity and infinities
    rng = np.random.default_rng(3)
    hi = rng.integers(0, 0x7F7F, 4000, dtype=np.uint32) << 16
    low = np.concatenate([np.full(1000, 0x8000), np.full(1000, 0x7FFF), np.full(1000, 0x8001),
                          rng.integers(0, 0x10000, 1000)]).astype(np.uint32)
    bits = (hi | low) ^ (rng.integers(0, 2, 4000, dtype=np.uint32) << 31)
    x = np.concatenate([bits.view(np.float32), np.array([3.4e38, -3.4e38, np.inf, -np.inf, 0.0, -0.0],
                                                        dtype=np.float32)])
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(f32_to_bf16_bits_rne(x), ref)
    assert np.isnan(bf16_bits_to_f64(f32_to_bf16_bits_rne(np.array([np.nan], np.float32))))[0]


@pytest.mark.parametrize("layout", ["HPD", "PHD"])
@pytest.mark.parametrize("kind", ["bf16", "fp8_per_tensor", "fp8_per_token_head"])
def test_append_places_rows_at_hand_computed_slots(layout, kind):
    P, pages, hkv, d = 4, 3, 2, 8
    rng = np.random.default_rng(5)
    shape = (pages, hkv, P, d) if layout == "HPD" else (pages, P, hkv, d)
    dtype = np.uint16 if kind == "bf16" else np.uint8
    cache = rng.integers(0, 100, shape).astype(dtype)
    scales = rng.random(shape[:3]).astype(np.float32) if kind == "fp8_per_token_head" else None
    rows = torch.randn(4, hkv, d).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    slots = [5, 0, -1, 11]                         # -> (page 1, slot 1), (0, 0), skipped, (2, 3)
    new, new_sc = append_kv(cache, scales, rows, "bf16", slots, P, kind, layout, tensor_scale=0.01)
    where = {(1, 1): 0, (0, 0): 1, (2, 3): 3}
    for page in range(pages):
        for slot in range(P):
            for h in range(hkv):
                idx = (page, h, slot) if layout == "HPD" else (page, slot, h)
                if (page, slot) not in where:
                    assert np.array_equal(new[idx], cache[idx])
                    if scales is not None:
                        assert new_sc[idx] == scales[idx]
                    continue
                t = where[(page, slot)]
                if kind == "bf16":
                    assert np.array_equal(new[idx], rows[t, h])
                elif kind == "fp8_per_token_head":
                    codes, sc = quantize_per_row(rows[t, h][None], "bf16")
                    assert np.array_equal(new[idx], codes[0]) and new_sc[idx] == sc[0]
                else:
                    # decoded code x scale within half an e4m3 step of the value
                    sc = np.float64(np.float32(0.01))
                    q = bf16_bits_to_f64(rows[t, h]) / sc
                    step = np.exp2(np.floor(np.log2(np.maximum(np.abs(q), 2.0 ** -6))) - 3)
                    err = np.abs(e4m3_code_to_f64(new[idx]) - np.clip(q, -448, 448))
                    assert np.all(err <= step / 2 * (1 + 1e-6))


def test_append_per_tensor_exact_multiples_and_fp32_to_bf16():
    # values that are exact e4m3 numbers times the scale encode to exactly those numbers;
    # a float32 source into a bf16 cache is rounded to nearest even
    scale = np.float32(0.125)
    vals = np.array([0.0, 1.0, -1.5, 448.0, -448.0, 2.0 ** -9, 3.25, -240.0], dtype=np.float32)
    rows = (vals * scale).astype(np.float32).reshape(1, 1, 8)
    cache = np.zeros((1, 1, 4, 8), np.uint8)
    new, _ = append_kv(cache, None, rows, "fp32", [2], 4, "fp8_per_tensor", tensor_scale=scale)
    assert np.array_equal(e4m3_code_to_f64(new[0, 0, 2]), vals.astype(np.float64))
    x = np.array([[[1.00390625, 1.005859375, -2.5, 1e-3, 7.0, -0.0, 65504.0, 1.0]]], dtype=np.float32)
    cb = np.zeros((1, 1, 4, 8), np.uint16)
    new, _ = append_kv(cb, None, x, "fp32", [1], 4, "bf16")
    ref = torch.from_numpy(x.reshape(-1)).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(new[0, 0, 1], ref)


def test_append_per_head_uses_each_heads_scale():
    # with per-head scales, head h's row encodes as the per-tensor encoding with scale[h]:
    # exact multiples of that scale give back exactly the e4m3 values
    scales = np.array([0.125, 2.0, 0.0078125], np.float32)
    vals = np.array([0.0, 1.0, -1.5, 448.0, -448.0, 2.0 ** -9, 3.25, -240.0], dtype=np.float32)
    rows = np.stack([vals * s for s in scales])[None].astype(np.float32)        # [1, 3, 8]
    cache = np.full((2, 3, 4, 8), 0x55, np.uint8)
    new, _ = append_kv(cache, None, rows, "fp32", [6], 4, "fp8_per_head", tensor_scale=scales)
    for h in range(3):
        assert np.array_equal(e4m3_code_to_f64(new[1, h, 2]), vals.astype(np.float64))
        one, _ = append_kv(cache, None, rows, "fp32", [6], 4, "fp8_per_tensor", tensor_scale=scales[h])
        assert np.array_equal(new[1, h, 2], one[1, h, 2])
    untouched = np.ones(new.shape[:3], bool)
    untouched[1, :, 2] = False
    assert np.all(new[untouched] == 0x55)


def test_append_int8_per_token_head_and_per_tensor():
    from oracle.quantize import quantize_int8_per_row
    rng = np.random.default_rng(13)
    rows = (rng.standard_normal((3, 2, 16)) * 4).astype(np.float32)
    cache = np.full((2, 2, 4, 16), 0x5A, np.uint8)
    scales = np.full((2, 2, 4), -1.0, np.float32)
    new, nsc = append_kv(cache, scales, rows, "fp32", [7, -1, 0], 4, "int8_per_token_head")
    for t, (page, slot) in ((0, (1, 3)), (2, (0, 0))):
        for h in range(2):
            c, s = quantize_int8_per_row(rows[t, h][None], "fp32")
            assert np.array_equal(new[page, h, slot].view(np.int8), c[0]) and nsc[page, h, slot] == s[0]
    keep = np.ones((2, 2, 4), bool)
    keep[1, :, 3] = keep[0, :, 0] = False
    assert np.all(new[keep] == 0x5A) and np.all(nsc[keep] == -1.0)
    # integers times the tensor scale encode to exactly those integers
    ints = np.array([0, 1, -1, 127, -127, 64, -3, 2], np.float32)
    scale = np.float32(0.0625)
    new, _ = append_kv(np.zeros((1, 1, 4, 8), np.uint8), None, (ints * scale).reshape(1, 1, 8), "fp32", [1], 4,
                       "int8_per_tensor", tensor_scale=scale)
    assert np.array_equal(new[0, 0, 1].view(np.int8), ints.astype(np.int8))
