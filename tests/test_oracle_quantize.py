"""Pins of the oracle's FP8 quantiser: torch's independent cast after the same
clamp and fp32 divide, the definition's error bound, and its special cases."""
import numpy as np
import torch

from oracle.formats import e4m3_code_to_f64
from oracle.quantize import quantize_per_row, quantize_per_tensor


def _torch_quant_rows(x32: torch.Tensor):
    amax = x32.abs().amax(dim=-1)
    scale = torch.where(amax == 0, torch.ones_like(amax), amax / 448.0)
    q = (x32 / scale[..., None]).clamp(-448, 448)
    return q.to(torch.float8_e4m3fn).view(torch.uint8), scale


def test_per_row_matches_torch_cast():
    g = torch.Generator().manual_seed(0)
    x = torch.randn(64, 3, 16, 128, generator=g).to(torch.bfloat16)
    x[5, 1, 3] = 0                                   # an all-zero row
    x[7, 0, 0, :4] = torch.tensor([1e-30, -3.0, 2.5e4, 0.0])
    codes, scale = quantize_per_row(x.view(torch.int16).numpy(), "bf16")
    ref_codes, ref_scale = _torch_quant_rows(x.float())
    assert np.array_equal(scale, ref_scale.numpy())
    assert np.array_equal(codes, ref_codes.numpy())
    assert scale[5, 1, 3] == 1.0 and not codes[5, 1, 3].any()


def test_per_tensor_matches_torch_cast():
    g = torch.Generator().manual_seed(1)
    x = torch.randn(33, 8, 128, generator=g)
    codes, scale = quantize_per_tensor(x.numpy(), "fp32")
    amax = x.abs().max()
    ref_scale = amax / 448.0
    ref = (x / ref_scale).clamp(-448, 448).to(torch.float8_e4m3fn).view(torch.uint8)
    assert np.float32(scale) == ref_scale.item()
    assert np.array_equal(codes, ref.numpy())


def test_amax_element_maps_to_largest_code_and_error_bound():
    rng = np.random.default_rng(2)
    x = rng.standard_normal((200, 128)).astype(np.float32)
    codes, scale = quantize_per_row(x, "fp32")
    i = np.argmax(np.abs(x), axis=1)
    top = codes[np.arange(200), i]
    assert np.all((top & 0x7F) == 0x7E)
    deq = e4m3_code_to_f64(codes) * scale[:, None].astype(np.float64)
    # RNE into a 3-bit mantissa: relative error <= 2^-4 for normals, absolute
    # error <= 2^-10 * scale in the subnormal range
    err = np.abs(deq - x)
    bound = np.maximum(np.abs(x) * 2.0 ** -4, 2.0 ** -10 * scale[:, None]) * (1 + 1e-6)
    assert np.all(err <= bound)
