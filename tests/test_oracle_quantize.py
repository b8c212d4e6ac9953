"""Pins of the oracle's FP8 quantiser: torch's independent cast after the same
clamp and fp32 divide, the definition's error bound, and its special cases."""
import numpy as np
import torch

from oracle.formats import e4m3_code_to_f64
from oracle.quantize import (quantize_int8_per_row, quantize_int8_per_tensor, quantize_per_head, quantize_per_row,
                             quantize_per_tensor)


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


def test_per_head_matches_torch_cast_head_by_head():
    # each head's scale is the amax over all of that head's values / 448, computed by
    # torch on the head's slice; codes are torch's cast of the clamped fp32 quotient
    g = torch.Generator().manual_seed(4)
    x = torch.randn(37, 5, 64, generator=g) * torch.tensor([0.01, 1.0, 30.0, 0.5, 2.0])[None, :, None]
    x[:, 3] = 0                                      # an all-zero head: scale 1, codes 0
    codes, scale = quantize_per_head(x.numpy(), "fp32", head_axis=1)
    assert scale.shape == (5,)
    for h in range(5):
        xs = x[:, h]
        amax = xs.abs().max()
        ref_scale = torch.where(amax == 0, torch.ones(()), amax / 448.0)
        ref = (xs / ref_scale).clamp(-448, 448).to(torch.float8_e4m3fn).view(torch.uint8)
        assert np.float32(scale[h]) == ref_scale.item()
        assert np.array_equal(codes[:, h], ref.numpy())
    assert scale[3] == 1.0 and not codes[:, 3].any()


def test_per_head_heads_are_independent_and_axis_follows_layout():
    g = torch.Generator().manual_seed(6)
    x = torch.randn(3, 4, 16, 32, generator=g).to(torch.bfloat16)      # [pages, H, P, d]
    bits = x.view(torch.int16).numpy().view(np.uint16)
    c1, s1 = quantize_per_head(bits, "bf16", head_axis=1)
    y = x.clone()
    y[:, 0] *= 64                                    # only head 0 changes
    c2, s2 = quantize_per_head(y.view(torch.int16).numpy().view(np.uint16), "bf16", head_axis=1)
    assert np.array_equal(c1[:, 1:], c2[:, 1:]) and np.array_equal(s1[1:], s2[1:]) and s2[0] == 64 * s1[0]
    # the same data in [pages, P, H, d] gives the same scales and transposed codes
    c3, s3 = quantize_per_head(np.ascontiguousarray(bits.transpose(0, 2, 1, 3)), "bf16", head_axis=2)
    assert np.array_equal(s3, s1) and np.array_equal(c3.transpose(0, 2, 1, 3), c1)


def test_per_head_dequantisation_in_the_attention_inputs():
    # PagedKV multiplies KV head g's decoded codes by scale[g]; dequant_q multiplies query
    # head h's codes by q_scale[h] (checked against torch's own float8 decode)
    from oracle.attention import PagedKV, dequant_q
    rng = np.random.default_rng(8)
    codes = rng.integers(0, 256, (2, 3, 4, 8)).astype(np.uint8)
    codes[(codes & 0x7F) == 0x7F] = 0x12             # no NaN codes
    sc = np.array([0.5, 0.03125, 3.0], np.float32)
    kv = PagedKV(codes, "fp8", "HPD", "per_head", sc)
    dec = torch.from_numpy(codes).view(torch.float8_e4m3fn).double().numpy()
    slots = np.array([0, 5, 6])                      # (page 0, slot 0), (1, 1), (1, 2)
    for gh in range(3):
        ref = dec[slots // 4, gh, slots % 4] * np.float64(sc[gh])
        assert np.array_equal(kv.tokens(slots, gh), ref)
    q = codes.reshape(4, 3, 16)
    qs = np.array([2.0, 0.25, 1.5], np.float32)
    ref = torch.from_numpy(q).view(torch.float8_e4m3fn).double().numpy() * qs[None, :, None].astype(np.float64)
    assert np.array_equal(dequant_q(q, "fp8", qs), ref)


def test_int8_per_row_matches_torch_round_half_even():
    # scale = amax/127 in fp32; codes = torch.round (ties to even) of the clamped quotient
    g = torch.Generator().manual_seed(9)
    x = torch.randn(50, 2, 128, generator=g) * 3
    x[0, 0] = 0                                                  # all-zero row: scale 1, codes 0
    x[1, 1, :6] = torch.tensor([127.0, 2.5, 3.5, -0.5, -1.5, 0.5])   # amax 127 -> scale 1: exact ties
    x[1, 1, 6:] = 0.25
    codes, scale = quantize_int8_per_row(x.numpy(), "fp32")
    amax = x.abs().amax(dim=-1)
    ref_scale = torch.where(amax == 0, torch.ones_like(amax), amax / 127.0)
    ref = torch.round(x / ref_scale[..., None]).clamp(-127, 127).to(torch.int8)
    assert np.array_equal(scale, ref_scale.numpy())
    assert codes.dtype == np.int8 and np.array_equal(codes, ref.numpy())
    assert list(codes[1, 1, :6]) == [127, 2, 4, 0, -2, 0]
    assert scale[0, 0] == 1.0 and not codes[0, 0].any()


def test_int8_per_tensor_matches_torch_and_error_bound():
    g = torch.Generator().manual_seed(10)
    x = (torch.randn(40, 4, 64, generator=g) * 5).to(torch.bfloat16)
    codes, scale = quantize_int8_per_tensor(x.view(torch.int16).numpy().view(np.uint16), "bf16")
    xf = x.float()
    ref_scale = xf.abs().max() / 127.0
    ref = torch.round(xf / ref_scale).clamp(-127, 127).to(torch.int8)
    assert np.float32(scale) == ref_scale.item() and np.array_equal(codes, ref.numpy())
    err = np.abs(codes.astype(np.float64) * np.float64(scale) - xf.numpy().astype(np.float64))
    assert np.all(err <= np.float64(scale) / 2 * (1 + 1e-6))
    assert np.abs(codes).max() == 127


def test_int8_dequantisation_in_the_attention_inputs():
    from oracle.attention import PagedKV
    rng = np.random.default_rng(12)
    codes = rng.integers(-127, 128, (2, 2, 4, 8)).astype(np.int8)
    sc = rng.random((2, 2, 4)).astype(np.float32)
    kv = PagedKV(codes.view(np.uint8), "int8", "HPD", "per_token_head", sc)     # bytes as stored
    slots = np.array([1, 6])
    for gh in range(2):
        ref = torch.from_numpy(codes[slots // 4, gh, slots % 4]).double().numpy() * \
            sc[slots // 4, gh, slots % 4].astype(np.float64)[:, None]
        assert np.array_equal(kv.tokens(slots, gh), ref)


def test_oracle_inputs_use_each_workloads_own_format():
    # the oracle's view of every named workload is quantised in that workload's format:
    # INT8 scales are amax/127 and FP8 scales amax/448 of the same bf16 values
    from paged_split_kv_stage1_amd.inputs import CONFIGS, make_workload
    from tests.oracle_inputs import oracle_inputs
    for name, cfg in CONFIGS.items():
        w = make_workload(name, batch=1, ctx=[40], rows=1)
        oi = oracle_inputs(w)
        if cfg.get("latent"):            # per (token, 128 channels) scales: amax / 448 of each block
            lat = w.k.float()[..., :w.dv].reshape(*w.k.shape[:-1], w.dv // 128, 128)
            ref = (lat.abs().amax(-1) / 448.0).numpy()
            used = ~w.unused_slots
            assert np.array_equal(oi["latent"].scale[:, 0][used], ref[:, 0][used]), name
            continue
        k = oi["k"]
        assert k.dtype == cfg["kv"] and k.scale_mode == cfg["scale"], name
        if cfg["scale"] == "per_tensor":
            amax = np.float32(w.k.float().abs().max().item())
            assert np.float32(k.scale) == np.float32(amax / np.float32(127.0 if cfg["kv"] == "int8" else 448.0)), name


def test_per_tensor_dequantisation_in_the_attention_inputs():
    # PagedKV with one per-tensor scale multiplies every decoded code by that float32
    # scale (FlashMLA PR #54, "Functionality": symmetric per-tensor K/V scales), checked
    # against torch's own float8 decode in both cache layouts; INT8 codes likewise
    from oracle.attention import PagedKV
    rng = np.random.default_rng(12)
    codes = rng.integers(0, 256, (3, 2, 4, 16)).astype(np.uint8)
    codes[(codes & 0x7F) == 0x7F] = 0x31             # no NaN codes
    sc = np.float32(0.0172119140625 * 1.1)           # not a power of two: a divide would differ
    dec = torch.from_numpy(codes).view(torch.float8_e4m3fn).double().numpy()
    slots = np.array([0, 3, 5, 9, 11])               # (page, slot) = (0,0) (0,3) (1,1) (2,1) (2,3)
    for layout in ("HPD", "PHD"):
        data = codes if layout == "HPD" else np.ascontiguousarray(codes.transpose(0, 2, 1, 3))
        kv = PagedKV(data, "fp8", layout, "per_tensor", sc)
        for g in range(2):
            ref = dec[slots // 4, g, slots % 4] * np.float64(sc)
            assert np.array_equal(kv.tokens(slots, g), ref)
    i8 = rng.integers(-127, 128, (3, 2, 4, 16)).astype(np.int8)
    kv = PagedKV(i8.view(np.uint8), "int8", "HPD", "per_tensor", sc)
    ref = torch.from_numpy(i8).double().numpy()[slots // 4, 1, slots % 4] * np.float64(sc)
    assert np.array_equal(kv.tokens(slots, 1), ref)


def test_scalar_q_scale_dequantisation():
    # FP8 queries with one per-tensor scale: every code decoded by torch times the scale
    from oracle.attention import dequant_q
    rng = np.random.default_rng(13)
    q = rng.integers(0, 256, (5, 4, 32)).astype(np.uint8)
    q[(q & 0x7F) == 0x7F] = 0x44
    qs = np.float32(0.0059814453125 * 3)
    ref = torch.from_numpy(q).view(torch.float8_e4m3fn).double().numpy() * np.float64(qs)
    assert np.array_equal(dequant_q(q, "fp8", qs), ref)
    assert np.array_equal(dequant_q(q, "fp8", np.array(qs)), ref)      # 0-d array form
