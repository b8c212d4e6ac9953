"""Pins of the oracle's number formats against torch's independent implementations
and against values fixed by the OCP E4M3FN definition."""
import numpy as np
import pytest
import torch

from oracle.formats import bf16_bits_to_f64, e4m3_code_to_f64, f64_to_e4m3_rne


def test_e4m3_decode_all_codes_match_torch():
    codes = torch.arange(256, dtype=torch.int32).to(torch.uint8)
    ref = codes.view(torch.float8_e4m3fn).to(torch.float64).numpy()
    got = e4m3_code_to_f64(codes.numpy())
    nan = np.isnan(ref)
    assert np.array_equal(nan, np.isnan(got))
    assert set(np.nonzero(nan)[0].tolist()) == {0x7F, 0xFF}
    assert np.array_equal(ref[~nan], got[~nan])
    assert np.array_equal(np.signbit(ref[~nan]), np.signbit(got[~nan]))


@pytest.mark.parametrize("code,value", [(0x7E, 448.0), (0xFE, -448.0), (0x38, 1.0), (0x08, 2.0 ** -6),
                                        (0x07, 7 * 2.0 ** -9), (0x01, 2.0 ** -9), (0x00, 0.0),
                                        (0x40, 2.0), (0x3C, 1.5), (0x77, 240.0), (0x78, 256.0)])
def test_e4m3_known_values(code, value):
    assert e4m3_code_to_f64(np.array([code]))[0] == value


def test_e4m3_negative_zero():
    assert np.signbit(e4m3_code_to_f64(np.array([0x80]))[0])
    assert f64_to_e4m3_rne(np.array([-0.0]))[0] == 0x80


def _sweep_values(rng):
    vals = e4m3_code_to_f64(np.arange(0, 0x7F))
    mids = (vals[1:] + vals[:-1]) / 2                       # exact ties
    nudged = np.concatenate([np.nextafter(mids.astype(np.float32), np.float32(0)),
                             np.nextafter(mids.astype(np.float32), np.float32(1e9))]).astype(np.float64)
    rnd = np.ldexp(rng.uniform(1, 2, 20000), rng.integers(-14, 9, 20000))
    x = np.concatenate([vals, mids, nudged, rnd, [448.0, 447.9, 2.0 ** -10, 3 * 2.0 ** -11]])
    x = np.clip(x, -448, 448)
    return np.concatenate([x, -x]).astype(np.float32)


def test_e4m3_encode_matches_torch_cast_after_clamp():
    x = _sweep_values(np.random.default_rng(0))
    ref = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    got = f64_to_e4m3_rne(x.astype(np.float64))
    assert np.array_equal(ref, got)


def test_e4m3_encode_ties_to_even():
    # 1 + 1/16 is halfway between 1 (0x38, even) and 1.125 (0x39): -> 0x38
    # 1 + 3/16 is halfway between 1.125 (0x39) and 1.25 (0x3A, even): -> 0x3A
    # 432 is halfway between 416 (0x7D) and 448 (0x7E, even): -> 0x7E
    got = f64_to_e4m3_rne(np.array([1.0625, 1.1875, 432.0, 2.0 ** -10, 3 * 2.0 ** -10]))
    assert got.tolist() == [0x38, 0x3A, 0x7E, 0x00, 0x02]


def test_e4m3_encode_rejects_out_of_range():
    with pytest.raises(ValueError):
        f64_to_e4m3_rne(np.array([449.0]))
    with pytest.raises(ValueError):
        f64_to_e4m3_rne(np.array([np.nan]))


def test_bf16_decode_matches_torch():
    bits = torch.arange(-32768, 32768, dtype=torch.int32).to(torch.int16)
    ref = bits.view(torch.bfloat16).to(torch.float64).numpy()
    got = bf16_bits_to_f64(bits.numpy())
    nan = np.isnan(ref)
    assert np.array_equal(nan, np.isnan(got))
    assert np.array_equal(ref[~nan], got[~nan])
