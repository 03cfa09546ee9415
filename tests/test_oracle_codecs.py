"""Pins of the FP8 E4M3FN codec and of the FP8 per-token quantizer.  CPU only."""
import numpy as np
import torch

from oracle.numerics import (E4M3_MAX, bf16_bits_to_f64, e4m3_decode, e4m3_encode,
                             e4m3_table, f64_to_bf16_bits)
from oracle.quant import fp8_token_dequant, fp8_token_quantize


def test_e4m3_table_closed_form():
    t = e4m3_table()
    finite = t[np.isfinite(t)]
    assert len(finite) == 254                       # 256 minus the two NaNs
    assert np.isnan(t[0x7F]) and np.isnan(t[0xFF])
    assert t[0x7E] == 448.0 and t[0xFE] == -448.0   # largest finite
    assert t[0x08] == 2.0 ** -6                     # smallest normal
    assert t[0x01] == 2.0 ** -9                     # smallest subnormal
    assert t[0x00] == 0.0 and t[0x80] == 0.0 and np.signbit(t[0x80])
    pos = t[:0x7F]
    assert np.all(np.diff(pos) > 0)
    # 8 values per binade for normals: spacing 2^(e-7-3)
    for e in range(1, 15):
        block = pos[e * 8:(e + 1) * 8]
        np.testing.assert_array_equal(np.diff(block), 2.0 ** (e - 10))


def test_e4m3_roundtrip_every_finite_code():
    codes = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], np.uint8)
    vals = e4m3_decode(codes).astype(np.float32)
    np.testing.assert_array_equal(e4m3_encode(vals), codes)


def test_e4m3_midpoints_round_to_even_and_saturate():
    pos = e4m3_table()[:0x7F]
    for c in range(0x7E):
        mid = (pos[c] + pos[c + 1]) / 2                 # exact in float32
        even = c if c % 2 == 0 else c + 1
        assert e4m3_encode(np.float32(mid)) == even
        assert e4m3_encode(np.nextafter(np.float32(mid), np.float32(1e9))) == c + 1
        assert e4m3_encode(np.nextafter(np.float32(mid), np.float32(-1e9))) == c
        assert e4m3_encode(-np.float32(mid)) == (even | 0x80)
    assert e4m3_encode(np.float32(1e6)) == 0x7E
    assert e4m3_encode(np.float32(-465.0)) == 0xFE


def test_e4m3_encode_agrees_with_torch_cast_inside_range():
    """torch's float8_e4m3fn cast is an independent implementation (it does not
    saturate, so only in-range values are compared)."""
    rng = np.random.default_rng(0)
    parts = [rng.standard_normal(200000).astype(np.float32) * s for s in (1e-3, 0.05, 1, 30, 200)]
    pos = e4m3_table()[:0x7F]
    mids = ((pos[:-1] + pos[1:]) / 2).astype(np.float32)
    parts += [mids, -mids, np.nextafter(mids, np.float32(1)), np.nextafter(mids, np.float32(0))]
    y = np.clip(np.concatenate(parts), -E4M3_MAX, E4M3_MAX).astype(np.float32)
    ref = torch.from_numpy(y).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    np.testing.assert_array_equal(e4m3_encode(y), ref)


def test_bf16_rounding_agrees_with_torch():
    rng = np.random.default_rng(1)
    x = (rng.standard_normal(100000) * 10 ** rng.uniform(-5, 5, 100000)).astype(np.float32)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    np.testing.assert_array_equal(f64_to_bf16_bits(x.astype(np.float64)), ref)
    np.testing.assert_array_equal(
        bf16_bits_to_f64(ref), torch.from_numpy(ref.view(np.int16)).view(torch.bfloat16).float().numpy())


def test_fp8_token_quantizer_properties():
    rng = np.random.default_rng(2)
    x = f = rng.standard_normal((500, 128))
    x[:, [3, 50, 77, 100]] *= 8
    x = bf16_bits_to_f64(f64_to_bf16_bits(x))           # exact bf16 inputs
    codes, s = fp8_token_quantize(x)
    assert s.dtype == np.float32
    amax = np.max(np.abs(x), axis=1)
    np.testing.assert_array_equal(s, (amax.astype(np.float32) / np.float32(448)).astype(np.float32))
    xh = fp8_token_dequant(codes, s)
    # the absmax element maps to +-448 (code 0x7E / 0xFE) up to one fp32 rounding of s
    top = np.argmax(np.abs(x), axis=1)
    assert np.all((codes[np.arange(500), top] & 0x7F) == 0x7E)
    # per-element error at most half an E4M3 step at that magnitude (relative 2^-4) or
    # half the subnormal step 2^-10 * s
    err = np.abs(xh - x)
    assert np.all(err <= np.maximum(np.abs(x) * 2.0 ** -4, s[:, None] * 2.0 ** -10) * (1 + 1e-6))
    # all-zero token: scale 1, codes 0
    z = np.zeros((1, 128))
    cz, sz = fp8_token_quantize(z)
    assert sz[0] == 1.0 and np.all(cz == 0)
