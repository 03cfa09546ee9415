"""Pins of the oracle's per-token channel-group INT8 format (WitCert Sec.
6.2.3, Table 4: token x G_c-channel groups, G_c = 32 the default, paging-safe)
with the subtractive dither of Sec. 4.2.  CPU only.

Pinned by what the format is for: each token encodes on its own (so a page
holds everything needed: the paging-safety the page cites), the residual
stays within half a step of its group, the residual variance is the uniform
s^2/12 the certificate assumes, and Tier B's radius built from the group steps
matches the simulated logit error."""
import math

import numpy as np
import pytest

from oracle.attention import tier_b_radius
from oracle.philox import dither
from oracle.pipeline import RegionSpec, encode_region, key_dither_steps
from oracle.quant import int8_dither_g32_dequant, int8_dither_g32_quantize

SM = 1.0 / math.sqrt(128.0)


def _x(rng, T):
    x = rng.standard_normal((T, 128)) * rng.uniform(0.1, 3.0, size=(1, 128))
    x[:, :4] *= 8.0
    return x.astype(np.float32).astype(np.float64)


def test_each_token_encodes_on_its_own():
    rng = np.random.default_rng(1)
    x = _x(rng, 300)
    xi = dither(7, 3, 1, 2, np.arange(300), 128)
    codes, s, clipped = int8_dither_g32_quantize(x, xi)
    assert clipped == 0 and s.shape == (300, 4)
    for t in (0, 17, 299):
        c1, s1, _ = int8_dither_g32_quantize(x[t:t + 1], xi[t:t + 1])
        np.testing.assert_array_equal(c1[0], codes[t])
        np.testing.assert_array_equal(s1[0].view(np.uint16), s[t].view(np.uint16))
    # the group step is the group's maximum over 126.5, rounded to fp16
    amax = np.max(np.abs(x.reshape(300, 4, 32)), axis=2)
    assert np.all(np.abs(s.astype(np.float64) - amax / 126.5) <= 2.0 ** -11 * amax / 126.5 + 1e-30)


def test_residual_within_half_a_step_and_uniform_variance():
    rng = np.random.default_rng(2)
    x = _x(rng, 4000)
    xi = rng.uniform(-0.5, 0.5, size=x.shape).astype(np.float32)
    codes, s, _ = int8_dither_g32_quantize(x, xi)
    r = int8_dither_g32_dequant(codes, s, xi) - x
    step = np.repeat(s.astype(np.float64), 32, axis=1)
    assert np.all(np.abs(r) <= 0.5 * step * (1 + 1e-4))        # fp32 rounding of x/s + xi
    # normalized residual r / s is uniform on [-1/2, 1/2]: variance 1/12
    u = (r / step)[step > 0]
    assert np.var(u) == pytest.approx(1.0 / 12.0, rel=0.03)
    assert abs(np.mean(u)) < 0.01


def test_tier_b_radius_from_group_steps_matches_simulated_error():
    rng = np.random.default_rng(3)
    x = _x(rng, 1)
    xs = np.repeat(x, 6000, axis=0)                   # one token, many dither draws
    xi = rng.uniform(-0.5, 0.5, size=xs.shape).astype(np.float32)
    codes, s, _ = int8_dither_g32_quantize(xs, xi)
    q = rng.standard_normal((1, 128))
    err = SM * ((int8_dither_g32_dequant(codes, s, xi) - xs) @ q[0])
    spec = RegionSpec("int8g32", "int8g32", seed=1, stream=0)
    enc = encode_region(x, x, spec, 0)
    steps = key_dither_steps(enc, spec, 1)
    u = tier_b_radius(q, steps, SM, 1, 1e-3)[0, 0]
    var = u * u / (2.0 * math.log(2.0 / 1e-3))
    assert np.var(err) == pytest.approx(var, rel=0.06)
