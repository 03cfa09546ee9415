"""Pins of the oracle's fixed-channel outlier bypass (WitCert Sec. 6.2.5: m
outlier RoPE pairs per (layer, KV head), stored exactly beside the INT8 codes
of the per-token group-scale format, and excluded from the group maximum).
CPU only.

Pinned against what the page states and what the mathematics fixes: the key
store's bytes per token match Table 6's B/tok/head column (golden fixture);
with no active slot the format is the plain group-scale one bit for bit; the
bypassed channels reconstruct exactly and leave the group maximum (the scale
of a group falls to that of its other channels); the direction of Table 5
(bypass alone barely moves the certificate, bypass with the maximum
excluded lowers it many times); and Tier B stays sound on fresh dither."""
import json
import math
import os

import numpy as np
import pytest

from oracle.attention import tier_b_radius
from oracle.philox import dither
from oracle.pipeline import RegionSpec, decode_cell, encode_region, key_dither_steps
from oracle.quant import (int8_dither_g32_dequant, int8_dither_g32_quantize, outlier_mask,
                          outlier_values)

SM = 1.0 / math.sqrt(128.0)
GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "witcert_table6_outlier_bytes.json")


def _bf16(x):
    x = np.asarray(x, np.float32)
    return (x.view(np.uint32) & np.uint32(0xFFFF0000)).view(np.float32).astype(np.float64)


def _keys(rng, T, pairs=(), scale=60.0):
    """bf16 keys with massive RoPE pairs: both channels of each pair at least
    `scale` in magnitude, random signs."""
    x = rng.standard_normal((T, 128))
    for j in pairs:
        for c in (j, j + 64):
            x[:, c] = scale * (1.0 + np.abs(x[:, c])) * np.sign(rng.standard_normal(T))
    return _bf16(x)


def test_key_store_bytes_match_table6():
    printed = json.load(open(GOLDEN))["printed"]
    rng = np.random.default_rng(0)
    k = _keys(rng, 40, pairs=(1, 9, 17, 33))
    for m_str, b in printed.items():
        m = int(m_str)
        pairs = np.arange(m)[None, :] * 3                       # m distinct pairs
        spec = RegionSpec("int8g32", "int8g32", outlier_pairs=pairs if m else None)
        enc = encode_region(k, k, spec, 0)
        per_tok = enc.k_codes.itemsize * enc.k_codes.shape[1] + enc.k_scale.itemsize * enc.k_scale.shape[1]
        if m:
            per_tok += 2 * enc.k_out.shape[1]                   # 16-bit stored values
        assert per_tok == b, (m, per_tok, b)


def test_no_active_slot_is_the_plain_format():
    rng = np.random.default_rng(1)
    x = _keys(rng, 50, pairs=(5,))
    xi = dither(3, 1, 0, 0, np.arange(50), 128)
    c0, s0, _ = int8_dither_g32_quantize(x, xi)
    for pairs in ([], [64, -1, 200], ):
        mask, active = outlier_mask(pairs)
        assert not mask.any() and not any(active)
        c1, s1, _ = int8_dither_g32_quantize(x, xi, bypass=mask)
        np.testing.assert_array_equal(c0, c1)
        np.testing.assert_array_equal(s0.view(np.uint16), s1.view(np.uint16))
    mask, active = outlier_mask([7, 7, 70, 2])                  # a repeat and an out-of-range index
    assert active == [True, False, False, True]
    assert set(np.flatnonzero(mask)) == {2, 7, 66, 71}
    ov = outlier_values(x, [7, 7, 70, 2])
    np.testing.assert_array_equal(ov[:, 0], x[:, 7])
    np.testing.assert_array_equal(ov[:, 1], x[:, 71])
    assert np.all(ov[:, 2:6] == 0)
    np.testing.assert_array_equal(ov[:, 6], x[:, 2])


def test_bypassed_channels_are_exact_and_leave_the_group_maximum():
    rng = np.random.default_rng(2)
    P = 9                                                        # channels 9 (group 0) and 73 (group 2)
    x = _keys(rng, 200, pairs=(P,), scale=500.0)
    xi = dither(11, 2, 3, 1, np.arange(200), 128)
    mask, _ = outlier_mask([P])
    codes, s, clipped = int8_dither_g32_quantize(x, xi, bypass=mask)
    assert clipped == 0
    assert np.all(codes[:, [P, P + 64]] == 0)
    xh = int8_dither_g32_dequant(codes, s, xi, bypass=mask, x_bypass=x)
    np.testing.assert_array_equal(xh[:, mask], x[:, mask])
    rest = np.abs(np.where(mask[None, :], 0.0, x)).reshape(200, 4, 32).max(axis=2)
    expect = (rest.astype(np.float32) / np.float32(126.5)).astype(np.float32).astype(np.float16)
    np.testing.assert_array_equal(s.view(np.uint16), expect.view(np.uint16))
    # kept in the maximum, the massive pair sets its two groups' steps
    _, s_in, _ = int8_dither_g32_quantize(x, xi, bypass=mask, amax_excludes_bypass=False)
    assert np.all(s_in[:, 0].astype(np.float64) > 50 * s[:, 0].astype(np.float64))
    assert np.all(s_in[:, 2].astype(np.float64) > 50 * s[:, 2].astype(np.float64))
    np.testing.assert_array_equal(s_in[:, [1, 3]].view(np.uint16), s[:, [1, 3]].view(np.uint16))
    r = (xh - x)[:, ~mask]
    step = np.repeat(s.astype(np.float64), 32, axis=1)[:, ~mask]
    assert np.all(np.abs(r) <= 0.5 * step * (1 + 1e-4))


def test_table5_direction_bypass_needs_the_amax_exclusion():
    """Four injected massive RoPE pairs (the page's controlled experiment):
    bypassing them alone barely lowers the Tier B radius; also excluding
    them from the group maximum lowers it many times."""
    rng = np.random.default_rng(3)
    pairs = [3, 20, 41, 58]
    T = 512
    x = _keys(rng, T, pairs=pairs, scale=60.0)
    xi = dither(5, 0, 0, 0, np.arange(T), 128)
    q = rng.standard_normal((8, 128))
    mask, _ = outlier_mask(pairs)
    radii = {}
    for name, byp, excl in (("none", None, True), ("bypass", mask, False), ("bypass+exclude", mask, True)):
        _, s, _ = int8_dither_g32_quantize(x, xi, bypass=byp, amax_excludes_bypass=excl)
        steps = np.repeat(s.astype(np.float64), 32, axis=1)
        if byp is not None:
            steps[:, byp] = 0.0
        radii[name] = np.median(tier_b_radius(q, steps, SM, T, 1e-6))
    assert radii["bypass"] <= radii["none"]
    assert radii["bypass"] >= 0.8 * radii["none"]                  # bypass alone: a small change
    assert radii["bypass+exclude"] <= radii["bypass"] / 10.0      # with the exclusion: many times lower


@pytest.mark.parametrize("seed", range(4))
def test_tier_b_and_tier_a_sound_with_the_bypass(seed):
    rng = np.random.default_rng(50 + seed)
    S = 600
    pairs = np.array([[3, 20, 41, 58]])
    k = _keys(rng, S, pairs=pairs[0], scale=30.0)
    q = _bf16(rng.standard_normal((4, 128)) * rng.uniform(0.5, 2.0))
    for trial in range(3):
        spec = RegionSpec("int8g32", "int8g32", seed=seed * 100 + trial, layer=2, stream=trial,
                          outlier_pairs=pairs)
        enc = encode_region(k, k, spec, 0)
        np.testing.assert_array_equal(enc.k_hat[:, enc.k_bypass], k[:, enc.k_bypass])
        steps = key_dither_steps(enc, spec, S)
        assert np.all(steps[:, enc.k_bypass] == 0) and np.all(steps[:, ~enc.k_bypass] > 0)
        res = decode_cell(q, [(k, enc, spec)], SM, delta_loc=1e-3)
        eps = res["l_tilde"] - res["l_exact"]
        assert np.all(np.abs(eps) <= res["u"])
        assert np.all(res["tv"] <= res["bound_b_raw"])
        assert np.all(res["tv"] <= res["bound_raw"])


def test_bypass_rejects_keys_that_are_not_16_bit_exact():
    x = np.full((2, 128), 1.0 + 2.0 ** -12)                        # not bf16-exact
    with pytest.raises(ValueError):
        outlier_values(x, [1])
