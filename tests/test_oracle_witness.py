"""Pins of the witness (WitCert Sec. 4.1): band layout, Lemma 1 (RoPE band
unitarity), Theorem 2 (Cauchy-Schwarz logit bound, tight case), fp16 round-up.
CPU only."""
import math

import numpy as np

from oracle.attention import band_norms
from oracle.numerics import fp16_round_up
from oracle.quant import band_coords, witness

THETA = 1.0e6


def rope(x, pos, theta=THETA):
    """Rotate-half RoPE written independently here: pair j = (j, j + d/2)."""
    x = np.asarray(x, np.float64)
    d = x.shape[-1]
    half = d // 2
    inv = theta ** (-np.arange(half) * 2.0 / d)
    ang = np.asarray(pos, np.float64)[..., None] * inv
    c, s = np.cos(ang), np.sin(ang)
    a, b = x[..., :half], x[..., half:]
    return np.concatenate([a * c - b * s, a * s + b * c], axis=-1)


def test_band_layout_partitions_coordinates_into_whole_pairs():
    bc = band_coords(128, 16)
    assert bc.shape == (16, 8)
    assert sorted(bc.ravel().tolist()) == list(range(128))
    for row in bc:
        first = set(int(i) for i in row if i < 64)
        second = set(int(i) - 64 for i in row if i >= 64)
        assert first == second and len(first) == 4          # whole RoPE pairs
        assert max(first) - min(first) == 3                  # contiguous pairs


def test_lemma1_witness_invariant_under_rope():
    rng = np.random.default_rng(0)
    r = rng.standard_normal((64, 128))
    w0, _ = witness(r, np.zeros_like(r))
    for n in [1, 7, 632, 12627, 131071, 10 ** 6]:
        rr = rope(r, np.full(64, n))
        w1, _ = witness(rr, np.zeros_like(rr))
        np.testing.assert_allclose(w1, w0, rtol=1e-12)
    # a band mixing coordinates from two pairs only partially would fail this:
    rr = rope(r, np.full(64, 5))
    half_band = np.linalg.norm(rr[:, [0, 1, 2, 3]], axis=1)
    half_band0 = np.linalg.norm(r[:, [0, 1, 2, 3]], axis=1)
    assert np.max(np.abs(half_band - half_band0)) > 1e-3


def test_theorem2_sound_and_tight_when_residual_aligned_with_query():
    rng = np.random.default_rng(1)
    sm = 1 / math.sqrt(128)
    bc = band_coords(128, 16)
    for _ in range(200):
        q = rng.standard_normal(128) * rng.uniform(0.1, 10)
        r = rng.standard_normal(128) * rng.uniform(1e-3, 1)
        w, w16 = witness(r[None], np.zeros((1, 128)))
        qn = band_norms(q[None])[0]
        c = sm * float(qn @ w[0])
        c16 = sm * float(qn @ w16[0].astype(np.float64))
        eps = abs(sm * float(q @ r))
        assert eps <= c * (1 + 1e-12) and c <= c16 * (1 + 1e-12)
        # tight case: r_b = alpha_b q_b with alpha_b > 0 gives equality
        alpha = rng.uniform(0.01, 1, 16)
        ra = np.zeros(128)
        for b in range(16):
            ra[bc[b]] = alpha[b] * q[bc[b]]
        wa, _ = witness(ra[None], np.zeros((1, 128)))
        ca = sm * float(qn @ wa[0])
        assert abs(sm * float(q @ ra) - ca) <= 1e-12 * ca


def test_bound_invariant_under_relative_rope_shift():
    rng = np.random.default_rng(2)
    sm = 1 / math.sqrt(128)
    q = rng.standard_normal(128)
    r = rng.standard_normal((10, 128)) * 0.01
    w, _ = witness(r, np.zeros_like(r))
    c0 = sm * (band_norms(q[None]) @ w.T)
    for m in [3, 999, 65536]:
        c1 = sm * (band_norms(rope(q, m)[None]) @ w.T)
        np.testing.assert_allclose(c1, c0, rtol=1e-12)


def test_fp16_round_up_is_minimal_upper_bound():
    rng = np.random.default_rng(3)
    w = np.concatenate([np.abs(rng.standard_normal(5000)) * 10 ** rng.uniform(-8, 4, 5000),
                        [0.0, 65504.0, 65504.5, 1e6, 2.0 ** -24, 2.0 ** -25]])
    h = fp16_round_up(w)
    hv = h.astype(np.float64)
    assert np.all(hv >= w)
    finite = np.isfinite(hv) & (hv > 0)
    prev = (h.view(np.uint16)[finite] - 1).view(np.float16).astype(np.float64)
    assert np.all(prev < w[finite])
    assert hv[-6 + 0] == 0.0 and np.isinf(hv[-3]) and np.isinf(hv[-4])


def test_witness_zero_for_identity_quantizer():
    x = np.random.default_rng(4).standard_normal((30, 128))
    w, w16 = witness(x, x)
    assert np.all(w == 0) and np.all(w16 == 0)
