"""Pins of the oracle's Tier B certificate (WitCert Sec. 4.2, Lemma 2; the
in-kernel form of Sec. 6.2.3): the sub-Gaussian radius u_t of a subtractively
dithered INT8 key and A_B = E_p~[e^u] propagated by Theorem 1.  CPU only.

Each pin checks the oracle against something other than its own formula: the
moment generating function of a uniform variable by quadrature, the variance
of the logit error over simulated dither draws, a constant radius (where
log A_B must equal u), exact keys (radius 0), and soundness of the bound on
fresh dither draws."""
import math

import numpy as np
import pytest
from scipy import integrate

from oracle.attention import decode_step, logsumexp, tier_b_radius, total_variation
from oracle.philox import dither
from oracle.pipeline import RegionSpec, decode_cell, encode_region, key_dither_steps
from oracle.quant import int8_dither_dequant, int8_dither_quantize

SM = 1.0 / math.sqrt(128.0)


@pytest.mark.parametrize("lam_a", [1e-3, 0.3, 1.0, 2.5, 6.0, 15.0])
def test_uniform_mgf_and_its_sub_gaussian_proxy(lam_a):
    """Lemma 2: for X uniform on [-a, a], E[e^{lam X}] = sinh(lam a)/(lam a)
    <= e^{(lam a)^2 / 6}; with a = s/2 the proxy is s^2/12, the variance."""
    a = 0.7
    lam = lam_a / a
    mgf, _ = integrate.quad(lambda x: math.exp(lam * x) / (2 * a), -a, a)
    assert mgf == pytest.approx(math.sinh(lam_a) / lam_a, rel=1e-9)
    assert mgf <= math.exp(lam_a ** 2 / 6.0) * (1 + 1e-12)
    s = 2 * a
    var, _ = integrate.quad(lambda x: x * x / (2 * a), -a, a)
    assert var == pytest.approx(s * s / 12.0, rel=1e-12)


def _int8_block(rng, n, d=128, amax=None):
    """n tokens of one 256-token block with per-channel maxima amax (so the
    block's scales are known), as bf16-exact float32 values."""
    x = rng.uniform(-1.0, 1.0, size=(n, d)) * amax[None, :]
    x[0] = amax                                        # the maximum sits on token 0
    return x.astype(np.float32).astype(np.float64)


def test_radius_variance_matches_the_simulated_logit_error():
    """Quantize many blocks with fresh dither through the oracle's INT8 write
    path; the logit error sm <q, k^ - k> over all non-maximum tokens has the
    variance sm^2/12 sum_c q_c^2 s_c^2 that the radius is built from."""
    rng = np.random.default_rng(11)
    d = 128
    amax = rng.uniform(0.2, 3.0, size=d).astype(np.float32).astype(np.float64)
    amax[:4] *= 8.0                                    # outlier channels
    q = rng.standard_normal((1, d))
    errs = []
    s_ref = None
    for blk in range(24):
        x = _int8_block(rng, 256, d, amax)
        xi = rng.uniform(-0.5, 0.5, size=x.shape).astype(np.float32)
        codes, scales, clipped = int8_dither_quantize(x, xi)
        assert clipped == 0
        xh = int8_dither_dequant(codes, scales, xi)
        errs.append(SM * ((xh - x)[1:] @ q[0]))      # token 0 holds the maxima
        s_ref = scales[0].astype(np.float64) if s_ref is None else s_ref
        np.testing.assert_array_equal(scales[0].astype(np.float64), s_ref)
    e = np.concatenate(errs)
    n = 2.0 * 256 / 1e-3
    u = tier_b_radius(q, np.broadcast_to(s_ref, (1, d)), SM, 256, 1e-3)[0, 0]
    var_oracle = u * u / (2.0 * math.log(n))
    assert np.var(e) == pytest.approx(var_oracle, rel=0.08)
    # and the error never leaves the per-channel support |r_c| <= s_c / 2
    assert np.max(np.abs(e)) <= SM * 0.5 * float(np.abs(q[0]) @ s_ref) * (1 + 1e-6)


def test_constant_radius_gives_log_a_equal_to_u():
    """With one dither step s on every channel and token the radius is the
    same for all tokens, so A_B = e^u whatever the logits."""
    rng = np.random.default_rng(3)
    q = rng.standard_normal((4, 128)).astype(np.float32).astype(np.float64)
    S, s, delta = 777, 0.013, 1e-6
    k = rng.standard_normal((S, 128))
    res = decode_step(q, k, k + 0.001, rng.standard_normal((S, 128)), None, SM,
                      s_key=np.full((S, 128), s), delta_loc=delta)
    for h in range(4):
        qn2 = math.fsum(float(x) * float(x) for x in q[h])
        u = math.sqrt(2.0 * (SM * SM * s * s * qn2 / 12.0) * math.log(2.0 * S / delta))
        assert res["log_a_b"][h] == pytest.approx(u, rel=1e-12)
        assert res["bound_b_raw"][h] == pytest.approx(0.5 * math.expm1(2 * u), rel=1e-12)
        assert res["meter_b"][h] == min(1.0, res["bound_b_raw"][h])


def test_keys_stored_exactly_have_radius_zero():
    rng = np.random.default_rng(4)
    q = rng.standard_normal((2, 128))
    k = rng.standard_normal((50, 128))
    res = decode_step(q, k, k, k, None, SM, s_key=np.zeros((50, 128)), delta_loc=1e-4)
    assert np.all(res["u"] == 0.0)
    assert np.all(res["log_a_b"] == 0.0) and np.all(res["bound_b_raw"] == 0.0)


def test_radius_grows_as_the_failure_budget_shrinks():
    rng = np.random.default_rng(5)
    q = rng.standard_normal((3, 128))
    sk = rng.uniform(0.0, 0.05, size=(300, 128))
    prev = None
    for delta in (0.5, 1e-2, 1e-5, 1e-9):
        u = tier_b_radius(q, sk, SM, 300, delta)
        if prev is not None:
            assert np.all(u > prev)
        prev = u


def test_bf16_cartridge_tokens_have_radius_zero_in_a_two_region_cell():
    """A BF16 shared prefix before a dithered INT8 suffix: the prefix tokens'
    steps are 0, the suffix tokens' steps are their block's scales."""
    rng = np.random.default_rng(6)
    kp = rng.standard_normal((40, 128)).astype(np.float32).astype(np.float64)
    ks = rng.standard_normal((300, 128)).astype(np.float32).astype(np.float64)
    sp = RegionSpec("bf16", "bf16", witness=False, exact_k=False)
    ss = RegionSpec("int8", "int8", seed=99, layer=2, stream=1)
    ep = encode_region(kp, kp, sp, 0)
    es = encode_region(ks, ks, ss, 0)
    steps = key_dither_steps(es, ss, 300)
    np.testing.assert_array_equal(steps[255], es.k_scale[0].astype(np.float64))
    np.testing.assert_array_equal(steps[256], es.k_scale[1].astype(np.float64))
    q = rng.standard_normal((4, 128))
    res = decode_cell(q, [(kp, ep, sp), (ks, es, ss)], SM, delta_loc=1e-3)
    assert np.all(res["u"][:, :40] == 0.0) and np.all(res["u"][:, 40:] > 0.0)
    with pytest.raises(ValueError):
        key_dither_steps(encode_region(ks, ks, RegionSpec("fp8", "fp8"), 0), RegionSpec("fp8", "fp8"), 300)


@pytest.mark.parametrize("seed", range(6))
def test_bound_is_sound_on_fresh_dither_draws(seed):
    """Non-adaptive queries, keys quantized with fresh dither (new stream per
    trial): every |eps_t| <= u_t and TV <= bound_B, as the certificate
    promises with probability >= 1 - delta (here delta = 1e-3 per cell)."""
    rng = np.random.default_rng(100 + seed)
    S = 600
    k = rng.standard_normal((S, 128))
    k[:, :4] *= 8.0
    k = k.astype(np.float32).astype(np.float64)
    q = (rng.standard_normal((4, 128)) * rng.uniform(0.5, 3.0)).astype(np.float32).astype(np.float64)
    for trial in range(4):
        spec = RegionSpec("int8", "int8", seed=seed * 1000 + trial, layer=1, stream=trial)
        enc = encode_region(k, k, spec, 0)
        res = decode_cell(q, [(k, enc, spec)], SM, delta_loc=1e-3)
        eps = res["l_tilde"] - res["l_exact"]
        assert np.all(np.abs(eps) <= res["u"])
        assert np.all(res["tv"] <= res["bound_b_raw"])
        # A_B >= 1 and Jensen: log A_B >= E_p~[u] (the bound is never below the mean radius)
        lb = np.sum(res["p_tilde"] * res["u"], axis=1)
        assert np.all(res["log_a_b"] >= lb - 1e-12)
