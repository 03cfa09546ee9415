"""Pins of the oracle's read path: softmax, TV, Theorem 1 bound, log-domain
numerics, split-merge identity.  CPU only."""
import json
import math
import os

import mpmath
import numpy as np
import pytest

from oracle import attention
from oracle.attention import (bound_from_log_a, decode_step, flawed_dispersion_certificate,
                              logsumexp, merge_partials, softmax, total_variation)

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _counterexample_cell():
    """Two tokens with l~ = (0, 0) and l = (0.1, -0.1): p~ = (1/2, 1/2), eps = (0.1, -0.1)."""
    d = 128
    q = np.zeros((1, d)); q[0, 0] = 1.0
    k_exact = np.zeros((2, d)); k_exact[0, 0] = 0.1; k_exact[1, 0] = -0.1
    k_hat = np.zeros((2, d))
    v = np.eye(2, d)
    return q, k_exact, k_hat, v


def test_counterexample_tv_matches_printed_value():
    g = json.load(open(os.path.join(GOLDEN, "witcert_counterexample.json")))
    q, ke, kh, v = _counterexample_cell()
    res = decode_step(q, ke, kh, v, None, sm_scale=1.0)
    np.testing.assert_allclose(res["p_tilde"][0], g["setup"]["p_tilde"], rtol=0, atol=1e-15)
    np.testing.assert_allclose(res["l_exact"][0] - res["l_tilde"][0], g["setup"]["eps"], atol=1e-15)
    assert round(float(res["tv"][0]), g["printed_digits"]) == g["printed"]["true_tv"]
    # closed form: TV = tanh(0.1) / 2
    assert abs(float(res["tv"][0]) - math.tanh(0.1) / 2) < 1e-15


def test_counterexample_flawed_eq1_matches_printed_value():
    g = json.load(open(os.path.join(GOLDEN, "witcert_counterexample.json")))
    val = flawed_dispersion_certificate(g["setup"]["p_tilde"], g["setup"]["c"])
    assert round(val, g["printed_digits"]) == g["printed"]["eq1_value"]
    assert round(g["printed"]["true_tv"] / val, 1) == g["printed"]["ratio"]


def test_theorem1_value_on_counterexample_is_sound():
    # A = E_p~[e^c] = e^0.1; bound = (e^0.2 - 1) / 2 >= TV = tanh(0.1)/2
    b = float(bound_from_log_a(0.1))
    assert abs(b - (math.exp(0.2) - 1) / 2) < 1e-15
    assert b >= math.tanh(0.1) / 2


def _mp_cell(q, ke, kh, vh, w16, sm):
    """50-digit brute force of the same definitions (no numpy arithmetic)."""
    mpmath.mp.dps = 50
    G, d = q.shape
    S = ke.shape[0]
    out = []
    for h in range(G):
        qh = [mpmath.mpf(float(x)) for x in q[h]]
        le = [mpmath.mpf(sm) * mpmath.fsum(qh[i] * mpmath.mpf(float(ke[t, i])) for i in range(d))
              for t in range(S)]
        lt = [mpmath.mpf(sm) * mpmath.fsum(qh[i] * mpmath.mpf(float(kh[t, i])) for i in range(d))
              for t in range(S)]
        ze = mpmath.fsum(mpmath.exp(x) for x in le)
        zt = mpmath.fsum(mpmath.exp(x) for x in lt)
        p = [mpmath.exp(x) / ze for x in le]
        pt = [mpmath.exp(x) / zt for x in lt]
        tv = mpmath.fsum(abs(a - b) for a, b in zip(p, pt)) / 2
        o = [mpmath.fsum(pt[t] * mpmath.mpf(float(vh[t, i])) for t in range(S)) for i in range(d)]
        # band norms with the rotate-half pairing, 16 bands of 4 pairs
        qn = []
        for b in range(16):
            idx = [4 * b + i for i in range(4)] + [64 + 4 * b + i for i in range(4)]
            qn.append(mpmath.sqrt(mpmath.fsum(qh[i] ** 2 for i in idx)))
        c = [mpmath.mpf(sm) * mpmath.fsum(qn[b] * mpmath.mpf(float(w16[t, b])) for b in range(16))
             for t in range(S)]
        A = mpmath.fsum(pt[t] * mpmath.exp(c[t]) for t in range(S))
        out.append(dict(tv=tv, out=o, log_a=mpmath.log(A), bound=(A * A - 1) / 2))
    return out


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_decode_step_matches_50_digit_brute_force(seed):
    rng = np.random.default_rng(seed)
    G, S, d = 2, 7, 128
    q = rng.standard_normal((G, d)).astype(np.float32).astype(np.float64)
    ke = rng.standard_normal((S, d))
    kh = ke + 0.05 * rng.standard_normal((S, d))
    vh = rng.standard_normal((S, d))
    w16 = np.abs(rng.standard_normal((S, 16))).astype(np.float16)
    sm = 1 / math.sqrt(128)
    res = decode_step(q, ke, kh, vh, w16, sm)
    ref = _mp_cell(q, ke, kh, vh, w16, sm)
    for h in range(G):
        assert abs(float(res["tv"][h]) - float(ref[h]["tv"])) < 1e-13
        assert abs(float(res["log_a"][h]) - float(ref[h]["log_a"])) < 1e-12
        assert abs(float(res["bound_raw"][h]) - float(ref[h]["bound"])) < 1e-11 * max(1, float(ref[h]["bound"]))
        np.testing.assert_allclose(res["out"][h], [float(x) for x in ref[h]["out"]], atol=1e-13)


def _adversarial_trials(rng, n):
    """Peaked/flat p~, large c, extreme sign patterns of eps with |eps| <= c."""
    for i in range(n):
        S = int(rng.integers(2, 40))
        temp = [0.01, 1.0, 10.0, 100.0][i % 4]
        lt = rng.standard_normal(S) * temp
        scale = [1e-3, 0.1, 1.0, 5.0][(i // 4) % 4]
        c = np.abs(rng.standard_normal(S)) * scale
        mode = (i // 16) % 4
        if mode == 0:
            eps = c * rng.choice([-1.0, 1.0], S)          # extreme signs
        elif mode == 1:
            eps = c * np.where(np.arange(S) % 2 == 0, 1.0, -1.0)
        elif mode == 2:
            eps = c * rng.uniform(-1, 1, S)
        else:                                             # all mass moves to one token
            eps = -c.copy(); j = int(rng.integers(S)); eps[j] = c[j]
        yield lt, lt + eps, c


def test_theorem1_sound_per_cell_adversarial():
    rng = np.random.default_rng(12345)
    worst = 0.0
    n = 0
    for lt, le, c in _adversarial_trials(rng, 20000):
        pt = softmax(lt)
        p = softmax(le)
        tv = float(total_variation(p, pt))
        log_a = float(logsumexp(lt + c) - logsumexp(lt))
        bound = float(bound_from_log_a(log_a))
        assert tv <= bound * (1 + 1e-12) + 1e-15, (tv, bound)
        # Lean-stated facts: A >= 1, Z = E_p~[e^{-eps}] <= A and 1 <= A Z
        A = math.exp(log_a)
        Z = float(np.sum(pt * np.exp(-(le - lt))))
        assert A >= 1 - 1e-12 and Z <= A * (1 + 1e-12) and A * Z >= 1 - 1e-12
        worst = max(worst, tv / bound if bound > 0 else 0)
        n += 1
    assert n == 20000 and worst <= 1.0


def test_bound_zero_iff_c_zero_and_identity_quantizer_gives_zero():
    rng = np.random.default_rng(3)
    q = rng.standard_normal((4, 128)).astype(np.float32).astype(np.float64)
    k = rng.standard_normal((50, 128))
    v = rng.standard_normal((50, 128))
    res = decode_step(q, k, k, v, np.zeros((50, 16), np.float16), 1 / math.sqrt(128))
    assert np.all(res["tv"] == 0) and np.all(res["bound_raw"] == 0) and np.all(res["log_a"] == 0)
    res2 = decode_step(q, k, k, v, np.full((50, 16), 1e-3, np.float16), 1 / math.sqrt(128))
    assert np.all(res2["bound_raw"] > 0)


def test_tv_range_and_shift_invariance():
    rng = np.random.default_rng(4)
    for _ in range(200):
        S = int(rng.integers(1, 30))
        a = rng.standard_normal(S) * 3
        b = rng.standard_normal(S) * 3
        tv = float(total_variation(softmax(a), softmax(b)))
        assert 0 <= tv <= 1
        tv2 = float(total_variation(softmax(a + 7.5), softmax(b - 2.25)))
        assert abs(tv - tv2) < 1e-12
        assert float(total_variation(softmax(a), softmax(a))) == 0


def test_log_domain_bound_matches_direct_and_overflows_to_inf():
    rng = np.random.default_rng(5)
    for _ in range(100):
        S = 20
        lt = rng.standard_normal(S)
        c = np.abs(rng.standard_normal(S))
        pt = softmax(lt)
        A = float(np.sum(pt * np.exp(c)))
        log_a = float(logsumexp(lt + c) - logsumexp(lt))
        assert abs(float(bound_from_log_a(log_a)) - 0.5 * (A * A - 1)) < 1e-12 * A * A
    # 1/2 (A^2 - 1) > FLT_MAX  <=>  2 log A > ln(2 FLT_MAX + 1)
    edge = 0.5 * math.log(2 * float(np.finfo(np.float32).max) + 1)
    assert np.isinf(bound_from_log_a(edge + 1e-6))
    assert np.isfinite(bound_from_log_a(edge - 1e-6))
    # c far beyond the float range: log-domain stays finite, bound is +inf
    lt = np.array([0.0, -1000.0]); c = np.array([0.0, 2000.0])
    log_a = float(logsumexp(lt + c) - logsumexp(lt))
    assert abs(log_a - 1000.0) < 1e-9 and np.isinf(bound_from_log_a(log_a))


def test_split_merge_equals_unsplit():
    rng = np.random.default_rng(6)
    S, d = 1000, 16
    lt = rng.standard_normal(S) * 4
    v = rng.standard_normal((S, d))
    m = lt.max(); z = np.exp(lt - m).sum(); acc = np.exp(lt - m) @ v
    cuts = np.sort(rng.choice(np.arange(1, S), 9, replace=False))
    parts = []
    for a, b in zip(np.r_[0, cuts], np.r_[cuts, S]):
        mm = lt[a:b].max()
        parts.append((mm, np.exp(lt[a:b] - mm).sum(), np.exp(lt[a:b] - mm) @ v[a:b]))
    m2, z2, acc2 = merge_partials(parts)
    assert m2 == m
    assert abs(z2 - z) < 1e-12 * z
    np.testing.assert_allclose(acc2 / z2, acc / z, atol=1e-13)


def test_kv_head_view_any_of_g():
    a = np.array([[0.1, 0.5, 0.2, 0.3, 0.9, 0.0, 0.0, 0.1]])
    np.testing.assert_array_equal(attention.kv_head_view(a, 4), [[0.5, 0.9]])
