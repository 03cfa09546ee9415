"""Pins of the oracle's two-sided form (WitCert Sec. 4.3, Proposition 1):
A- = E_p~[e^{-c}], TV <= 1/2 (A/A- - A-/A), meter min(1, 1/2 (A^2 - 1),
1/2 (A/A- - A-/A)).  CPU only.

Pinned against the page's numeric remark, soundness on random cells with
|eps| <= c (TV from its definition), the A- <= 1 <= A ordering, and the
massive-activation regime the proposition is about (linear against
quadratic growth of the two shapes)."""
import json
import math
import os

import numpy as np
import pytest

from oracle.attention import decode_step, softmax, total_variation

SM = 1.0 / math.sqrt(128.0)
GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "witcert_two_sided_remark.json")


def _cell_from(l_tilde, c):
    """A decode_step whose logits are l_tilde (G=1) and whose witness term is
    c: keys along one axis, the witness carried by band 0 with q's band norm 1."""
    S = len(l_tilde)
    q = np.zeros((1, 128))
    q[0, 0] = 1.0 / SM                       # band 0 norm = 1/SM, so c_t = w_t0
    kh = np.zeros((S, 128))
    kh[:, 0] = np.asarray(l_tilde)
    w = np.zeros((S, 16))
    w[:, 0] = np.asarray(c)
    return decode_step(q, kh, kh, np.zeros((S, 128)), w, SM)


def test_pages_remark_two_sided_is_looser_at_a2_aminus06():
    g = json.load(open(GOLDEN))
    a, am = g["setup"]["A"], g["setup"]["A_minus"]
    one = 0.5 * (a * a - 1.0)
    two = 0.5 * (a / am - am / a)
    assert one == g["printed"]["one_sided"]
    assert (two > one) == g["printed"]["two_sided_is_looser"]
    assert two == pytest.approx(1.516667, abs=1e-6)
    # the oracle's sinh form is the same quantity
    assert math.sinh(math.log(a) - math.log(am)) == pytest.approx(two, rel=1e-15)


def test_two_point_cell_matches_the_definitions():
    """Two tokens with equal stored logits and c = (0, 1): A = (1 + e)/2,
    A- = (1 + 1/e)/2, both forms by hand."""
    res = _cell_from([0.0, 0.0], [0.0, 1.0])
    a, am = (1 + math.e) / 2, (1 + 1 / math.e) / 2
    assert math.exp(res["log_a"][0]) == pytest.approx(a, rel=1e-14)
    assert math.exp(res["log_a_minus"][0]) == pytest.approx(am, rel=1e-14)
    assert res["bound_two_sided"][0] == pytest.approx(0.5 * (a / am - am / a), rel=1e-13)
    assert res["meter_two_sided"][0] == min(1.0, 0.5 * (a * a - 1), res["bound_two_sided"][0])


@pytest.mark.parametrize("seed", range(8))
def test_two_sided_bound_is_sound_for_any_errors_within_c(seed):
    """Random stored logits, bounds c and errors |eps| <= c (including the
    extremes eps = +-c): TV(p, p~) from its definition never exceeds either
    form; and A- <= 1 <= A."""
    rng = np.random.default_rng(200 + seed)
    S = 64
    lt = rng.standard_normal(S) * rng.uniform(0.5, 4.0)
    c = rng.exponential(0.3, size=S) * rng.uniform(0.1, 3.0)
    res = _cell_from(lt, c)
    assert res["log_a_minus"][0] <= 0.0 <= res["log_a"][0]
    pt = softmax(lt)
    for trial in range(50):
        eps = c * rng.choice([-1.0, 1.0], size=S) * (1.0 if trial % 2 else rng.uniform(0, 1, S))
        tv = total_variation(softmax(lt - eps), pt)
        assert tv <= res["bound_two_sided"][0] * (1 + 1e-12)
        assert tv <= res["bound_raw"][0] * (1 + 1e-12)


def test_massive_activation_regime_linear_against_quadratic():
    """One token with mass eta and a huge bound C (M = eta e^C >> 1): the
    one-sided shape grows like M^2, the two-sided like M (Sec. 4.3)."""
    eta = 1e-3
    ratios = []
    for C in (10.0, 12.0, 14.0):
        S = 1000
        lt = np.zeros(S)
        lt[0] = math.log(eta * (S - 1) / (1 - eta))      # token 0 has p~ mass eta
        c = np.zeros(S)
        c[0] = C
        res = _cell_from(lt, c)
        M = eta * math.exp(C)
        assert res["bound_raw"][0] == pytest.approx(0.5 * ((1 - eta + M) ** 2 - 1), rel=1e-9)
        ratios.append(res["bound_two_sided"][0] / M)
    assert all(0.4 < r < 0.6 for r in ratios)               # ~ M / 2
