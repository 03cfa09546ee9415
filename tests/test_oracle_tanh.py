"""Pins of the oracle's deterministic tanh shape (WitCert Sec. 6.4.2: the
compared system's tanh(max_t Delta_t), max-merged across splits, here with
Delta_t = c_t from the same witness).  CPU only.

Soundness is pinned against TV from its definition for errors within c, and
against the sharper oscillation bound TV <= tanh((max eps - min eps) / 4),
which is reached exactly by two tokens with opposite errors."""
import math

import numpy as np
import pytest

from oracle.attention import decode_step, softmax, total_variation

SM = 1.0 / math.sqrt(128.0)


def _cell(lt, c):
    S = len(lt)
    q = np.zeros((1, 128))
    q[0, 0] = 1.0 / SM
    kh = np.zeros((S, 128))
    kh[:, 0] = lt
    w = np.zeros((S, 16))
    w[:, 0] = c
    return decode_step(q, kh, kh, np.zeros((S, 128)), w, SM)


def test_two_tokens_reach_the_oscillation_bound():
    """p~ = (s(x), 1 - s(x)), errors (+C, -C): TV = s(x) - s(x - 2C) peaks at
    x = C with value tanh(C/2) = half of what tanh(max c) allows at most."""
    C = 0.7
    lt = np.array([C / 2, -C / 2])                  # log-odds C
    res = _cell(lt, [C, C])
    pt = softmax(lt)
    p = softmax(lt - np.array([C, -C]))
    tv = total_variation(p, pt)
    assert tv == pytest.approx(math.tanh(C / 2), rel=1e-12)
    assert res["bound_tanh"][0] == pytest.approx(math.tanh(C), rel=1e-15)
    assert tv <= res["bound_tanh"][0]


@pytest.mark.parametrize("seed", range(8))
def test_tanh_shape_is_sound_for_any_errors_within_c(seed):
    rng = np.random.default_rng(300 + seed)
    S = 48
    lt = rng.standard_normal(S) * rng.uniform(0.3, 5.0)
    c = rng.exponential(0.2, size=S) * rng.uniform(0.1, 4.0)
    res = _cell(lt, c)
    assert res["bound_tanh"][0] == pytest.approx(math.tanh(float(np.max(c))), rel=1e-15)
    pt = softmax(lt)
    for trial in range(60):
        eps = c * rng.choice([-1.0, 1.0], size=S) * (1.0 if trial % 3 else rng.uniform(0, 1, S))
        tv = total_variation(softmax(lt - eps), pt)
        assert tv <= math.tanh((eps.max() - eps.min()) / 4) * (1 + 1e-12) + 1e-15
        assert tv <= res["bound_tanh"][0]


def test_capped_where_the_e_form_explodes():
    """One token of mass eta with a huge c: the e-form's bound grows without
    limit while the tanh shape stays below 1."""
    S = 500
    lt = np.zeros(S)
    lt[0] = math.log(1e-3 * (S - 1) / (1 - 1e-3))
    c = np.full(S, 0.01)
    c[0] = 30.0
    res = _cell(lt, c)
    assert res["bound_raw"][0] > 1e18
    assert res["bound_tanh"][0] <= 1.0
