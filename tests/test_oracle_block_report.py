"""Pins of the oracle's block-decomposable risk report (WitCert Sec. 6.3.5:
replacing block j by its exact values lowers A by exactly its contribution,
so blocks are paged in by decreasing contribution).  CPU only.

Checked against identities the page states or the definitions force:
contributions add up to A - 1 (from the meter's log A), masses to 1,
replacing a block's keys by exact keys (p~ held fixed) lowers A by exactly
its contribution, Tier B's block contribution mass_j (e^{u_j} - 1), and the
order against a brute-force ranking."""
import math

import numpy as np
import pytest

from oracle.pipeline import RegionSpec, block_report, decode_cell, encode_region

SM = 1.0 / math.sqrt(128.0)


def _cell(rng, fmt, n_pre, n_suf, delta=None):
    kp = rng.standard_normal((n_pre, 128)).astype(np.float32).astype(np.float64)
    ks = rng.standard_normal((n_suf, 128)).astype(np.float32).astype(np.float64)
    ks[:, :4] *= 8.0
    ks = ks.astype(np.float32).astype(np.float64)
    sp = RegionSpec("bf16", "bf16", witness=False, exact_k=False)
    ss = RegionSpec(fmt, fmt, seed=5, layer=1, stream=2)
    ep, es = encode_region(kp, kp, sp, 0), encode_region(ks, ks, ss, 0)
    q = (rng.standard_normal((4, 128)) * 2.0).astype(np.float32).astype(np.float64)
    regs = ([(kp, ep, sp)] if n_pre else []) + [(ks, es, ss)]
    return decode_cell(q, regs, SM, delta_loc=delta), ep, es


@pytest.mark.parametrize("fmt", ["fp8", "int8"])
def test_contributions_add_up_to_a_minus_one(fmt):
    rng = np.random.default_rng(1)
    res, _, _ = _cell(rng, fmt, 300, 1000)
    rep = block_report(res, [300, 1000], [300, 1280])
    assert rep["block_mass"].shape == (4, 2 + 5)
    np.testing.assert_allclose(rep["block_mass"].sum(axis=1), 1.0, rtol=1e-12)
    np.testing.assert_allclose(rep["block_excess"].sum(axis=1), np.expm1(res["log_a"]), rtol=1e-10)
    assert np.all(rep["block_excess"][:, :2] == 0.0)          # BF16 cartridge: c = 0
    assert np.all(rep["block_mass"][:, 2:6] > 0.0)
    assert np.all(rep["block_mass"][:, 6] == 0.0)             # capacity past the 1000 tokens


def test_replacing_a_block_lowers_a_by_its_contribution():
    rng = np.random.default_rng(2)
    res, _, _ = _cell(rng, "fp8", 0, 900)
    rep = block_report(res, [900], [900])
    pt, c = res["p_tilde"], res["c"]
    A = np.sum(pt * np.exp(c), axis=1)
    for j in range(4):
        c2 = c.copy()
        c2[:, 256 * j:256 * (j + 1)] = 0.0                    # block j exact: c = 0
        A2 = np.sum(pt * np.exp(c2), axis=1)
        np.testing.assert_allclose(A - A2, rep["block_excess"][:, j], rtol=1e-10)


def test_tier_b_block_contribution_and_order():
    rng = np.random.default_rng(3)
    res, _, es = _cell(rng, "int8", 100, 1100, delta=1e-4)
    rep = block_report(res, [100, 1100], [128, 1280])
    # u is shared by a block: its contribution is mass (e^u - 1) and they add
    # up to A_B - 1
    np.testing.assert_allclose(rep["block_excess_b"].sum(axis=1), np.expm1(res["log_a_b"]), rtol=1e-10)
    assert np.all(rep["block_excess_b"][:, 0] == 0.0)         # BF16 cartridge block: u = 0
    for h in range(4):
        brute = sorted(range(rep["block_order"].shape[1]),
                       key=lambda j: (-rep["block_excess_b"][h, j], j))
        assert list(rep["block_order"][h]) == brute
