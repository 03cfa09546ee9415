"""Pins of the oracle's value side and joint output bound (WitCert Sec. 3:
||y - y^|| <= 2 TV max_t ||v_t|| + sum_t p~_t rho_t; Sec. 4.2 "Value side and
the joint event").  CPU only.

The output bound is checked against the actual output error computed from
its definition (exact keys and values against the stored ones), on a case
where it is tight, and the stored value records against numpy's norms."""
import math

import numpy as np
import pytest

from oracle.attention import decode_step, softmax
from oracle.pipeline import RegionSpec, decode_cell, encode_region
from oracle.quant import value_witness

SM = 1.0 / math.sqrt(128.0)


def _bf16(x):
    return np.asarray(x, np.float32).astype(np.float64)   # float32-exact inputs


def test_value_records_round_up_to_one_fp16_step():
    rng = np.random.default_rng(1)
    v = _bf16(rng.standard_normal((300, 128)) * rng.uniform(0.01, 30.0, size=(300, 1)))
    vh = v + rng.standard_normal(v.shape) * 1e-3
    rec = value_witness(vh, v).astype(np.float64)
    for col, ref in ((0, np.linalg.norm(vh - v, axis=1)), (1, np.linalg.norm(v, axis=1))):
        assert np.all(rec[:, col] >= ref)
        assert np.all(rec[:, col] <= ref * (1 + 2.0 ** -10) + 1e-30)
    assert np.all(value_witness(v, v)[:, 0] == 0)


@pytest.mark.parametrize("fmt", ["fp8", "int8"])
@pytest.mark.parametrize("seed", range(4))
def test_output_bound_dominates_the_actual_output_error(fmt, seed):
    """y from exact keys and exact values, y^ the attention over the stored
    cache: ||y - y^|| <= 2 meter max||v|| + sum p~ rho on every head."""
    rng = np.random.default_rng(40 + seed)
    S = 700
    k = _bf16(rng.standard_normal((S, 128)))
    k[:, :4] *= 8.0
    k = _bf16(k)
    v = _bf16(rng.standard_normal((S, 128)) * rng.uniform(0.5, 4.0))
    q = _bf16(rng.standard_normal((4, 128)) * rng.uniform(0.5, 3.0))
    spec = RegionSpec(fmt, fmt, seed=seed, layer=3, stream=seed, value_witness=True)
    enc = encode_region(k, v, spec, 1)
    res = decode_cell(q, [(k, enc, spec)], SM)
    y = softmax(SM * (q @ k.T)) @ v
    err = np.linalg.norm(y - res["out"], axis=1)
    assert np.all(err <= res["out_bound"])
    assert np.all(res["out_bound"] >= res["value_err"])
    # the value term alone is the error of the output with exact keys
    y_vk = res["p_tilde"] @ v
    assert np.all(np.linalg.norm(y_vk - res["out"], axis=1) <= res["value_err"])


def test_output_bound_is_tight_for_a_shared_value_error():
    """Keys stored exactly (TV = 0) and one error vector e on every token:
    y - y^ = -e exactly, and the bound is ||e|| up to the fp16 round-up."""
    rng = np.random.default_rng(7)
    S = 200
    k = rng.standard_normal((S, 128))
    v = rng.standard_normal((S, 128))
    e = rng.standard_normal(128) * 1e-2
    vh = v + e[None, :]
    q = rng.standard_normal((2, 128))
    rec = value_witness(vh, v)
    res = decode_step(q, k, k, vh, None, SM, v_rec=rec)
    y = softmax(SM * (q @ k.T)) @ v
    err = np.linalg.norm(y - res["out"], axis=1)
    assert np.allclose(err, np.linalg.norm(e), rtol=1e-12)
    assert np.all(res["meter"] == 0.0)
    assert np.all(res["out_bound"] >= err)
    assert np.all(res["out_bound"] <= err * (1 + 2.0 ** -10))


def test_two_region_norm_maximum_spans_both_regions():
    rng = np.random.default_rng(8)
    kp, ks = _bf16(rng.standard_normal((50, 128))), _bf16(rng.standard_normal((90, 128)))
    vp = _bf16(rng.standard_normal((50, 128)) * 5.0)             # the larger norms sit in the prefix
    vs = _bf16(rng.standard_normal((90, 128)))
    sp = RegionSpec("bf16", "fp8", witness=False, exact_k=False, value_witness=True)
    ss = RegionSpec("fp8", "fp8", value_witness=True)
    ep, es = encode_region(kp, vp, sp, 0), encode_region(ks, vs, ss, 0)
    q = rng.standard_normal((4, 128))
    res = decode_cell(q, [(kp, ep, sp), (ks, es, ss)], SM)
    top = max(np.max(np.linalg.norm(vp, axis=1)), np.max(np.linalg.norm(vs, axis=1)))
    assert np.all(res["v_norm_max"] >= top) and np.all(res["v_norm_max"] <= top * (1 + 2.0 ** -10))
    pt = res["p_tilde"]
    rho = np.concatenate([ep.v_rec[:, 0], es.v_rec[:, 0]]).astype(np.float64)
    np.testing.assert_allclose(res["value_err"], pt @ rho, rtol=1e-15)
    assert np.all(ep.v_rec[:, 0] > 0)                            # FP8 values: rho > 0
