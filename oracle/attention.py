"""Read path: one decode step of grouped-query attention and its risk meter.

TEST INFRASTRUCTURE ONLY: nothing on the product path imports this module.

For one (layer, request, KV head) slice with S cached tokens in logical order
(shared prefix first, then the request's suffix; cartridge page, "One kernel
spans cartridge and live KV": both regions form one sequence under one
softmax), and each of the G query heads q_h sharing that KV head:

    l_t  = sm_scale * <q_h, k_t>        exact keys
    l~_t = sm_scale * <q_h, k^_t>       reconstructed (stored) keys
    p = softmax(l),  p~ = softmax(l~)
    out_h = sum_t p~_t v^_t
    TV_h  = 1/2 sum_t |p_t - p~_t|                        (WitCert, Sec. 3)
    c_t   = sm_scale * sum_b ||q_{h,b}|| w_{t,b}           (WitCert, Thm. 2)
    log A = logsumexp(l~ + c) - logsumexp(l~)   (A = E_p~[e^c], Thm. 1, evaluated
                                                 in the log domain, Sec. 3)
    bound_raw = 1/2 (A^2 - 1) = 1/2 expm1(2 log A); +inf when it exceeds the
                largest float32 (Sec. 6.2.4: overflow to +inf is sound)
    meter = min(1, bound_raw)                              (Sec. 3 / Sec. 4.3)

Two-sided form (WitCert Sec. 4.3, Proposition 1), with A- = E_p~[e^{-c}]:
    log A-          = logsumexp(l~ - c) - logsumexp(l~)
    bound_two_sided = 1/2 (A/A- - A-/A) = sinh(log A - log A-); +inf past float32
    meter_two_sided = min(1, bound_raw, bound_two_sided)

Deterministic tanh shape (WitCert Sec. 6.4.2, the shape tanh(max_t Delta_t) of
the compared system, evaluated with the same witness: Delta_t = c_t):
    bound_tanh = tanh(max_t c_t)   (max-merged across splits)

Tier B, the sub-Gaussian certificate of a subtractively dithered cache
(WitCert Sec. 4.2, Lemma 2; the in-kernel form of Sec. 6.2.3):
    var_t   = sm_scale^2 / 12 * sum_c q_c^2 s_{c,t}^2    (s: the key's dither step
              of channel c at token t; 0 for exact keys)
    u_t     = sqrt(2 var_t log(2 S / delta_loc))          (S tokens, joint over t)
    log A_B = logsumexp(l~ + u) - logsumexp(l~)           (A_B = E_p~[e^u])
    bound_b = 1/2 expm1(2 log A_B), meter_b = min(1, bound_b)  (Thm. 1 applied to u)

Value side and the joint output bound (WitCert Sec. 3 and Sec. 4.2 "Value
side and the joint event"), with rho_t = ||v^_t - v_t|| and ||v_t|| stored per
token (rounded up):
    value_err  = sum_t p~_t rho_t
    v_norm_max = max_t ||v_t||
    out_bound  = 2 meter v_norm_max + value_err  >= ||y - y^||,
                 y = sum_t p_t v_t (exact keys and values), y^ = out
  (meter = min(1, bound_raw) bounds TV; with keys stored exactly TV = 0).

Everything is evaluated in float64; nothing is split or reordered beyond what
the definitions state.
"""
from __future__ import annotations

import math

import numpy as np

from .quant import band_coords

FLT_MAX = float(np.finfo(np.float32).max)


def logsumexp(x: np.ndarray, axis: int = -1) -> np.ndarray:
    m = np.max(x, axis=axis, keepdims=True)
    return (m + np.log(np.sum(np.exp(x - m), axis=axis, keepdims=True))).squeeze(axis)


def softmax(x: np.ndarray, axis: int = -1) -> np.ndarray:
    m = np.max(x, axis=axis, keepdims=True)
    e = np.exp(x - m)
    return e / np.sum(e, axis=axis, keepdims=True)


def band_norms(q: np.ndarray, n_bands: int = 16) -> np.ndarray:
    """||q_b|| for each band b (q shape (..., d))."""
    q = np.asarray(q, np.float64)
    coords = band_coords(q.shape[-1], n_bands)
    return np.sqrt(np.sum(q[..., coords] ** 2, axis=-1))


def total_variation(p: np.ndarray, p_tilde: np.ndarray) -> np.ndarray:
    return 0.5 * np.sum(np.abs(p - p_tilde), axis=-1)


def bound_from_log_a(log_a) -> np.ndarray:
    """Theorem 1's 1/2 (A^2 - 1) from log A, +inf past the float32 range."""
    log_a = np.asarray(log_a, np.float64)
    with np.errstate(over="ignore"):
        b = 0.5 * np.expm1(2.0 * log_a)
    return np.where(b > FLT_MAX, np.inf, b)


def tier_b_radius(q, s_key, sm_scale: float, n_tokens: int, delta_loc: float) -> np.ndarray:
    """u_{h,t} of WitCert Sec. 4.2: the radius that bounds the logit error of
    a subtractively dithered key with probability >= 1 - delta_loc jointly
    over n_tokens tokens (Lemma 2: the dither residual of step s is
    sub-Gaussian with proxy s^2 / 12).

    q: (G, d); s_key: (S, d) dither step per token and channel.  Returns (G, S).
    """
    q = np.asarray(q, np.float64)
    s = np.asarray(s_key, np.float64)
    var = (float(sm_scale) ** 2 / 12.0) * ((q * q) @ (s * s).T)
    return np.sqrt(2.0 * var * math.log(2.0 * n_tokens / float(delta_loc)))


def decode_step(q, k_exact, k_hat, v_hat, w16, sm_scale: float, s_key=None, delta_loc=None,
                v_rec=None):
    """One (layer, request, KV head) cell.

    q: (G, d) query heads sharing this KV head (float32 values).
    k_exact, k_hat, v_hat: (S, d) exact keys, reconstructed keys and values.
    w16: (S, B) stored witness (float16) or None when the stored keys are the
         exact keys (then c = 0).
    s_key, delta_loc: (S, d) dither steps of the stored keys and the failure
         probability of Tier B; both given adds u, log_a_b, bound_b_raw, meter_b.
    v_rec: (S, 2) stored value records (rho, ||v||); adds value_err,
         v_norm_max and out_bound.
    Returns a dict of float64 arrays: out (G, d), out_exact (G, d), tv, log_a,
    bound_raw, meter (G,), plus the per-token logits and bounds for checks.
    """
    q = np.asarray(q, np.float64)
    ke = np.asarray(k_exact, np.float64)
    kh = np.asarray(k_hat, np.float64)
    vh = np.asarray(v_hat, np.float64)
    sm = float(sm_scale)
    l_exact = sm * (q @ ke.T)                 # (G, S)
    l_tilde = sm * (q @ kh.T)
    p = softmax(l_exact)
    pt = softmax(l_tilde)
    out = pt @ vh
    out_exact = p @ vh
    tv = total_variation(p, pt)
    if w16 is None:
        c = np.zeros_like(l_tilde)
    else:
        qn = band_norms(q, np.asarray(w16).shape[1])          # (G, B)
        c = sm * (qn @ np.asarray(w16, np.float64).T)         # (G, S)
    log_a = logsumexp(l_tilde + c) - logsumexp(l_tilde)
    bound_raw = bound_from_log_a(log_a)
    meter = np.minimum(1.0, bound_raw)
    log_a_minus = logsumexp(l_tilde - c) - logsumexp(l_tilde)
    with np.errstate(over="ignore"):
        two = np.sinh(log_a - log_a_minus)
    two = np.where(two > FLT_MAX, np.inf, two)
    res = dict(out=out, out_exact=out_exact, tv=tv, log_a=log_a,
               bound_raw=bound_raw, meter=meter, l_exact=l_exact,
               l_tilde=l_tilde, c=c, p=p, p_tilde=pt, log_a_minus=log_a_minus,
               bound_tanh=np.tanh(np.max(c, axis=1)) if c.shape[1] else np.zeros(c.shape[0]),
               bound_two_sided=two, meter_two_sided=np.minimum(np.minimum(1.0, bound_raw), two))
    if s_key is not None and delta_loc is not None:
        u = tier_b_radius(q, s_key, sm, l_tilde.shape[1], delta_loc)
        log_a_b = logsumexp(l_tilde + u) - logsumexp(l_tilde)
        bound_b = bound_from_log_a(log_a_b)
        res.update(u=u, log_a_b=log_a_b, bound_b_raw=bound_b, meter_b=np.minimum(1.0, bound_b))
    if v_rec is not None:
        rec = np.asarray(v_rec, np.float64)
        value_err = pt @ rec[:, 0]
        v_norm_max = float(np.max(rec[:, 1])) if rec.shape[0] else 0.0
        res.update(value_err=value_err, v_norm_max=np.full(value_err.shape, v_norm_max),
                   out_bound=2.0 * meter * v_norm_max + value_err)
    return res


def kv_head_view(per_qhead: np.ndarray, group: int) -> np.ndarray:
    """Any-of-G view: the maximum over the G query heads of each KV head."""
    a = np.asarray(per_qhead)
    return a.reshape(a.shape[:-1] + (a.shape[-1] // group, group)).max(axis=-1)


def merge_partials(parts):
    """Merge per-split (m, z, acc) online-softmax states (flash decoding).

    parts: list of (m, z, acc) with acc = sum_t e^{l_t - m} v_t.  The merged
    state equals the unsplit one exactly (up to rounding); used only to check
    that splitting the sequence does not change the definition.
    """
    m = max(pm for pm, _, _ in parts)
    z = sum(pz * math.exp(pm - m) for pm, pz, _ in parts)
    acc = sum(pa * math.exp(pm - m) for pm, _, pa in parts)
    return m, z, acc


def flawed_dispersion_certificate(p_tilde, c) -> float:
    """The unsound Eq. (1) of WitCert Sec. 3 (kept only to pin our reading).

    1/2 e^{2 c_max} (E_p~[|c - c_bar|] + c_bar (e^{c_max} - 1)), c_bar = E_p~[c].
    """
    p_tilde = np.asarray(p_tilde, np.float64)
    c = np.asarray(c, np.float64)
    cbar = float(np.sum(p_tilde * c))
    cmax = float(np.max(c))
    return 0.5 * math.exp(2 * cmax) * (float(np.sum(p_tilde * np.abs(c - cbar)))
                                        + cbar * (math.exp(cmax) - 1.0))
