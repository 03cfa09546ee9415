"""GPU parity of the meter at its numeric edges (WitCert Sec. 3 numerics:
log-domain evaluation, the trivial bound on overflow; Sec. 4.3: min(1, .);
Sec. 6.2.4: fp32 overflow to +inf is sound and counts as over threshold).

Cells are built so that log A takes chosen values: every token of a cell has
the same key, so p~ is uniform and log A equals c, which scales with the
query.  Queries scaled up to several hundred times drive bound_raw through 1,
to either side of the float overflow edge (2 log A = ln(2 FLT_MAX + 1)) and
far past it.  A ramp of logits exercises the lazy rescale of the running
maxima; dithered INT8 keys do the same for Tier B; queries beyond the fp16
range of the witness operand give the trivial bound.  Plans: the team launch,
the per-chunk plan and the vector-ALU kernel.

Bars: outputs within 2e-3 of their norm and TV within 1e-5, as everywhere.
log A: within 1e-5 of the oracle below, and above by at most 1e-5 plus
2^-18 max_t c_t, the upward rounding of c the kernels apply so that the
bound stays sound (c not below its exact value for the stored witness);
bound_raw, meter and the two-sided form are held to the interval that this
log A interval maps to (1e-5 relative slack); within 1e-3 of the overflow
edge both +inf and a finite value are accepted (the float overflow of
1/2 expm1(2 log A) sits there).
Tier B's radius is not rounded in either direction: 1e-5 plus 2^-18 max u on
both sides."""
import math

import numpy as np
import pytest
import torch

from cells import SM_SCALE
from oracle.numerics import e4m3_table
from oracle.pipeline import RegionSpec, decode_cell, encode_region

pytestmark = pytest.mark.gpu

FLT_MAX = float(np.finfo(np.float32).max)
EDGE = 0.5 * math.log(2.0 * FLT_MAX + 1.0)          # log A where bound_raw leaves the float range
RAISE = 2.0 ** -18
G = 4


def _kvq():
    from quantized_kv_cache_gqa_amd import kvq
    return kvq


PLANS = {"team": 0, "per-chunk": 0x01, "vector-alu": 0x02}


def run(q, k, v, fmt, plan, tier_b=None, seed=5):
    """Store k/v (fp32 tensors, bf16-exact) in `fmt` and decode with the full
    meter; returns the GPU outputs and the oracle's result of every cell."""
    kvq = _kvq()
    dev = q.device
    B, Hkv, S, _ = k.shape
    kb, vb = k.to(torch.bfloat16), v.to(torch.bfloat16)
    st = kvq.alloc_stored(B, Hkv, S, fmt, fmt, True, dev)
    kvq.quantize_into(st, kb, vb, seed=seed)
    view = kvq.RegionView(st, S, k_exact=kb, seed=seed)
    status = torch.zeros(4, dtype=torch.int32, device=dev)
    out, m = kvq.decode_attn(q, Hkv, None, view, sm_scale=SM_SCALE, plan_flags=PLANS[plan], status=status,
                             tier_b_delta=tier_b, two_sided=True)
    torch.cuda.synchronize()
    assert int(status[0]) == 0
    p = kvq.plan(q, Hkv, None, view, sm_scale=SM_SCALE, plan_flags=PLANS[plan], tier_b_delta=tier_b,
                 two_sided=True)
    if plan == "team" and tier_b is None:
        assert p["team"] > 0, p
    refs = {}
    for b in range(B):
        for kvh in range(Hkv):
            qq = q[b, kvh * G:(kvh + 1) * G].double().cpu().numpy()
            kk, vv = kb[b, kvh].double().cpu().numpy(), vb[b, kvh].double().cpu().numpy()
            spec = RegionSpec(fmt, fmt, seed=seed, layer=0, stream=b)
            refs[b, kvh] = decode_cell(qq, [(kk, encode_region(kk, vv, spec, kvh), spec)], SM_SCALE,
                                       delta_loc=tier_b)
    return out, {k_: v_.double().cpu().numpy() for k_, v_ in m.items()}, refs


def bound_of(log_a):
    """bound_raw = 1/2 (A^2 - 1) as the kernels report it (+inf past the float range)."""
    if log_a > EDGE + 1.0:
        return math.inf
    b = 0.5 * math.expm1(2.0 * log_a)
    return math.inf if b > FLT_MAX else b


def within(g, lo, hi, rel=1e-5):
    if math.isinf(hi) and math.isinf(g):
        return True
    return lo - rel * max(1.0, abs(lo)) <= g <= hi + rel * max(1.0, abs(hi))


def check(out, m, refs, overflowed=(), tier_a=True):
    """Every cell and head against the oracle under the bars above; heads in
    `overflowed` must report the trivial bound (their witness operand
    overflowed).  tier_a=False: logits of thousands of nats (Tier B's cells),
    where fp32 logits carry errors above the 1e-5 bar: only Tier B is held
    to its bar there, the rest only to what holds at any precision."""
    worst = dict(log_a_excess=0.0, out=0.0, tv=0.0)
    for (b, kvh), ref in refs.items():
        for h in range(G):
            qh = kvh * G + h
            if not tier_a:
                assert 0.0 <= m["tv"][b, qh] <= 1.0 and np.all(np.isfinite(out[b, qh].cpu().numpy()))
            else:
                o, r = out[b, qh].double().cpu().numpy(), ref["out"][h]
                rel = np.linalg.norm(o - r) / max(np.linalg.norm(r), 1e-30)
                assert rel <= 2e-3, (b, qh, rel)
                assert abs(m["tv"][b, qh] - ref["tv"][h]) <= 1e-5, (b, qh, m["tv"][b, qh], ref["tv"][h])
                worst["out"] = max(worst["out"], rel)
                worst["tv"] = max(worst["tv"], abs(m["tv"][b, qh] - ref["tv"][h]))
            if (b, qh) in overflowed:
                assert math.isinf(m["log_a"][b, qh]) and math.isinf(m["bound_raw"][b, qh]), (b, qh)
                assert m["meter"][b, qh] == 1.0 and m["meter_two_sided"][b, qh] == 1.0
                assert m["bound_tanh"][b, qh] == 1.0
                continue
            cmax = float(np.max(ref["c"][h])) if ref["c"].shape[1] else 0.0
            ra, ga = float(ref["log_a"][h]), float(m["log_a"][b, qh])
            if not tier_a:
                assert 0.0 <= m["meter"][b, qh] <= 1.0
                _check_tier_b(m, ref, b, qh, h)
                continue
            lo, hi = ra - 1e-5, ra + 1e-5 + RAISE * cmax
            assert lo <= ga <= hi, (b, qh, ga, ra, cmax)
            worst["log_a_excess"] = max(worst["log_a_excess"], ga - ra)
            gb = float(m["bound_raw"][b, qh])
            if abs(ra - EDGE) < 1e-3 + RAISE * cmax:      # either answer near the overflow edge
                assert math.isinf(gb) or gb >= bound_of(lo) * (1 - 1e-5), (b, qh, gb)
            else:
                assert within(gb, bound_of(lo), bound_of(hi)), (b, qh, gb, bound_of(lo), bound_of(hi))
                assert math.isinf(gb) == math.isinf(ref["bound_raw"][h]), (b, qh, gb, ref["bound_raw"][h])
            gm = float(m["meter"][b, qh])
            assert min(1.0, bound_of(lo)) - 1e-5 <= gm <= min(1.0, bound_of(hi)) + 1e-5, (b, qh, gm)
            # two-sided form: log A- moves down with c, the bound up
            rm, gmn = float(ref["log_a_minus"][h]), float(m["log_a_minus"][b, qh])
            assert rm - 1e-5 - RAISE * cmax <= gmn <= rm + 1e-5, (b, qh, gmn, rm)
            two_lo = math.sinh(min(lo - (rm + 1e-5), 700.0))
            two_hi = math.sinh(min(hi - (rm - 1e-5 - RAISE * cmax), 700.0))
            g2 = float(m["bound_two_sided"][b, qh])
            assert (math.isinf(g2) and two_hi > FLT_MAX * 0.999) or within(g2, two_lo, min(two_hi, math.inf)), \
                (b, qh, g2, two_lo, two_hi)
            assert m["meter_two_sided"][b, qh] <= 1.0
            tl, th = math.tanh(cmax), math.tanh(cmax * (1 + RAISE))
            assert tl - 1e-5 <= m["bound_tanh"][b, qh] <= th + 1e-5, (b, qh)
            if "log_a_b" in m:
                _check_tier_b(m, ref, b, qh, h)
    return worst


def _check_tier_b(m, ref, b, qh, h):
    umax = float(np.max(ref["u"][h]))
    rb, gbb = float(ref["log_a_b"][h]), float(m["log_a_b"][b, qh])
    tol = 1e-5 + RAISE * umax
    assert abs(gbb - rb) <= tol, (b, qh, gbb, rb, umax)
    blo, bhi = bound_of(rb - tol), bound_of(rb + tol)
    gB = float(m["bound_b_raw"][b, qh])
    if abs(rb - EDGE) >= 1e-3 + tol:
        assert within(gB, blo, bhi), (b, qh, gB, blo, bhi)
        assert math.isinf(gB) == math.isinf(ref["bound_b_raw"][h]), (b, qh, gB)
    assert min(1.0, blo) - 1e-5 <= m["meter_b"][b, qh] <= min(1.0, bhi) + 1e-5


# log A targets of the 16 query heads (2 requests x 2 KV heads x 4)
TARGETS = [0.0, 0.05, 0.3, 0.5493, 0.5494, 1.0, 2.0, 5.0, 10.0, 20.0, 44.69, 44.70, 44.72, 50.0, 80.0, 200.0]


def _same_key_cells(dev, S, fmt, seed):
    """Every token of a cell holds one key, values are random; the query
    direction is random, its scale free.  FP8: channel 0 of the key is 2^22
    and the query's channel 0 is 0; the other channels lie below the E4M3
    subnormal floor of that token's scale, so the stored key is (2^22, 0,
    .., 0): l~ = 0 exactly however large the query, c = sm_scale sum_b
    ||q_b|| w_b with w the other channels' norms per band, and log A = c."""
    g = torch.Generator(device="cpu").manual_seed(seed)
    k0 = torch.randn(2, 2, 1, 128, generator=g)
    q0 = torch.randn(2, 2 * G, 128, generator=g)
    if fmt == "fp8":
        k0[..., 0] = 2.0 ** 22
        q0[..., 0] = 0.0
    else:
        k0[..., [3, 40, 77, 101]] *= 8.0
    k = k0.expand(2, 2, S, 128).contiguous()
    v = torch.randn(2, 2, S, 128, generator=g)
    return q0.to(dev), k.to(torch.bfloat16).float().to(dev), v.to(dev)


@pytest.mark.parametrize("plan", list(PLANS))
def test_meter_through_one_the_overflow_edge_and_past_it(gpu_lib, plan):
    dev = torch.device("cuda")
    S = 1600
    q0, k, v = _same_key_cells(dev, S, "fp8", 31)
    _, _, refs1 = run(q0, k[:, :, :64].contiguous(), v[:, :, :64].contiguous(), "fp8", "per-chunk")
    q = q0.clone()
    for b in range(2):
        for qh in range(2 * G):
            c1 = float(refs1[b, qh // G]["c"][qh % G][0])         # c of the unscaled query (nats)
            q[b, qh] *= TARGETS[b * 2 * G + qh] / c1
    out, m, refs = run(q, k, v, "fp8", plan)
    la = [float(refs[b, qh // G]["log_a"][qh % G]) for b in range(2) for qh in range(2 * G)]
    assert np.allclose(la, TARGETS, rtol=1e-6, atol=1e-9), la   # the construction: log A = c
    assert all(np.all(r["l_tilde"] == 0.0) and r["tv"].max() == 0.0 for r in refs.values())
    w = check(out, m, refs)
    inf = [(b, qh) for b in range(2) for qh in range(2 * G) if math.isinf(m["bound_raw"][b, qh])]
    assert len(inf) >= 3 and m["meter"].max() == 1.0 and m["meter"].min() == 0.0
    print(f"[meter edge, {plan}] worst {w}, +inf bounds {len(inf)}/16", flush=True)


@pytest.mark.parametrize("plan", list(PLANS))
def test_lazy_rescale_on_a_ramp_of_logits(gpu_lib, plan):
    """Keys carry a component along the group's mean query that grows along
    the sequence: logits climb by about 25 nats, so every running maximum
    moves many times, across tiles, chunks and team members."""
    dev = torch.device("cuda")
    gen = torch.Generator(device="cpu").manual_seed(9)
    S = 3000
    q = torch.randn(2, 2 * G, 128, generator=gen)
    k = torch.randn(2, 2, S, 128, generator=gen)
    v = torch.randn(2, 2, S, 128, generator=gen)
    for b in range(2):
        for kvh in range(2):
            u = q[b, kvh * G:(kvh + 1) * G].sum(0)
            u = u / u.norm()
            proj = float(q[b, kvh * G:(kvh + 1) * G].matmul(u).min())
            gamma = 25.0 / (SM_SCALE * proj)
            k[b, kvh] += torch.linspace(0.0, 1.0, S)[:, None] * gamma * u[None, :]
    out, m, refs = run(q.to(dev), k.to(torch.bfloat16).float().to(dev), v.to(dev), "fp8", plan)
    lt = refs[0, 0]["l_tilde"]
    assert lt.max() - lt.min() > 20.0
    w = check(out, m, refs)
    print(f"[lazy rescale, {plan}] worst {w}", flush=True)


@pytest.mark.parametrize("plan", ["per-chunk", "vector-alu"])
def test_tier_b_through_one_the_overflow_edge_and_past_it(gpu_lib, plan):
    """Dithered INT8 keys, one 256-token block per cell, every token the same
    key: Tier B's radius is constant, so log A_B = u; queries scaled to put it
    at the targets.  Tier A runs on the same cells (its c varies with the
    dither)."""
    dev = torch.device("cuda")
    S = 256
    q0, k, v = _same_key_cells(dev, S, "int8", 47)
    delta = 1e-6
    _, _, refs1 = run(q0, k, v, "int8", "per-chunk", tier_b=delta)
    q = q0.clone()
    targets = [0.0, 0.2, 0.5493, 1.0, 5.0, 20.0, 44.70, 44.72] * 2
    for b in range(2):
        for qh in range(2 * G):
            u1 = float(refs1[b, qh // G]["u"][qh % G][0])
            q[b, qh] *= targets[b * 2 * G + qh] / u1
    out, m, refs = run(q, k, v, "int8", plan, tier_b=delta)
    lab = [float(refs[b, qh // G]["log_a_b"][qh % G]) for b in range(2) for qh in range(2 * G)]
    assert np.allclose(lab, targets, rtol=1e-6, atol=1e-9), lab
    w = check(out, m, refs, tier_a=False)
    inf = sum(math.isinf(x) for x in m["bound_b_raw"].ravel())
    assert inf >= 2 and m["meter_b"].max() == 1.0
    print(f"[tier B edge, {plan}] worst {w}, +inf bounds {inf}/16", flush=True)


@pytest.mark.parametrize("plan", list(PLANS))
def test_witness_operand_overflow_gives_the_trivial_bound(gpu_lib, plan):
    """Queries so large that a band factor sm_scale ||q_b|| log2(e) reaches
    2^15, beyond the fp16 operand of the witness dot: the matrix-core
    kernels report log A = bound = +inf, meter 1 and tanh 1 (the trivial
    bound), even where the exact c is 0 (keys stored exactly: E4M3 values times 2^-20, absmax
    448 * 2^-20, so the scale is 2^-20 and the witness 0).  Outputs and the
    TV still match the oracle."""
    dev = torch.device("cuda")
    gen = np.random.default_rng(3)
    S = 900
    tab = e4m3_table()[:0x7F]
    codes = gen.integers(0, 0x7F, (2, 2, S, 128))
    sign = np.where(gen.random((2, 2, S, 128)) < 0.5, -1.0, 1.0)
    k = tab[codes] * sign * 2.0 ** -20
    k[..., 0] = 448.0 * 2.0 ** -20
    v = gen.standard_normal((2, 2, S, 128))
    q = gen.standard_normal((2, 2 * G, 128)) * 2.0e5
    kt = torch.from_numpy(k).float().to(dev)
    out, m, refs = run(torch.from_numpy(q).float().to(dev), kt, torch.from_numpy(v).float().to(dev), "fp8", plan)
    for ref in refs.values():
        assert np.all(ref["c"] == 0.0) and np.all(ref["log_a"] == 0.0)   # stored exactly
    # the vector-ALU kernel forms c in fp32 with no fp16 operand: no overflow
    # there, it reports the exact c = 0
    over = {(b, qh) for b in range(2) for qh in range(2 * G)} if plan != "vector-alu" else set()
    w = check(out, m, refs, overflowed=over)
    print(f"[operand overflow, {plan}] worst {w}", flush=True)
