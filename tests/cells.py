"""Shared test plumbing: run one layer of a workload through the HIP library and
the same cells through the oracle, then compare.

The two sides share only the seeded inputs from ``workloads``: the GPU side
quantizes and attends with libkvq.so, the oracle re-derives every code, scale,
witness and result from the exact inputs on the CPU.
"""
from __future__ import annotations

import math
from typing import Dict, List, Optional, Tuple

import numpy as np
import torch

from oracle.numerics import f64_to_bf16_bits
from oracle.pipeline import RegionSpec, decode_cell, encode_region
from workloads import Config, gen_layer

SM_SCALE = float(np.float32(1.0 / math.sqrt(128.0)))
PREFIX_STREAM = 1_000_000

# kvq_attn_args.plan_flags of every call GpuCase.run and plan() make, unless
# a call names its own (a test or fixture sets it with monkeypatch.setattr)
PLAN_FLAGS = 0


def dither_seed(cfg: Config) -> int:
    return (cfg.seed * 0x9E3779B97F4A7C15) % (1 << 64)


def _spec(cfg: Config, region, layer: int, stream: int, value_witness: bool = False,
          outlier_pairs=None) -> RegionSpec:
    return RegionSpec(k_fmt=region.k_fmt, v_fmt=region.v_fmt, seed=dither_seed(cfg), layer=layer,
                      stream=stream, witness=region.witness, exact_k=region.exact_k,
                      value_witness=value_witness,
                      outlier_pairs=outlier_pairs if region.k_fmt == "int8g32" else None)


def outlier_pairs(cfg: Config, m: int) -> np.ndarray:
    """(h_kv, m) fixed outlier RoPE pairs per KV head: the workload's heavy
    channels' pairs first, then other pairs, a different filler per head; KV
    head 1 also carries a repeated and an out-of-range slot (inactive)."""
    from workloads import outlier_channels
    heavy = sorted({int(c) % 64 for c in outlier_channels(cfg)})
    out = np.zeros((cfg.h_kv, m), np.int32)
    for h in range(cfg.h_kv):
        row = heavy[:m]
        j = 5 + 11 * h
        while len(row) < m:
            if j % 64 not in row:
                row.append(j % 64)
            j += 7
        out[h] = row
        if h == 1 and m >= 4:
            out[h, m - 2] = out[h, 0]                     # repeats slot 0
            out[h, m - 1] = 64 + h                        # no such pair
    return out


class GpuCase:
    """One layer of a workload quantized and stored by the HIP write path."""

    def __init__(self, cfg: Config, layer: int = 0, device="cuda", page_seed: int = 0,
                 fp32_exact: bool = False, value_witness: bool = False, n_outlier_pairs: int = 0):
        from quantized_kv_cache_gqa_amd import kvq
        self.kvq = kvq
        self.cfg, self.layer, self.device = cfg, layer, device
        self.fp32_exact = fp32_exact
        self.value_witness = value_witness
        self.opairs = outlier_pairs(cfg, n_outlier_pairs) if n_outlier_pairs else None
        op_dev = torch.from_numpy(self.opairs).to(device) if n_outlier_pairs else None
        self.inp = gen_layer(cfg, layer, device, want_fp32_keys=fp32_exact)
        G, hkv = cfg.group, cfg.h_kv
        seed = dither_seed(cfg)
        self.prefix_view = None
        self.prefix_store = None
        if cfg.prefix is not None and cfg.prefix.length > 0:
            pr = cfg.prefix
            P = pr.length
            kin = (self.inp["prefix_k32"] if fp32_exact else self.inp["prefix_k"])[None].contiguous()
            vin = self.inp["prefix_v"][None].contiguous()
            if fp32_exact:
                vin = vin.float()
            st = kvq.alloc_stored(1, hkv, P, pr.k_fmt, pr.v_fmt, pr.witness or fp32_exact, device,
                                  value_witness=value_witness,
                                  outlier_pairs=op_dev if pr.k_fmt == "int8g32" else None)
            kvq.quantize_into(st, kin, vin, seed=seed, layer=layer, stream_id=PREFIX_STREAM)
            exact = kin[0] if (pr.exact_k or fp32_exact) else None
            self.prefix_store = st
            self.prefix_view = kvq.RegionView(st, P, k_exact=exact, seed=seed, layer=layer,
                                              stream_id=PREFIX_STREAM,
                                              use_witness=pr.witness or fp32_exact)
        sf = cfg.suffix
        cap = sf.length
        kin = self.inp["suffix_k32"] if fp32_exact else self.inp["suffix_k"]
        vin = self.inp["suffix_v"].float() if fp32_exact else self.inp["suffix_v"]
        st = kvq.alloc_stored(cfg.batch, hkv, cap, sf.k_fmt, sf.v_fmt, sf.witness or fp32_exact, device,
                              value_witness=value_witness,
                              outlier_pairs=op_dev if sf.k_fmt == "int8g32" else None)
        kvq.quantize_into(st, kin, vin, seed=seed, layer=layer, stream_id=0)
        self.suffix_store = st
        exact = kin if (sf.exact_k or fp32_exact) else None
        lens = self.inp["suffix_lens"]
        if sf.paged:
            self.suffix_view = self._paged_view(st, exact, lens, page_seed)
        else:
            self.suffix_view = kvq.RegionView(st, cap, k_exact=exact, lengths=lens, seed=seed,
                                              layer=layer, stream_id=0,
                                              use_witness=sf.witness or fp32_exact)

    def _paged_view(self, st, exact, lens, page_seed):
        """Scatter the dense suffix into shuffled pages [n_pages, h_kv, page, ...]."""
        kvq = self.kvq
        cfg = self.cfg
        ps = cfg.suffix.page_size
        cap = cfg.suffix.length
        if cap % ps:
            raise ValueError("paged suffix capacity must be a multiple of the page size")
        mp = cap // ps
        n_pages = cfg.batch * mp
        perm = torch.from_numpy(np.random.default_rng(page_seed).permutation(n_pages).astype(np.int32))
        table = perm.view(cfg.batch, mp).to(self.device)

        def scatter(t):
            if t is None:
                return None
            b, h, c = t.shape[:3]
            rest = t.shape[3:]
            src = t.view(b, h, mp, ps, *rest).permute(0, 2, 1, 3, *range(4, 4 + len(rest)))
            src = src.reshape(b * mp, h, ps, *rest)
            out = torch.empty_like(src)
            out[table.view(-1).long()] = src
            return out.contiguous()

        paged = kvq.Stored(st.fmt_k, st.fmt_v, scatter(st.k), scatter(st.v), scatter(st.k_scale),
                           scatter(st.v_scale), scatter(st.witness), scatter(st.v_witness),
                           scatter(st.k_outliers), st.outlier_pairs)
        self.page_table = table
        return kvq.RegionView(paged, cap, k_exact=scatter(exact), lengths=lens, page_table=table,
                              page_size=ps, seed=dither_seed(cfg), layer=self.layer, stream_id=0,
                              use_witness=st.witness is not None)

    def run(self, split_tokens: int = 0, meter: bool = True, meter_only: bool = False,
            workspace=None, tier_b_delta=None, value_bound: bool = False, two_sided: bool = False,
            report: bool = False, plan_flags=None, expect_status: Optional[int] = 0, lib=None):
        """One decode (or meter) call; the call's status word must read
        expect_status afterwards (None: not checked)."""
        status = torch.zeros(4, dtype=torch.int32, device=self.device)
        out, m = self.kvq.decode_attn(self.inp["q"], self.cfg.h_kv, self.prefix_view,
                                      self.suffix_view, sm_scale=SM_SCALE, split_tokens=split_tokens,
                                      meter=meter, meter_only=meter_only, workspace=workspace,
                                      tier_b_delta=tier_b_delta, value_bound=value_bound,
                                      two_sided=two_sided, report=report,
                                      plan_flags=PLAN_FLAGS if plan_flags is None else plan_flags,
                                      status=status, lib=lib)
        torch.cuda.synchronize()
        if expect_status is not None:
            assert int(status[0]) == expect_status, f"status word {int(status[0]):#x}"
        return out, m


def plan(case: GpuCase, split_tokens: int = 0, meter_only: bool = False, tier_b_delta=None,
         value_bound: bool = False, two_sided: bool = False, report: bool = False,
         plan_flags=None) -> dict:
    return case.kvq.plan(case.inp["q"], case.cfg.h_kv, case.prefix_view, case.suffix_view,
                         sm_scale=SM_SCALE, split_tokens=split_tokens, meter_only=meter_only,
                         tier_b_delta=tier_b_delta, value_bound=value_bound, two_sided=two_sided,
                         report=report, plan_flags=PLAN_FLAGS if plan_flags is None else plan_flags)


def oracle_cell(case: GpuCase, b: int, kvh: int, tier_b_delta=None):
    """The oracle's view of cell (b, kvh): encoded regions and the decode result
    (with Tier B when tier_b_delta is given)."""
    cfg, inp, layer = case.cfg, case.inp, case.layer
    G = cfg.group
    q = inp["q"][b, kvh * G:(kvh + 1) * G].double().cpu().numpy()
    regions = []
    encs = {}
    if case.prefix_view is not None:
        key = "prefix_k32" if case.fp32_exact else "prefix_k"
        k = inp[key][kvh].double().cpu().numpy()
        v = inp["prefix_v"][kvh].double().cpu().numpy()
        spec = _spec(cfg, cfg.prefix, layer, PREFIX_STREAM, case.value_witness, case.opairs)
        if case.fp32_exact:
            spec.witness = True
            spec.exact_k = True
        enc = encode_region(k, v, spec, kvh)
        regions.append((k, enc, spec))
        encs["prefix"] = enc
    n = int(inp["suffix_lens"][b])
    key = "suffix_k32" if case.fp32_exact else "suffix_k"
    k = inp[key][b, kvh, :n].double().cpu().numpy()
    v = inp["suffix_v"][b, kvh, :n].double().cpu().numpy()
    spec = _spec(cfg, cfg.suffix, layer, b, case.value_witness, case.opairs)
    if case.fp32_exact:
        spec.witness = True
        spec.exact_k = True
    enc = encode_region(k, v, spec, kvh)
    regions.append((k, enc, spec))
    encs["suffix"] = enc
    return encs, decode_cell(q, regions, SM_SCALE, delta_loc=tier_b_delta)


def _bits(t: torch.Tensor) -> np.ndarray:
    t = t.cpu()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16)
    if t.dtype == torch.float16:
        return t.view(torch.int16).numpy().view(np.uint16)
    if t.dtype == torch.float32:
        return t.view(torch.int32).numpy().view(np.uint32)
    return t.numpy()


def check_stored(case: GpuCase, b: int, kvh: int, encs) -> None:
    """Codes, scales and witness bit-exact against the oracle's encoders."""
    n = int(case.inp["suffix_lens"][b])
    pairs = [("suffix", case.suffix_store, (b, kvh), n)]
    if case.prefix_store is not None:
        pairs.append(("prefix", case.prefix_store, (0, kvh), case.cfg.prefix.length))
    for name, st, (bb, hh), nn in pairs:
        enc = encs[name]
        np.testing.assert_array_equal(_bits(st.k[bb, hh, :nn]), np.asarray(enc.k_codes).view(_bits(st.k[bb, hh, :1]).dtype),
                                      err_msg=f"{name} key codes")
        np.testing.assert_array_equal(_bits(st.v[bb, hh, :nn]), np.asarray(enc.v_codes).view(_bits(st.v[bb, hh, :1]).dtype),
                                      err_msg=f"{name} value codes")
        for sc, ref, what in ((st.k_scale, enc.k_scale, "key"), (st.v_scale, enc.v_scale, "value")):
            if ref is None:
                continue
            if ref.dtype == np.float32:
                np.testing.assert_array_equal(_bits(sc[bb, hh, :nn]), ref.view(np.uint32),
                                              err_msg=f"{name} {what} scales")
            else:
                nb = ref.shape[0]
                np.testing.assert_array_equal(_bits(sc[bb, hh, :nb]), ref.view(np.uint16),
                                              err_msg=f"{name} {what} scales")
        if enc.w16 is not None and st.witness is not None:
            np.testing.assert_array_equal(_bits(st.witness[bb, hh, :nn]), enc.w16.view(np.uint16),
                                          err_msg=f"{name} witness")
        assert (enc.k_out is None) == (st.k_outliers is None)
        if enc.k_out is not None:
            ref = f64_to_bf16_bits(enc.k_out).astype(np.uint16)
            np.testing.assert_array_equal(_bits(st.k_outliers[bb, hh, :nn]).view(np.uint16), ref,
                                          err_msg=f"{name} outlier values")
        if enc.v_rec is not None and st.v_witness is not None:
            np.testing.assert_array_equal(_bits(st.v_witness[bb, hh, :nn]), enc.v_rec.view(np.uint16),
                                          err_msg=f"{name} value records")
        assert enc.clipped == 0


TOL_OUT = 2e-3
TOL_METER = 1e-5
# The kernels round c upward (its band factors are raised by 2^-19 so that
# the fp32 roundings of the witness dot cannot take c below its exact value
# for the stored witness, which keeps the bound sound): their log A may then
# exceed the oracle's by up to this fraction of max_t c_t, never fall below.
C_RAISE_REL = 2.0 ** -18


def log_a_within(g: float, r: float, cmax: float) -> bool:
    """log A within 1e-5 of the oracle's, plus the one-sided allowance of the
    upward-rounded c."""
    return r - TOL_METER <= g <= r + TOL_METER + C_RAISE_REL * cmax


def check_results(case: GpuCase, out, meter: Dict[str, torch.Tensor], b: int, kvh: int, ref,
                  check_out: bool = True) -> Dict[str, float]:
    """Attention output within 2e-3 relative; TV, bound and meter within 1e-5."""
    G = case.cfg.group
    worst = dict(out_rel=0.0, tv=0.0, bound=0.0, meter=0.0)
    for h in range(G):
        qh = kvh * G + h
        if check_out:
            og = out[b, qh].double().cpu().numpy()
            orf = ref["out"][h]
            rel = np.linalg.norm(og - orf) / max(np.linalg.norm(orf), 1e-30)
            assert rel <= TOL_OUT, (b, qh, rel)
            assert np.max(np.abs(og - orf)) <= TOL_OUT * np.max(np.abs(orf)) + 1e-30, (b, qh)
            worst["out_rel"] = max(worst["out_rel"], rel)
        if "tv" in meter:
            tv = float(meter["tv"][b, qh])
            assert abs(tv - ref["tv"][h]) <= TOL_METER, (b, qh, tv, ref["tv"][h])
            worst["tv"] = max(worst["tv"], abs(tv - ref["tv"][h]))
        if "bound_raw" in meter:
            # log A within its bar; bound_raw within 1e-5 (relative above 1), or,
            # above 1, through log A (reading 14: "relative 1e-5 on bound_raw,
            # or absolute 1e-5 on log A"); +inf matches +inf, except within
            # 1e-3 of the overflow edge
            cmax = float(np.max(ref["c"][h])) if np.size(ref["c"][h]) else 0.0
            lg, lr = float(meter["log_a"][b, qh]), float(ref["log_a"][h])
            assert log_a_within(lg, lr, cmax), (b, qh, "log_a", lg, lr, cmax)
            worst["log_a"] = max(worst.get("log_a", 0.0), abs(lg - lr))
            bg = float(meter["bound_raw"][b, qh])
            br = float(ref["bound_raw"][h])
            if math.isinf(br) or math.isinf(bg):
                edge = 0.5 * math.log(2 * float(np.finfo(np.float32).max) + 1)
                assert math.isinf(br) == math.isinf(bg) or abs(lr - edge) < 1e-3 + C_RAISE_REL * cmax
            else:
                # (the raise's share: d bound / d log A relative to max(1, bound)
                # is at most 3 below bound 1 and at most 3 above it)
                err = abs(bg - br) / max(1.0, br)
                assert err <= TOL_METER + 3 * C_RAISE_REL * cmax or (br > 1.0 and log_a_within(lg, lr, cmax)), \
                    (b, qh, bg, br)
                worst["bound"] = max(worst["bound"], err)
            mg = float(meter["meter"][b, qh])
            assert abs(mg - float(ref["meter"][h])) <= TOL_METER + 3 * C_RAISE_REL * cmax, (b, qh, mg)
            worst["meter"] = max(worst["meter"], abs(mg - float(ref["meter"][h])))
        if "bound_b_raw" in meter:
            # Tier B: the same bar as Tier A (log A and bound within 1e-5,
            # relative above 1; meter within 1e-5)
            la = float(meter["log_a_b"][b, qh])
            assert abs(la - float(ref["log_a_b"][h])) <= TOL_METER * max(1.0, abs(float(ref["log_a_b"][h]))), \
                (b, qh, la, ref["log_a_b"][h])
            bg, br = float(meter["bound_b_raw"][b, qh]), float(ref["bound_b_raw"][h])
            if math.isinf(br) or math.isinf(bg):
                assert math.isinf(br) == math.isinf(bg)
            else:
                assert abs(bg - br) / max(1.0, br) <= TOL_METER, (b, qh, bg, br)
            assert abs(float(meter["meter_b"][b, qh]) - float(ref["meter_b"][h])) <= TOL_METER
            worst["bound_b"] = max(worst.get("bound_b", 0.0), abs(bg - br) / max(1.0, br))
        if "out_bound" in meter:
            # value side: v_norm_max is a maximum of stored fp16 values (exact);
            # value_err within 1e-5 relative; out_bound within what the meter's
            # 1e-5 and value_err's 1e-5 allow
            vm, vr = float(meter["v_norm_max"][b, qh]), float(ref["v_norm_max"][h])
            assert vm == vr, (b, qh, vm, vr)
            ve, vre = float(meter["value_err"][b, qh]), float(ref["value_err"][h])
            assert abs(ve - vre) <= TOL_METER * max(vre, 1e-30), (b, qh, ve, vre)
            ob, obr = float(meter["out_bound"][b, qh]), float(ref["out_bound"][h])
            assert abs(ob - obr) <= 2 * TOL_METER * vr + TOL_METER * vre + 1e-30, (b, qh, ob, obr)
            worst["value_err"] = max(worst.get("value_err", 0.0), abs(ve - vre) / max(vre, 1e-30))
        if "bound_two_sided" in meter:
            # two-sided form: the Tier A bar (1e-5, relative above 1)
            lm, lmr = float(meter["log_a_minus"][b, qh]), float(ref["log_a_minus"][h])
            assert abs(lm - lmr) <= TOL_METER * max(1.0, abs(lmr)), (b, qh, lm, lmr)
            tg, tr = float(meter["bound_two_sided"][b, qh]), float(ref["bound_two_sided"][h])
            if math.isinf(tr) or math.isinf(tg):
                assert math.isinf(tr) == math.isinf(tg)
            else:
                assert abs(tg - tr) / max(1.0, tr) <= TOL_METER, (b, qh, tg, tr)
            mt, mtr = float(meter["meter_two_sided"][b, qh]), float(ref["meter_two_sided"][h])
            assert abs(mt - mtr) <= TOL_METER, (b, qh, mt, mtr)
            worst["two_sided"] = max(worst.get("two_sided", 0.0), abs(tg - tr) / max(1.0, tr))
            th, thr = float(meter["bound_tanh"][b, qh]), float(ref["bound_tanh"][h])
            assert abs(th - thr) <= TOL_METER, (b, qh, th, thr)
    return worst


def check_block_report(case: GpuCase, meter, b: int, kvh: int, ref, with_b: bool) -> None:
    """The block report of cell (b, kvh) against the oracle's: masses and
    contributions within 1e-5 (relative above 1); the order ranks the GPU's
    own keys and, along it, the oracle's keys do not increase beyond that
    tolerance (near-equal blocks may swap)."""
    from oracle.pipeline import block_report
    cfg = case.cfg
    pre = cfg.prefix.length if cfg.prefix is not None else 0
    caps = ([pre] if pre else []) + [cfg.suffix.length]
    lens = ([pre] if pre else []) + [int(case.inp["suffix_lens"][b])]
    rep = block_report(ref, lens, caps)
    nb = meter["block_mass"].shape[-1]
    assert nb == sum(-(-c // 256) for c in caps)
    for h in range(cfg.group):
        qh = kvh * cfg.group + h
        keys = ["block_mass", "block_excess"] + (["block_excess_b"] if with_b else [])
        for k in keys:
            g = meter[k][b, qh].double().cpu().numpy()
            r = rep[k][h]
            assert np.all(np.abs(g - r) <= 1e-5 * np.maximum(1.0, np.abs(r))), (k, b, qh)
        kk = "block_excess_b" if with_b else "block_excess"
        key = meter[kk][b, qh].double().cpu().numpy()
        order = meter["block_order"][b, qh].cpu().numpy()
        assert sorted(order.tolist()) == list(range(nb))
        assert np.all(np.diff(key[order]) <= 0)
        rkey = rep[kk][h][order]
        assert np.all(np.diff(rkey) <= 2e-5 * np.maximum(1.0, np.abs(rkey[1:])))
