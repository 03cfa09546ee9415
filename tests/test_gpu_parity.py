"""GPU parity of the HIP path against the oracle, through the C ABI.

Bars: stored codes, scales and witness bit-exact; attention output within 2e-3
relative; TV, bound and meter within 1e-5 (relative above 1 for the bound).
"""
import dataclasses
import math
import time

import numpy as np
import pytest
import torch

import cells as cellmod
from quantized_kv_cache_gqa_amd import kvq
from cells import GpuCase, SM_SCALE, check_block_report, check_results, check_stored, oracle_cell, plan
from oracle.numerics import e4m3_table
from workloads import (CONFIGS, INT8_DITHER_B8_S32K, LONG_B4_S128K_SPLIT, QWEN3_B64_S12628_K8V8,
                       QWEN3_SHARED_CARTRIDGE_PAGED, TINY_K16V8_CARTRIDGE, small_variant)

pytestmark = pytest.mark.gpu


def _all_cells(case, cells=None, check_out=True, split_tokens=0, meter_only=False, tier_b_delta=None,
               value_bound=False, two_sided=False):
    cfg = case.cfg
    out, m = case.run(split_tokens=split_tokens, meter_only=meter_only, tier_b_delta=tier_b_delta,
                      value_bound=value_bound, two_sided=two_sided)
    cells = cells or [(b, h) for b in range(cfg.batch) for h in range(cfg.h_kv)]
    worst = {}
    for b, kvh in cells:
        encs, ref = oracle_cell(case, b, kvh, tier_b_delta=tier_b_delta)
        check_stored(case, b, kvh, encs)
        w = check_results(case, out, m, b, kvh, ref, check_out=check_out and not meter_only)
        for k, v in w.items():
            worst[k] = max(worst.get(k, 0.0), v)
    print(f"[{cfg.name}] cells={len(cells)} worst={worst}", flush=True)
    return out, m, worst


def test_fp8_hardware_decode_matches_e4m3_table(gpu_lib):
    """One stored token with scale 1 and p~ = 1: the output is the decoded value
    row itself, so every E4M3 code's hardware decode is compared exactly."""
    kvq = gpu_lib
    dev = "cuda"
    st = kvq.alloc_stored(2, 1, 1, "bf16", "fp8", False, dev)
    codes = torch.arange(256, dtype=torch.int32)
    codes[codes == 0x7F] = 0
    codes[codes == 0xFF] = 0
    st.v.copy_(codes.to(torch.uint8).view(2, 1, 1, 128).to(dev))
    st.v_scale.fill_(1.0)
    view = kvq.RegionView(st, 1)
    q = torch.zeros((2, 1, 128), dtype=torch.float32, device=dev)
    out, _ = kvq.decode_attn(q, 1, None, view, sm_scale=SM_SCALE, meter=False)
    torch.cuda.synchronize()
    ref = e4m3_table()
    ref[[0x7F, 0xFF]] = 0.0
    np.testing.assert_array_equal(out.cpu().numpy().reshape(-1), ref.astype(np.float32))


@pytest.mark.parametrize("scale", [1e-30, 1.0, 1e30])
@pytest.mark.parametrize("paged", [False, True])
def test_bf16_values_keep_their_range(gpu_lib, scale, paged):
    """BF16 values enter the matrix product exactly (no fp16 conversion), so
    values far outside fp16's range, huge or tiny, come out to the output bar
    against the oracle (exact attention: BF16 keys, no witness); 700 ragged
    tokens over several tiles, both the dense and the paged suffix."""
    from oracle.attention import decode_step
    kvq = gpu_lib
    dev = "cuda"
    rng = np.random.default_rng(23)
    B, H, S, G = 2, 2, 704, 4
    lens = [700, 333]
    k = torch.from_numpy(rng.standard_normal((B, H, S, 128)).astype(np.float32)).to(torch.bfloat16)
    v = torch.from_numpy((rng.standard_normal((B, H, S, 128)) * scale).astype(np.float32)).to(torch.bfloat16)
    q = torch.from_numpy(rng.standard_normal((B, H * G, 128)).astype(np.float32))
    st = kvq.alloc_stored(B, H, S, "bf16", "bf16", False, dev)
    st.k.copy_(k.to(dev))
    st.v.copy_(v.to(dev))
    ln = torch.tensor(lens, dtype=torch.int32, device=dev)
    if paged:
        # 16-token pages in shuffled order: page table [B, S / 16]
        ps, mp = 16, S // 16
        table = torch.from_numpy(rng.permutation(B * mp).astype(np.int32)).view(B, mp).to(dev)

        def scatter(t):
            src = t.view(B, H, mp, ps, 128).permute(0, 2, 1, 3, 4).reshape(B * mp, H, ps, 128)
            out = torch.empty_like(src)
            out[table.view(-1).long()] = src
            return out.contiguous()

        pst = kvq.Stored("bf16", "bf16", scatter(st.k), scatter(st.v), None, None, None, None, None, None)
        view = kvq.RegionView(pst, S, lengths=ln, page_table=table, page_size=ps, use_witness=False)
    else:
        view = kvq.RegionView(st, S, lengths=ln, use_witness=False)
    out, _ = kvq.decode_attn(q.to(dev), H, None, view, sm_scale=SM_SCALE, meter=False)
    torch.cuda.synchronize()
    assert bool(torch.isfinite(out).all())
    for b in range(B):
        for h in range(H):
            n = lens[b]
            kk = k[b, h, :n].double().numpy()
            vv = v[b, h, :n].double().numpy()
            ref = decode_step(q[b, h * G:(h + 1) * G].double().numpy(), kk, kk, vv, None, SM_SCALE)
            og = out[b, h * G:(h + 1) * G].double().cpu().numpy()
            for g in range(G):
                rel = np.linalg.norm(og[g] - ref["out"][g]) / np.linalg.norm(ref["out"][g])
                assert rel <= 2e-3, (scale, paged, b, h, g, rel)
                assert np.max(np.abs(og[g] - ref["out"][g])) <= 2e-3 * np.max(np.abs(ref["out"][g]))


def test_write_path_edge_values_bit_exact(gpu_lib):
    """Zero rows, tiny and huge magnitudes, E4M3 midpoints: codes, scales and
    witness against the oracle encoders."""
    from oracle.pipeline import RegionSpec, encode_region
    kvq = gpu_lib
    rng = np.random.default_rng(11)
    T = 300
    x = rng.standard_normal((1, 1, T, 128)).astype(np.float32)
    x[0, 0, 0] = 0.0                                  # all-zero token
    x[0, 0, 1] = -0.0
    x[0, 0, 2] *= 1e-30                               # tiny magnitudes
    x[0, 0, 3] *= 1e30
    x[0, 0, 4, :] = np.float32(2.0 ** -12)            # below half the smallest subnormal step
    mids = (e4m3_table()[1:0x7E] + e4m3_table()[2:0x7F]) / 2
    x[0, 0, 5, :] = 0
    x[0, 0, 5, :len(mids[:127])] = mids[:127] / 448.0 * 448.0
    x[0, 0, 5, 127] = 448.0                           # absmax makes s = 1: y = x exactly
    x[0, 0, 6:40] *= 8                                # outliers
    for kf, vf in (("fp8", "fp8"), ("int8", "int8"), ("bf16", "fp8")):
        xf = x.copy()
        if kf == "int8":
            xf[0, 0, 3] = x[0, 0, 3] * 1e-26          # keep the fp16 block scale finite
        xb = torch.from_numpy(xf).to(torch.bfloat16)  # bf16 exact inputs
        for src in ("bf16", "fp32"):
            kin = (xb if src == "bf16" else torch.from_numpy(xf)).cuda()
            st = kvq.alloc_stored(1, 1, T, kf, vf, True, "cuda")
            kvq.quantize_into(st, kin, kin, seed=12345, layer=3, stream_id=7)
            torch.cuda.synchronize()
            kx = kin[0, 0].double().cpu().numpy()
            spec = RegionSpec(kf, vf, seed=12345, layer=3, stream=7)
            enc = encode_region(kx, kx, spec, 0)
            got_k = st.k[0, 0].cpu()
            if kf == "bf16":
                np.testing.assert_array_equal(got_k.view(torch.int16).numpy().view(np.uint16),
                                              enc.k_codes, err_msg=f"{kf}/{src}")
            else:
                np.testing.assert_array_equal(got_k.numpy(), enc.k_codes, err_msg=f"{kf}/{src}")
            np.testing.assert_array_equal(st.v[0, 0].cpu().numpy(), enc.v_codes, err_msg=f"v {kf}/{src}")
            if kf == "fp8":
                np.testing.assert_array_equal(st.k_scale[0, 0].cpu().numpy().view(np.uint32),
                                              enc.k_scale.view(np.uint32))
            elif kf == "int8":
                np.testing.assert_array_equal(st.k_scale[0, 0].cpu().numpy().view(np.uint16),
                                              enc.k_scale.view(np.uint16))
            np.testing.assert_array_equal(st.witness[0, 0].cpu().numpy().view(np.uint16),
                                          enc.w16.view(np.uint16), err_msg=f"witness {kf}/{src}")
            assert enc.clipped == 0


SMALL = {
    "tiny-cartridge": lambda: TINY_K16V8_CARTRIDGE,
    "shared-cartridge-paged": lambda: small_variant(QWEN3_SHARED_CARTRIDGE_PAGED, batch=3, h_kv=2, lens=(1024, 1000, 17)),
    "fp8-b64": lambda: small_variant(QWEN3_B64_S12628_K8V8, batch=2, h_kv=2, suffix_len=3000, lens=(3000, 1234)),
    "int8-dither": lambda: small_variant(INT8_DITHER_B8_S32K, batch=2, h_kv=2, suffix_len=1000, lens=(1000, 513)),
    "long-split": lambda: small_variant(LONG_B4_S128K_SPLIT, batch=2, h_kv=2, suffix_len=5000, lens=(5000, 4097)),
}


@pytest.fixture(params=["auto", "generic", "noteam"])
def kernel(request, monkeypatch):
    """Run a test with the library's kernel choice, with the vector-ALU kernel,
    and with team launches off (TV spill in the workspace)."""
    if request.param == "generic":
        monkeypatch.setattr(cellmod, "PLAN_FLAGS", kvq.PLAN_VECTOR_ALU)
    elif request.param == "noteam":
        monkeypatch.setattr(cellmod, "PLAN_FLAGS", kvq.PLAN_NO_TEAM)
    return request.param


@pytest.mark.parametrize("name", list(SMALL))
def test_small_config_parity_all_cells(gpu_lib, kernel, name):
    cfg = SMALL[name]()
    case = GpuCase(cfg, layer=5 if cfg.layers > 5 else 0, page_seed=3)
    out, m, worst = _all_cells(case, split_tokens=cfg.split_tokens)
    if cfg.suffix.k_fmt == "bf16" and not cfg.suffix.exact_k:
        # stored keys are the exact keys: TV and bound are exactly zero
        assert torch.all(m["tv"] == 0) and torch.all(m["bound_raw"] == 0)


def test_cfg1_fp32_exact_cache_meter_nonzero(gpu_lib):
    """BF16 storage of fp32 keys as the quantizer: nonzero TV and witness bound."""
    case = GpuCase(TINY_K16V8_CARTRIDGE, fp32_exact=True)
    out, m, worst = _all_cells(case)
    assert float(m["tv"].max()) > 0 and float(m["bound_raw"].min()) > 0
    assert torch.all(m["tv"] <= m["bound_raw"])


@pytest.mark.parametrize("split", [64, 256, 1024])
def test_split_size_does_not_change_results(gpu_lib, kernel, split):
    cfg = small_variant(QWEN3_B64_S12628_K8V8, batch=2, h_kv=1, suffix_len=2500, lens=(2500, 70))
    case = GpuCase(cfg)
    _all_cells(case, split_tokens=split)


def test_group_sizes_and_tiny_lengths(gpu_lib):
    for hq, lens in ((8, (1, 2)), (16, (63, 65)), (64, (129, 1))):
        cfg = dataclasses.replace(small_variant(QWEN3_B64_S12628_K8V8, batch=2, h_kv=8, suffix_len=130, lens=lens),
                                  h_q=hq)
        case = GpuCase(cfg)
        _all_cells(case, cells=[(0, 0), (1, 7), (1, 3)])


def test_prefix_only_request_and_empty_suffix(gpu_lib, kernel):
    cfg = small_variant(QWEN3_SHARED_CARTRIDGE_PAGED, batch=2, h_kv=1, lens=(0, 16))
    case = GpuCase(cfg, page_seed=9)
    _all_cells(case)


def test_meter_only_matches_decode(gpu_lib, kernel):
    cfg = small_variant(LONG_B4_S128K_SPLIT, batch=1, h_kv=2, suffix_len=3000)
    case = GpuCase(cfg)
    _, m1 = case.run(split_tokens=1024)
    _, m2 = case.run(split_tokens=1024, meter_only=True)
    for k in ("tv", "bound_raw", "meter", "log_a"):
        assert torch.equal(m1[k], m2[k]), k
    _all_cells(case, meter_only=True, split_tokens=1024)


@pytest.mark.parametrize("idx", [3, 4])
def test_bitwise_deterministic_across_calls(gpu_lib, idx):
    cfg = small_variant(CONFIGS[idx], batch=2, h_kv=2, suffix_len=700)
    case = GpuCase(cfg)
    o1, m1 = case.run()
    o2, m2 = case.run()
    assert torch.equal(o1, o2)
    for k in m1:
        assert torch.equal(m1[k], m2[k])


def test_bound_dominates_tv_every_cell(gpu_lib):
    """Theorem 1 + 2 on the GPU's own numbers (per cell, never in aggregate)."""
    for idx in (3, 4, 5):
        cfg = small_variant(CONFIGS[idx], batch=2, h_kv=8, suffix_len=777)
        case = GpuCase(cfg)
        _, m = case.run()
        tv, bound = m["tv"], m["bound_raw"]
        assert torch.all(tv >= 0) and torch.all(tv <= 1)
        assert torch.all(tv <= bound + 1e-6), (idx, float((tv - bound).max()))
        assert torch.all(m["meter"] == torch.clamp(bound, max=1.0))


def _team_plan(case, monkeypatch):
    """The plan the library reports with team launches allowed, checked against
    what a team launch must satisfy, and the spill plan it replaces."""
    p = plan(case)
    cfg = case.cfg
    groups = cfg.batch * cfg.h_kv
    assert p["team"] > 0, p
    assert p["chunk"] % 16 == 0 and p["chunk"] * p["team"] >= cfg.suffix.length, p
    assert p["chunk"] <= 2048 and p["team"] <= 64, p
    assert p["n_teams"] * p["rounds"] >= groups > p["n_teams"] * (p["rounds"] - 1), p
    assert p["grid"] % 8 == 0 and p["grid"] >= p["team"] * p["n_teams"], p
    assert plan(case, meter_only=True) == p          # one workspace fits both calls
    monkeypatch.setattr(cellmod, "PLAN_FLAGS", kvq.PLAN_NO_TEAM)
    assert plan(case)["team"] == 0
    monkeypatch.setattr(cellmod, "PLAN_FLAGS", 0)
    # no status word to report a run-out to: the per-chunk plan, which has no waits
    nostat = kvq.plan(case.inp["q"], cfg.h_kv, case.prefix_view, case.suffix_view, sm_scale=SM_SCALE,
                      with_status=False)
    assert nostat["team"] == 0 and nostat["workspace_bytes"] > p["workspace_bytes"], nostat
    return p


def test_team_many_members_and_empty_chunks(gpu_lib, monkeypatch):
    """Four groups, requests of 5000 and 1500 tokens in a 5000-token region:
    tens of members of 64+ tokens each, those past the short request's end
    with empty chunks; parity on every cell and agreement with the
    spill-to-workspace path."""
    cfg = small_variant(LONG_B4_S128K_SPLIT, batch=2, h_kv=2, suffix_len=5000, lens=(5000, 1500))
    case = GpuCase(cfg)
    p = _team_plan(case, monkeypatch)
    assert p["team"] >= 16 and p["chunk"] * (p["team"] - 1) >= 1500, p   # members with no tokens
    out_t, m_t, _ = _all_cells(case)
    monkeypatch.setattr(cellmod, "PLAN_FLAGS", kvq.PLAN_NO_TEAM)
    out_s, m_s = case.run()
    # the two paths round the fp16 P.V weights against different running
    # maxima: compare per head as the oracle bar does (norm-relative)
    rel = (out_t - out_s).double().norm(dim=-1) / out_s.double().norm(dim=-1).clamp_min(1e-30)
    assert float(rel.max()) <= 2e-3, float(rel.max())
    for k in ("tv", "bound_raw", "meter", "log_a"):
        assert torch.allclose(m_t[k], m_s[k], rtol=1e-5, atol=1e-6), k


def test_team_several_rounds_sampled_cells(gpu_lib, monkeypatch):
    """640 groups of ragged 3000-token requests: more groups than resident
    teams, so every team runs several rounds (tags of successive rounds, slot
    parity reuse); sampled cells against the oracle, bitwise repeatable."""
    lens = tuple(3000 - 37 * i for i in range(80))
    cfg = small_variant(QWEN3_B64_S12628_K8V8, batch=80, h_kv=8, suffix_len=3000, lens=lens)
    case = GpuCase(cfg)
    p = _team_plan(case, monkeypatch)
    assert p["rounds"] >= 3, p
    cells = [(0, 0), (1, 7), (33, 4), (64, 2), (79, 7), (79, 0)]
    o1, m1, _ = _all_cells(case, cells=cells)
    o2, m2 = case.run()
    assert torch.equal(o1, o2)
    for k in m1:
        assert torch.equal(m1[k], m2[k]), k


@pytest.mark.parametrize("group", [4, 8])
def test_team_wait_budget_runs_out_to_nan_not_a_hang(gpu_lib, monkeypatch, group):
    """Fault injected from the host: one member of every team never publishes
    and the wait budget is small.  The launch still ends promptly, every
    result of the affected groups is NaN (never a stale or partial value),
    and the next call without the hooks is correct again.  A group of 8 runs
    its paired 4-head teams in one launch."""
    make = lambda: small_variant(QWEN3_B64_S12628_K8V8, batch=2, h_kv=2, suffix_len=3000, lens=(3000, 2500))
    cfg = make() if group == 4 else _g8(make)()
    case = GpuCase(cfg, value_witness=True)
    p = _team_plan(case, monkeypatch)
    assert p["team"] >= 2, p
    assert plan(case, value_bound=True, two_sided=True)["team"] == p["team"]
    # the test build of the library (same kernels) exposes the two hooks
    tlib = kvq.load_test()
    tlib.kvq_test_set_team_hooks(64, 1)
    try:
        t0 = time.time()
        out, m = case.run(lib=tlib, expect_status=kvq.DEVSTATUS_TEAM_WAIT)   # reported, not silent
        assert time.time() - t0 < 30
        assert torch.isnan(out).all()
        for k in ("tv", "bound_raw", "meter", "log_a"):
            assert torch.isnan(m[k]).all(), k
        out, m = case.run(value_bound=True, two_sided=True, lib=tlib,       # the team kernel with
                          expect_status=kvq.DEVSTATUS_TEAM_WAIT)            # the extensions
        assert torch.isnan(out).all()
        for k in ("tv", "meter", "value_err", "out_bound", "v_norm_max", "log_a_minus", "meter_two_sided",
                  "bound_tanh"):
            assert torch.isnan(m[k]).all(), k
    finally:
        tlib.kvq_test_set_team_hooks(0, -1)
    o_t, m_t = case.run(lib=tlib)                   # hooks off: status clear, results as the product's
    _all_cells(case)
    o_p, m_p = case.run()
    assert torch.equal(o_t, o_p) and all(torch.equal(m_t[k], m_p[k]) for k in m_p)
    _all_cells(case, value_bound=True, two_sided=True)


@pytest.mark.parametrize("group", [4, 8])
def test_graph_capture_of_a_team_launch(gpu_lib, monkeypatch, group):
    """A call captured into a graph keeps the team plan: the launch takes its
    tags from the epoch in the workspace, which every launch advances on the
    device.  Every replay equals the eager team result bit for bit, with
    eager team calls on the same workspace between the replays; a
    per-chunk call on that workspace between them changes nothing either.
    A group of 8 captures its one launch of paired 4-head teams."""
    from quantized_kv_cache_gqa_amd import kvq
    make = lambda: small_variant(QWEN3_B64_S12628_K8V8, batch=2, h_kv=2, suffix_len=3000, lens=(3000, 2500))
    cfg = make() if group == 4 else _g8(make)()
    case = GpuCase(cfg)
    p = _team_plan(case, monkeypatch)
    if group == 8:
        assert p["launches"] == 1 and p["grid"] >= 2 * p["team"] * p["n_teams"], p
    ws = kvq.Workspace(torch.device("cuda"))

    def call(out=None, meter_bufs=None, plan_flags=0):
        return kvq.decode_attn(case.inp["q"], cfg.h_kv, case.prefix_view, case.suffix_view,
                               sm_scale=SM_SCALE, workspace=ws, out=out, meter_bufs=meter_bufs,
                               plan_flags=plan_flags)

    o_team, m_team = call()
    monkeypatch.setattr(cellmod, "PLAN_FLAGS", kvq.PLAN_NO_TEAM)
    o_chunk, m_chunk = case.run()
    monkeypatch.setattr(cellmod, "PLAN_FLAGS", 0)
    torch.cuda.synchronize()
    og = torch.empty_like(o_chunk)
    mg = {k: torch.empty_like(v) for k, v in m_chunk.items()}
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        call(out=og, meter_bufs=mg)
    for it in range(4):
        og.fill_(float("nan"))
        for v in mg.values():
            v.fill_(float("nan"))
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(og, o_team)
        for k in m_team:
            assert torch.equal(mg[k], m_team[k]), k
        g.replay()                                  # twice in a row: fresh tags again
        torch.cuda.synchronize()
        assert torch.equal(og, o_team)
        o2, m2 = call()
        torch.cuda.synchronize()
        assert torch.equal(o2, o_team)
        for k in m_team:
            assert torch.equal(m2[k], m_team[k]), k
        if it == 1:                                 # the per-chunk plan on the same workspace
            o3, m3 = call(plan_flags=kvq.PLAN_NO_TEAM)
            torch.cuda.synchronize()
            assert torch.equal(o3, o_chunk)
            for k in m_chunk:
                assert torch.equal(m3[k], m_chunk[k]), k
    assert ws.read_status() == 0


def _two_region_fp8(paged):
    """A shared FP8 cartridge (exact keys, witness) before an FP8 suffix, both
    with the TV and the meter: the one-launch form with the full meter."""
    from workloads.configs import RegionCfg
    base = small_variant(LONG_B4_S128K_SPLIT, batch=2, h_kv=2, suffix_len=1504, lens=(1504, 700))
    suf = dataclasses.replace(base.suffix, paged=paged, page_size=16)
    pre = RegionCfg(length=700, k_fmt="fp8", v_fmt="fp8", exact_k=True, witness=True)
    return dataclasses.replace(base, prefix=pre, suffix=suf, name=base.name + "-cartridge")


TWO_REGION = {
    "tiny-cartridge": lambda: TINY_K16V8_CARTRIDGE,
    "shared-cartridge-paged": SMALL["shared-cartridge-paged"],
    "fp8": lambda: _two_region_fp8(False),
    "fp8-paged": lambda: _two_region_fp8(True),
}


@pytest.mark.parametrize("name", list(TWO_REGION))
def test_two_regions_in_one_launch(gpu_lib, monkeypatch, name):
    """Cartridge + suffix in one launch (every chunk of either region may be the
    last to arrive and merge): every cell against the oracle, and bitwise the
    results of one launch per region, for the decode and the meter-only call."""
    cfg = TWO_REGION[name]()
    case = GpuCase(cfg, page_seed=5)
    split = 128
    # decode launches only (the finish launch has its own test)
    monkeypatch.setattr(cellmod, "PLAN_FLAGS", kvq.PLAN_NO_TEAM | kvq.PLAN_FINALIZE_IN_PLACE)
    p = plan(case, split_tokens=split)
    assert (p["team"], p["launches"]) == (0, 1), p
    assert plan(case, split_tokens=split, meter_only=True)["launches"] == 1
    o1, m1, _ = _all_cells(case, split_tokens=split)
    _, q1 = case.run(split_tokens=split, meter_only=True)
    monkeypatch.setattr(cellmod, "PLAN_FLAGS",
                        kvq.PLAN_NO_TEAM | kvq.PLAN_FINALIZE_IN_PLACE | kvq.PLAN_LAUNCH_PER_REGION)
    assert plan(case, split_tokens=split)["launches"] == 2
    o2, m2 = case.run(split_tokens=split)
    _, q2 = case.run(split_tokens=split, meter_only=True)
    assert torch.equal(o1, o2)
    for k in m1:
        assert torch.equal(m1[k], m2[k]), k
        assert torch.equal(q1[k], q2[k]), k


PAGED_LONG = {
    "fp8": lambda ps: small_variant(QWEN3_B64_S12628_K8V8, batch=2, h_kv=2, suffix_len=9216, lens=(9216, 8200),
                                    suffix_paged=True, suffix_page_size=ps),
    "cartridge-bf16": lambda ps: small_variant(QWEN3_SHARED_CARTRIDGE_PAGED, batch=2, h_kv=2, suffix_len=9216,
                                               lens=(9216, 5000), suffix_page_size=ps),
}


@pytest.mark.parametrize("page_size", [8, 16])
@pytest.mark.parametrize("name", list(PAGED_LONG))
def test_paged_chunks_longer_than_the_page_window(gpu_lib, name, page_size):
    """Paged suffixes in 8,192-token chunks: each wavefront walks 128 tiles,
    so the page ids of its tiles are fetched in three windows of 64 (the last
    past the chunk's end), with 8- and 16-token pages, a full and a ragged
    request, every cell against the oracle."""
    cfg = PAGED_LONG[name](page_size)
    case = GpuCase(cfg, page_seed=11)
    p = plan(case, split_tokens=8192)
    assert p["team"] == 0 and p["chunk"] == 8192, p
    _all_cells(case, split_tokens=8192)


def _tier_b_two_region():
    """A BF16 shared prefix (radius 0) before a dithered INT8 suffix: two
    launches, one per key format, both accumulating E_p~[e^u]."""
    from workloads.configs import RegionCfg
    base = small_variant(INT8_DITHER_B8_S32K, batch=2, h_kv=2, suffix_len=700, lens=(700, 300))
    pre = RegionCfg(length=300, k_fmt="bf16", v_fmt="bf16", exact_k=False, witness=False)
    return dataclasses.replace(base, prefix=pre, name=base.name + "-bf16-cartridge")


TIER_B = {
    "int8-dither": SMALL["int8-dither"],
    "int8-dither-long": lambda: small_variant(INT8_DITHER_B8_S32K, batch=1, h_kv=2, suffix_len=3000, lens=(2900,)),
    "shared-cartridge-paged-bf16": SMALL["shared-cartridge-paged"],
    "bf16-int8": _tier_b_two_region,
}


@pytest.mark.parametrize("name", list(TIER_B))
@pytest.mark.parametrize("delta", [1e-3, 1e-9])
def test_tier_b_certificate_every_cell(gpu_lib, kernel, name, delta):
    """Tier B (WitCert Sec. 4.2) on every cell against the oracle: log A_B,
    bound and meter within 1e-5; Tier A, TV and the output unchanged; the team
    launch is never planned with Tier B; TV <= bound_B on these (non-adaptive)
    queries."""
    cfg = TIER_B[name]()
    case = GpuCase(cfg, page_seed=2)
    assert plan(case, tier_b_delta=delta)["team"] == 0
    split = 256 if name == "int8-dither-long" else 0
    out, m, worst = _all_cells(case, split_tokens=split, tier_b_delta=delta)
    assert "bound_b" in worst
    if cfg.suffix.k_fmt == "bf16" and (cfg.prefix is None or cfg.prefix.k_fmt == "bf16"):
        assert torch.all(m["log_a_b"] == 0) and torch.all(m["bound_b_raw"] == 0)
    else:
        assert torch.all(m["log_a_b"] > 0)
    assert torch.all(m["tv"] <= m["bound_b_raw"])
    out2, m2 = case.run(split_tokens=split)
    assert torch.equal(out, out2)
    for k in m2:
        assert torch.equal(m[k], m2[k]), k


VALUE = {
    "shared-cartridge-paged": SMALL["shared-cartridge-paged"],
    "fp8-b64": SMALL["fp8-b64"],
    "int8-dither": SMALL["int8-dither"],
    "long-split": SMALL["long-split"],
    "fp8-paged-cartridge": lambda: _two_region_fp8(True),
}


@pytest.mark.parametrize("name", list(VALUE))
def test_value_side_and_joint_output_bound_every_cell(gpu_lib, kernel, monkeypatch, name):
    """Value records written bit-exactly; value_err, v_norm_max and the joint
    output bound 2 meter max||v|| + sum p~ rho on every cell against the
    oracle; the same plan as without the value side (a team where one
    applies), whose other results are bitwise those without it."""
    cfg = VALUE[name]()
    case = GpuCase(cfg, page_seed=4, value_witness=True)
    pv = plan(case, value_bound=True)
    assert pv["team"] == plan(case)["team"]
    if kernel == "auto" and name in ("fp8-b64", "long-split"):
        assert pv["team"] > 0
    out, m, worst = _all_cells(case, value_bound=True)
    assert "value_err" in worst
    assert torch.all(m["out_bound"] >= m["value_err"])
    if cfg.suffix.v_fmt != "bf16":
        assert torch.all(m["value_err"] > 0)
    o2, m2 = case.run()
    assert torch.equal(out, o2)
    for k in m2:
        assert torch.equal(m[k], m2[k]), k
    _, mo = case.run(meter_only=True, value_bound=True)
    for k in ("value_err", "v_norm_max", "out_bound"):
        assert torch.equal(mo[k], m[k]), k


TWO_SIDED = {
    "shared-cartridge-paged": SMALL["shared-cartridge-paged"],
    "fp8-b64": SMALL["fp8-b64"],
    "int8-dither": SMALL["int8-dither"],
    "long-split": SMALL["long-split"],
    "fp8-cartridge": lambda: _two_region_fp8(False),
}


@pytest.mark.parametrize("name", list(TWO_SIDED))
def test_two_sided_form_every_cell(gpu_lib, kernel, monkeypatch, name):
    """Proposition 1's A- and the two-sided meter on every cell against the
    oracle; TV <= bound_two_sided and meter_two_sided <= meter; the same plan
    as without it (a team where one applies), whose other results are
    bitwise those without it."""
    cfg = TWO_SIDED[name]()
    case = GpuCase(cfg, page_seed=6)
    pt = plan(case, two_sided=True)
    assert pt["team"] == plan(case)["team"]
    if kernel == "auto" and name in ("fp8-b64", "long-split"):
        assert pt["team"] > 0
    out, m, worst = _all_cells(case, two_sided=True)
    assert "two_sided" in worst
    assert torch.all(m["tv"] <= m["bound_two_sided"])
    assert torch.all(m["meter_two_sided"] <= m["meter"])
    assert torch.all(m["log_a_minus"] <= 0) and torch.all(m["log_a"] >= 0)
    assert torch.all(m["tv"] <= m["bound_tanh"] + 1e-6) and torch.all(m["bound_tanh"] <= 1)
    o2, m2 = case.run()
    assert torch.equal(out, o2)
    for k in m2:
        assert torch.equal(m[k], m2[k]), k


REPORT = {
    "shared-cartridge-paged": (SMALL["shared-cartridge-paged"], True),
    "int8-dither": (SMALL["int8-dither"], True),
    "long-split": (SMALL["long-split"], False),
    "bf16-int8": (_tier_b_two_region, True),
}


@pytest.mark.parametrize("name", list(REPORT))
@pytest.mark.parametrize("with_b", [False, True])
def test_block_report_every_cell(gpu_lib, kernel, monkeypatch, name, with_b):
    """The block-decomposable report on every cell against the oracle: block
    masses and contributions within 1e-5 (relative above 1), Tier B's when
    requested; the page-in order ranks the GPU's own keys and agrees with the
    oracle's values; the other results bitwise those of the per-chunk plan
    without the report."""
    make, b_ok = REPORT[name]
    if with_b and not b_ok:
        pytest.skip("Tier B needs INT8 or BF16 keys")
    cfg = make()
    case = GpuCase(cfg, page_seed=8)
    delta = 1e-6 if with_b else None
    assert plan(case, report=True, tier_b_delta=delta)["team"] == 0
    out, m = case.run(report=True, tier_b_delta=delta)
    for b in range(cfg.batch):
        for kvh in range(cfg.h_kv):
            _, ref = oracle_cell(case, b, kvh, tier_b_delta=delta)
            check_block_report(case, m, b, kvh, ref, with_b)
            for h in range(cfg.group):
                qh = kvh * cfg.group + h
                a_1 = math.expm1(float(ref["log_a"][h]))
                assert abs(float(m["block_excess"][b, qh].double().sum()) - a_1) <= 1e-4 * max(1.0, a_1)
    monkeypatch.setattr(cellmod, "PLAN_FLAGS", cellmod.PLAN_FLAGS | kvq.PLAN_NO_TEAM)
    o2, m2 = case.run(tier_b_delta=delta)
    assert torch.equal(out, o2)
    for k in m2:
        assert torch.equal(m[k], m2[k]), k


def _g32(paged=False, cartridge=False):
    """Dithered INT8 with per-(token, 32-channel group) scales (WitCert Sec.
    6.2.3, Table 4), dense or in shuffled 16-token pages, with an INT8-G32
    shared prefix when asked."""
    from workloads.configs import RegionCfg
    base = small_variant(INT8_DITHER_B8_S32K, batch=2, h_kv=2, suffix_len=1024, lens=(1024, 513))
    suf = dataclasses.replace(base.suffix, k_fmt="int8g32", v_fmt="int8g32", paged=paged, page_size=16)
    pre = RegionCfg(length=300, k_fmt="int8g32", v_fmt="int8g32", exact_k=True, witness=True) \
        if cartridge else None
    tag = "-g32" + ("-paged" if paged else "") + ("-cartridge" if cartridge else "")
    return dataclasses.replace(base, prefix=pre, suffix=suf, name=base.name + tag)


G32 = {
    "dense": lambda: _g32(),
    "paged": lambda: _g32(paged=True),
    "paged-cartridge": lambda: _g32(paged=True, cartridge=True),
}


@pytest.mark.parametrize("name", list(G32))
def test_int8_group_scales_every_cell(gpu_lib, kernel, monkeypatch, name):
    """Codes, per-(token, group) scales, witness and value records bit-exact;
    output, Tier A, Tier B (radius from the token's group scales), the value
    side and the two-sided form on every cell against the oracle; then the
    plain call (no extensions) over smaller chunks and the block report."""
    cfg = G32[name]()
    case = GpuCase(cfg, page_seed=9, value_witness=True)
    out, m, worst = _all_cells(case, tier_b_delta=1e-3, value_bound=True, two_sided=True)
    assert {"bound_b", "value_err", "two_sided"} <= set(worst)
    assert torch.all(m["log_a_b"] > 0) and torch.all(m["tv"] <= m["bound_b_raw"])
    assert torch.all(m["tv"] <= m["bound_raw"])
    _all_cells(case, split_tokens=128)                  # the kernels without the extensions
    _, mb = case.run(report=True)
    for b in range(cfg.batch):
        for kvh in range(cfg.h_kv):
            _, ref = oracle_cell(case, b, kvh)
            check_block_report(case, mb, b, kvh, ref, False)



OUTLIERS = {
    "dense-m4": (lambda: _g32(), 4),
    "paged-m8": (lambda: _g32(paged=True), 8),
    "paged-cartridge-m2": (lambda: _g32(paged=True, cartridge=True), 2),
    "dense-m16": (lambda: _g32(), 16),
}


@pytest.mark.parametrize("name", list(OUTLIERS))
def test_outlier_pairs_every_cell(gpu_lib, kernel, name):
    """Fixed outlier RoPE pairs beside group-scale INT8 keys (WitCert Sec.
    6.2.5): codes, scales (the pairs left out of the group maximum) and the
    stored exact values bit-exact; output, Tier A, Tier B (no dither on the
    bypassed channels) and the value side on every cell against the oracle,
    KV head 1 with a repeated and an out-of-range slot; the bypass lowers
    Tier B's log A_B on these keys with heavy RoPE pairs."""
    make, m = OUTLIERS[name]
    cfg = make()
    case = GpuCase(cfg, page_seed=10, value_witness=True, n_outlier_pairs=m)
    out, mo, worst = _all_cells(case, tier_b_delta=1e-3, value_bound=True)
    assert {"bound_b", "value_err"} <= set(worst)
    assert torch.all(mo["tv"] <= mo["bound_b_raw"]) and torch.all(mo["tv"] <= mo["bound_raw"])
    _all_cells(case, split_tokens=128)                  # the kernels without the extensions
    plain = GpuCase(cfg, page_seed=10)
    _, mp = plain.run(tier_b_delta=1e-3)
    assert float(mo["log_a_b"].median()) < float(mp["log_a_b"].median())


FINISH = {
    "int8-dither": (lambda: small_variant(INT8_DITHER_B8_S32K, batch=2, h_kv=2, suffix_len=3000, lens=(3000, 1000)),
                    1e-6),
    "long-split": (lambda: small_variant(LONG_B4_S128K_SPLIT, batch=2, h_kv=2, suffix_len=9000, lens=(9000, 4097)),
                   None),
    "fp8-cartridge": (lambda: _two_region_fp8(False), None),
}


@pytest.mark.parametrize("name", list(FINISH))
def test_finish_launch_matches_the_oracle_and_the_in_kernel_finalize(gpu_lib, monkeypatch, name):
    """Several chunks per group: the TV and the block report run in the finish
    launch.  Both that and the decode launch's own finalize (KVQ_PLAN_FINALIZE_IN_PLACE)
    match the oracle on every cell; the page-in order is the same, the TV
    differs by summation order only."""
    monkeypatch.setattr(cellmod, "PLAN_FLAGS", kvq.PLAN_NO_TEAM)
    make, delta = FINISH[name]
    cfg = make()
    case = GpuCase(cfg, page_seed=12)
    res = {}
    for mode in ("finish", "kept"):
        if mode == "kept":
            monkeypatch.setattr(cellmod, "PLAN_FLAGS", kvq.PLAN_NO_TEAM | kvq.PLAN_FINALIZE_IN_PLACE)
        p = plan(case, split_tokens=512, report=True, tier_b_delta=delta)
        assert p["chunks"] > 1 and (p["launches"] >= 2) == (mode == "finish"), p
        out, m = case.run(split_tokens=512, report=True, tier_b_delta=delta)
        for b in range(cfg.batch):
            for kvh in range(cfg.h_kv):
                encs, ref = oracle_cell(case, b, kvh, tier_b_delta=delta)
                check_results(case, out, m, b, kvh, ref)
                check_block_report(case, m, b, kvh, ref, delta is not None)
        res[mode] = (out, m)
    (o1, m1), (o2, m2) = res["finish"], res["kept"]
    assert torch.equal(o1, o2)
    assert torch.equal(m1["block_order"], m2["block_order"])
    assert torch.equal(m1["block_mass"], m2["block_mass"])
    torch.testing.assert_close(m1["tv"], m2["tv"], rtol=0, atol=1e-6)


def _g8(make):
    """The same cells with 8 query heads per KV head (h_q = 8 h_kv)."""
    def f():
        cfg = make()
        return dataclasses.replace(cfg, h_q=8 * cfg.h_kv, name=cfg.name + "-g8")
    return f


GROUP8 = {
    "fp8": _g8(lambda: small_variant(QWEN3_B64_S12628_K8V8, batch=2, h_kv=2, suffix_len=3000, lens=(3000, 1234))),
    "int8-dither": _g8(lambda: small_variant(INT8_DITHER_B8_S32K, batch=2, h_kv=2, suffix_len=1000, lens=(1000, 513))),
    "int8g32-paged-m4": _g8(lambda: _g32(paged=True)),
    "fp8-cartridge": _g8(lambda: _two_region_fp8(False)),
}


@pytest.mark.parametrize("name", list(GROUP8))
def test_group_of_eight_every_cell(gpu_lib, kernel, name):
    """GQA groups of 8: on the matrix cores as one team launch of paired
    4-head teams, or as two per-chunk launch sets of 4 query heads, or on the
    vector-ALU kernel; every cell against the oracle with Tier A, the value
    side, the two-sided form and, for INT8 keys, Tier B; the block report
    where the plan takes it."""
    cfg = GROUP8[name]()
    m = 4 if name.endswith("m4") else 0
    case = GpuCase(cfg, page_seed=13, value_witness=True, n_outlier_pairs=m)
    delta = 1e-4 if "int8" in name else None
    p = plan(case, tier_b_delta=delta, value_bound=True, two_sided=True)
    if p["team"]:
        assert p["launches"] == 1 and p["grid"] >= 2 * p["team"] * p["n_teams"], p
    elif kernel != "generic":
        assert p["launches"] % 2 == 0, p                 # two sets of launches
    _all_cells(case, tier_b_delta=delta, value_bound=True, two_sided=True)
    _all_cells(case, split_tokens=256)
    if "g32" not in name:
        _, mr = case.run(report=True)
        for b in range(cfg.batch):
            for kvh in range(cfg.h_kv):
                _, ref = oracle_cell(case, b, kvh)
                check_block_report(case, mr, b, kvh, ref, False)


def test_group_of_eight_team_pairs_against_two_launches(gpu_lib, monkeypatch):
    """A group of 8 on the team plan: one launch whose raw teams 2t and 2t + 1
    take query heads 0-3 and 4-7, on a shape with several rounds, ragged
    requests, the value side and the two-sided form; sampled cells against the
    oracle, bitwise repeatable, and within rounding of two launches of 4 heads
    (KVQ_PLAN_GROUP8_SEPARATE, whose plan has its own team size and chunk)."""
    lens = tuple(3000 - 61 * i for i in range(40))
    cfg = _g8(lambda: small_variant(QWEN3_B64_S12628_K8V8, batch=40, h_kv=8, suffix_len=3000, lens=lens))()
    case = GpuCase(cfg, value_witness=True)
    kw = dict(value_bound=True, two_sided=True)
    p = _team_plan(case, monkeypatch)
    assert p["rounds"] >= 3, p
    pe = plan(case, **kw)
    assert pe["team"] and pe["launches"] == 1, pe
    assert pe["grid"] >= 2 * pe["team"] * pe["n_teams"] and pe["grid"] % 8 == 0, pe
    o1, m1, _ = _all_cells(case, cells=[(0, 0), (13, 7), (39, 3), (39, 0)], **kw)
    o1b, m1b = case.run(**kw)
    assert torch.equal(o1, o1b)
    monkeypatch.setattr(cellmod, "PLAN_FLAGS", kvq.PLAN_GROUP8_SEPARATE)
    q = plan(case, **kw)
    assert q["team"] and q["launches"] == 2, q
    o2, m2 = case.run(**kw)
    # the same bars as against the oracle: rows within 2e-3 of their norm,
    # meter fields within 1e-5
    rel = (o1 - o2).norm(dim=-1) / o2.norm(dim=-1).clamp_min(1e-30)
    assert rel.max().item() <= 2e-3, rel.max().item()
    for k in m1:
        if m1[k] is not None:
            assert torch.equal(m1[k], m1b[k]), k
            torch.testing.assert_close(m1[k], m2[k], rtol=1e-5, atol=1e-5, msg=k)


def test_team_epoch_restarts_below_its_limit(gpu_lib, monkeypatch):
    """The team epoch kept in the workspace's first word moves past each
    launch's tags and restarts from 0 before the tags could leave the
    signalling-NaN range; the launch that restarts it clears the team region,
    so words planted there with the tags the next launch waits for (the
    control word and the region are caller memory, set here from the host)
    are gone, and results stay exact across the restart."""
    from quantized_kv_cache_gqa_amd import kvq
    cfg = small_variant(QWEN3_B64_S12628_K8V8, batch=2, h_kv=2, suffix_len=3000, lens=(3000, 2500))
    case = GpuCase(cfg)
    p = _team_plan(case, monkeypatch)
    ws = kvq.Workspace(torch.device("cuda"))
    team_off = 256 + (1 << 20)                     # after the control words and the counters
    epoch_max = (1 << 22) - (1 << 18) - 1

    def call():
        return kvq.decode_attn(case.inp["q"], cfg.h_kv, case.prefix_view, case.suffix_view,
                               sm_scale=SM_SCALE, workspace=ws)

    o_ref, m_ref = call()
    torch.cuda.synchronize()
    ctl = ws.buf[:8].view(torch.int32)
    assert int(ctl[0]) == p["rounds"] + 1 and int(ctl[1]) == 0
    region = ws.buf[team_off:p["workspace_bytes"]].view(torch.int64)
    # every team word: tag of the first round after a restart, value 1e30
    region.fill_((0x7F800001 << 32) | 0x7149F2CA)
    ctl[0] = epoch_max - p["rounds"]                # this launch restarts the epoch at its end
    torch.cuda.synchronize()
    o, m = call()
    torch.cuda.synchronize()
    assert int(ctl[0]) == 0 and int(ctl[1]) == 0
    assert int(region.count_nonzero()) == 0         # the restart cleared the region
    for expect in (p["rounds"] + 1, 2 * (p["rounds"] + 1)):
        assert torch.equal(o, o_ref)
        for k in m_ref:
            assert torch.equal(m[k], m_ref[k]), k
        o, m = call()
        torch.cuda.synchronize()
        assert int(ctl[0]) == expect and int(ctl[1]) == 0
    assert ws.read_status() == 0


def _gq(make, g):
    def f():
        cfg = make()
        return dataclasses.replace(cfg, h_q=g * cfg.h_kv, name=cfg.name + f"-g{g}")
    return f


SMALL_GROUPS = {f"{name}-g{g}": (_gq(make, g), g) for g in (1, 2) for name, make in (
    ("fp8", lambda: small_variant(QWEN3_B64_S12628_K8V8, batch=2, h_kv=2, suffix_len=3000, lens=(3000, 1234))),
    ("int8-dither", lambda: small_variant(INT8_DITHER_B8_S32K, batch=2, h_kv=2, suffix_len=1000, lens=(1000, 513))),
    ("int8g32-paged-m4", lambda: _g32(paged=True)),
    ("fp8-cartridge", lambda: _two_region_fp8(False)),
)}


@pytest.mark.parametrize("name", list(SMALL_GROUPS))
def test_groups_of_one_and_two_every_cell(gpu_lib, kernel, name):
    """1 or 2 query heads per KV head: on the matrix cores as a 4-head tile
    padded with copies of the last head (library choice; the padding heads'
    results are never written), or on the vector-ALU kernel; every cell
    against the oracle with Tier A, the value side, the two-sided form and,
    for INT8 keys, Tier B; the block report where the plan takes it."""
    make, g = SMALL_GROUPS[name]
    cfg = make()
    m = 4 if "m4" in name else 0
    case = GpuCase(cfg, page_seed=14, value_witness=True, n_outlier_pairs=m)
    delta = 1e-4 if "int8" in name else None
    out, mm, _ = _all_cells(case, tier_b_delta=delta, value_bound=True, two_sided=True)
    assert out.shape[1] == cfg.h_q and mm["tv"].shape[1] == cfg.h_q
    _all_cells(case, split_tokens=256)
    if "g32" not in name:
        _, mr = case.run(report=True)
        for b in range(cfg.batch):
            for kvh in range(cfg.h_kv):
                _, ref = oracle_cell(case, b, kvh)
                check_block_report(case, mr, b, kvh, ref, False)


def test_group_scale_append_matches_a_whole_write(gpu_lib):
    """The per-token group-scale format is written token by token (paging-safe,
    WitCert Sec. 6.2.3): appending the newest tokens one call at a time, at
    any position, stores the same codes, scales, witness, value records and
    outlier values as one call over the whole range; and the meter-only call
    gives the decode call's meter bitwise."""
    from quantized_kv_cache_gqa_amd import kvq
    cfg = _g32()
    case = GpuCase(cfg, page_seed=15, value_witness=True, n_outlier_pairs=4)
    st = case.suffix_store
    kin, vin = case.inp["suffix_k"], case.inp["suffix_v"]
    op = torch.from_numpy(case.opairs).to("cuda")
    inc = kvq.alloc_stored(cfg.batch, cfg.h_kv, cfg.suffix.length, "int8g32", "int8g32", True, "cuda",
                           value_witness=True, outlier_pairs=op)
    from cells import dither_seed
    cuts = [0, 1, 17, 300, 301, cfg.suffix.length - 1, cfg.suffix.length]
    for t0, t1 in zip(cuts[:-1], cuts[1:]):
        kvq.quantize_into(inc, kin, vin, tok_begin=t0, tok_end=t1, seed=dither_seed(cfg), layer=0, stream_id=0)
    torch.cuda.synchronize()
    for name in ("k", "v", "k_scale", "v_scale", "witness", "v_witness", "k_outliers"):
        assert torch.equal(getattr(inc, name), getattr(st, name)), name
    out, m = case.run()
    _, mo = case.run(meter_only=True)
    for k in mo:
        assert torch.equal(mo[k], m[k]), k
