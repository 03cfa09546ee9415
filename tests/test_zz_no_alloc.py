"""kvq_decode_attn_noalloc (the decode call on the library's static per-device
scratch, for callers that cannot allocate) against kvq_decode_attn with a
caller workspace, through the C ABI: two calls in a row on the same scratch,
the second with a smaller input, each bitwise equal to the workspace call's
results and within the oracle's bars on sampled cells; a shape whose plan
needs more than the scratch holds is rejected before any launch."""
import ctypes

import pytest
import torch

from cells import SM_SCALE, GpuCase, check_results, oracle_cell
from workloads import LONG_B4_S128K_SPLIT, QWEN3_B64_S12628_K8V8, small_variant

pytestmark = pytest.mark.gpu

KEYS = ("tv", "bound_raw", "meter", "log_a")


def _both(case, plan_flags=0):
    """The same decode through kvq_decode_attn (fresh workspace) and through
    kvq_decode_attn_noalloc; returns both results and the plan."""
    from quantized_kv_cache_gqa_amd import kvq
    cfg = case.cfg
    out_w, m_w = case.run(plan_flags=plan_flags)
    out_s = torch.full_like(out_w, float("nan"))
    m_s = {k: torch.full_like(m_w[k], float("nan")) for k in KEYS}
    status = torch.zeros(4, dtype=torch.int32, device=out_w.device)
    kvq.decode_attn_noalloc(case.inp["q"], cfg.h_kv, case.prefix_view, case.suffix_view, sm_scale=SM_SCALE,
                            out=out_s, meter_bufs=m_s, status=status, plan_flags=plan_flags)
    torch.cuda.synchronize()
    assert int(status[0]) == 0
    p = kvq.plan(case.inp["q"], cfg.h_kv, case.prefix_view, case.suffix_view, sm_scale=SM_SCALE,
                 plan_flags=plan_flags)
    return out_w, m_w, out_s, m_s, p


def _check(case, out_w, m_w, out_s, m_s, cells):
    assert torch.equal(out_s, out_w)
    for k in KEYS:
        assert torch.equal(m_s[k], m_w[k]), k
    for b, kvh in cells:
        _, ref = oracle_cell(case, b, kvh)
        check_results(case, out_s, m_s, b, kvh, ref)


def test_noalloc_two_calls_second_smaller_match_the_workspace_call(gpu_lib):
    from quantized_kv_cache_gqa_amd import kvq
    # 1: 160 groups of a K8/V8 step with the TV: the team plan (several rounds)
    lens = tuple(2600 - 53 * i for i in range(20))
    big = GpuCase(small_variant(QWEN3_B64_S12628_K8V8, batch=20, h_kv=8, suffix_len=2600, lens=lens), layer=3)
    out_w, m_w, out_s, m_s, p = _both(big)
    assert p["team"] > 0 and p["workspace_bytes"] <= kvq.SCRATCH_BYTES, p
    _check(big, out_w, m_w, out_s, m_s, [(0, 0), (7, 5), (19, 7)])
    print(f"[noalloc] call 1: plan team {p['team']} x {p['n_teams']} teams, {p['rounds']} rounds", flush=True)
    # 2: a smaller input on the same scratch, the per-chunk plan with several
    #    chunks per group (TV spill, finish launch) and then its team plan
    small = GpuCase(small_variant(LONG_B4_S128K_SPLIT, batch=2, h_kv=2, suffix_len=3000, lens=(3000, 1100)))
    for flags in (kvq.PLAN_NO_TEAM, 0):
        out_w, m_w, out_s, m_s, p = _both(small, plan_flags=flags)
        assert p["workspace_bytes"] <= kvq.SCRATCH_BYTES, p
        _check(small, out_w, m_w, out_s, m_s, [(b, h) for b in range(2) for h in range(2)])
        print(f"[noalloc] call 2 (flags {flags}): plan {p}", flush=True)


def test_noalloc_rejects_a_plan_beyond_the_scratch(gpu_lib):
    """The batch-64 x 12,628-token step on the per-chunk plan spills 207 MB of
    TV pairs: more than the scratch, so the call returns KVQ_ERR_WORKSPACE
    before anything is enqueued (its pointers are never touched)."""
    from quantized_kv_cache_gqa_amd import kvq
    lib = kvq.load()
    fake = 1 << 20
    reg = kvq.Region(k_format=1, v_format=1, k=fake, v=fake, k_scale=fake, v_scale=fake, witness=fake,
                     k_exact=fake, k_exact_format=0, length=12628)
    a = kvq.AttnArgs(batch=64, num_q_heads=32, num_kv_heads=8, head_dim=128, sm_scale=SM_SCALE, split_tokens=0,
                     plan_flags=kvq.PLAN_NO_TEAM, status=fake, q=fake, prefix=kvq.Region(), suffix=reg, out=fake)
    m = kvq.MeterOut(tv=fake, bound_raw=fake, meter=fake, log_a=fake)
    assert lib.kvq_decode_attn_noalloc(ctypes.byref(a), ctypes.byref(m), None) == 6
