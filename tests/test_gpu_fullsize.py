"""Parity at the workloads' full sizes on sampled cells that the oracle
computes one by one: the meter extensions, the group-scale INT8 format with
outlier pairs, and GQA groups of 1 and 8 (every cell of the plain workloads
is in test_gpu_fullsize_every_cell.py)."""
import pytest
import torch

from cells import GpuCase, check_block_report, check_results, check_stored, oracle_cell
from workloads import CONFIGS

pytestmark = pytest.mark.gpu

SAMPLES = {
    3: [(0, 0), (63, 7), (17, 3), (40, 5)],
    4: [(0, 0), (7, 7), (3, 2)],
    5: [(0, 0), (3, 7), (2, 4)],
}


EXTENSIONS = {4: 1e-9, 5: None}                   # Tier B's delta (INT8 keys only)


@pytest.mark.parametrize("idx", [4, 5])
def test_full_size_meter_extensions_sampled_cells(gpu_lib, idx):
    """Tier B (INT8), the value side and joint output bound, the two-sided
    form and the block report (512 blocks at 131,072 tokens) in one call at
    full size, on sampled cells against the oracle."""
    cfg = CONFIGS[idx]
    layer = cfg.layers - 1
    delta = EXTENSIONS[idx]
    case = GpuCase(cfg, layer=layer, page_seed=1, value_witness=True)
    out, m = case.run(split_tokens=cfg.split_tokens, tier_b_delta=delta, value_bound=True, two_sided=True,
                      report=True)
    worst = {}
    for b, kvh in SAMPLES[idx]:
        encs, ref = oracle_cell(case, b, kvh, tier_b_delta=delta)
        check_stored(case, b, kvh, encs)
        w = check_results(case, out, m, b, kvh, ref)
        check_block_report(case, m, b, kvh, ref, with_b=delta is not None)
        for k, v in w.items():
            worst[k] = max(worst.get(k, 0.0), v)
    assert {"value_err", "two_sided"} <= set(worst) and ("bound_b" in worst) == (delta is not None)
    assert torch.all(m["tv"] <= m["bound_two_sided"] + 1e-6)
    print(f"[{cfg.name} layer {layer} extensions] sampled={len(SAMPLES[idx])} worst={worst}", flush=True)
    del case
    torch.cuda.empty_cache()


@pytest.mark.parametrize("pairs", [0, 4])
def test_full_size_group_scales_and_outlier_pairs_sampled_cells(gpu_lib, pairs):
    """The 32,768-token INT8 workload stored with per-(token, 32-channel
    group) scales, without and with 4 fixed outlier RoPE pairs (WitCert Sec.
    6.2.3, 6.2.5), in 16-token pages: Tier A, Tier B and the value side at
    full size on sampled cells against the oracle."""
    import dataclasses
    base = CONFIGS[4]
    suf = dataclasses.replace(base.suffix, k_fmt="int8g32", v_fmt="int8g32", paged=True, page_size=16)
    cfg = dataclasses.replace(base, suffix=suf, name=base.name + f"-g32-paged-m{pairs}")
    layer = cfg.layers - 1
    case = GpuCase(cfg, layer=layer, page_seed=1, value_witness=True, n_outlier_pairs=pairs)
    out, m = case.run(tier_b_delta=1e-9, value_bound=True)
    worst = {}
    for b, kvh in SAMPLES[4]:
        encs, ref = oracle_cell(case, b, kvh, tier_b_delta=1e-9)
        check_stored(case, b, kvh, encs)
        w = check_results(case, out, m, b, kvh, ref)
        for k, v in w.items():
            worst[k] = max(worst.get(k, 0.0), v)
    assert {"bound_b", "value_err"} <= set(worst)
    assert torch.all(m["tv"] <= m["bound_raw"] + 1e-6) and torch.all(m["tv"] <= m["bound_b_raw"] + 1e-6)
    print(f"[{cfg.name} layer {layer}] sampled={len(SAMPLES[4])} worst={worst}", flush=True)
    del case
    torch.cuda.empty_cache()


@pytest.mark.parametrize("q_heads", [8, 64])
def test_full_size_gqa_groups_sampled_cells(gpu_lib, monkeypatch, q_heads):
    """The batch-64 x 12,628-token FP8 workload with 8 or 64 query heads over
    its 8 KV heads (GQA groups 1 and 8), in the launch the library plans for
    it: the 4-head tile padded with copies of the last head, or paired 4-head
    teams in one launch.  Sampled cells against the oracle."""
    import dataclasses
    from cells import plan
    base = CONFIGS[3]
    cfg = dataclasses.replace(base, h_q=q_heads, name=base.name + f"-hq{q_heads}")
    layer = cfg.layers - 1
    case = GpuCase(cfg, layer=layer, page_seed=1)
    p = plan(case)
    if q_heads == 64 and p["team"]:
        assert p["launches"] == 1 and p["grid"] >= 2 * p["team"] * p["n_teams"], p
    out, m = case.run()
    worst = {}
    for b, kvh in SAMPLES[3]:
        encs, ref = oracle_cell(case, b, kvh)
        check_stored(case, b, kvh, encs)
        w = check_results(case, out, m, b, kvh, ref)
        for k, v in w.items():
            worst[k] = max(worst.get(k, 0.0), v)
    assert torch.all(m["tv"] <= m["bound_raw"] + 1e-6)
    assert torch.all(torch.isfinite(out))
    print(f"[{cfg.name} layer {layer}] plan={p} sampled={len(SAMPLES[3])} worst={worst}", flush=True)
    del case
    torch.cuda.empty_cache()
