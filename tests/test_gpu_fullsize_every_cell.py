"""Every (request, KV head) cell of whole layers of the full-size workloads
against the oracle, in the launch plans the library and the bench use.

- configs 2, 3, 4 and 5: one whole layer each (the last: its layer id is the
  largest in the dither tag), all fields: stored codes, scales and witness
  bit-exact, outputs within 2e-3, TV, bound and meter within 1e-5;
- config 5 in both plans: the team launch the bench times (library split)
  and the workload's own 1,024-token split-K chunks, one oracle pass checking
  both;
- config 3: the meter fields and outputs of every cell of the other 35
  layers as well (about 7 s per layer with 16 workers).

The oracle runs in spawned worker processes (no GPU) over the dumped arrays;
the cell counts printed equal batch x KV heads for every layer checked
(the pages' lesson, WitCert Sec. 3 "Minimal counterexample": per cell, never
in aggregate)."""
import concurrent.futures as cf
import multiprocessing as mp
import os
import shutil

import pytest
import torch

import fullsize_pool
from cells import GpuCase, plan
from workloads import CONFIGS

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def pool():
    # (spawned workers inherit this environment: one BLAS thread each)
    for k in ("OMP_NUM_THREADS", "OPENBLAS_NUM_THREADS", "MKL_NUM_THREADS"):
        os.environ.setdefault(k, "1")
    ex = cf.ProcessPoolExecutor(max_workers=fullsize_pool.workers(), mp_context=mp.get_context("spawn"),
                                initializer=fullsize_pool.init_worker)
    yield ex
    ex.shutdown(wait=True, cancel_futures=True)


def check_layer(pool, tmp, cfg, layer, plans, stored=True):
    """plans: {name: (split_tokens, plan_flags)}; every cell of the layer in
    every plan against one oracle pass."""
    case = GpuCase(cfg, layer=layer, page_seed=1)
    results, plans_used = {}, {}
    for name, (split, flags) in plans.items():
        results[name] = case.run(split_tokens=split, plan_flags=flags)
        plans_used[name] = plan(case, split_tokens=split, plan_flags=flags)
    d = str(tmp / f"{cfg.index}-{layer}")
    fullsize_pool.dump(case, results, d)
    del case, results
    torch.cuda.empty_cache()
    cells = [(b, h) for b in range(cfg.batch) for h in range(cfg.h_kv)]
    per = max(1, len(cells) // (4 * fullsize_pool.workers()))
    futs = [pool.submit(fullsize_pool.check_cells, d, cfg, layer, cells[i:i + per], stored=stored)
            for i in range(0, len(cells), per)]
    n, worst = 0, {}
    for f in futs:
        k, w = f.result()
        n += k
        for name, ww in w.items():
            acc = worst.setdefault(name, {})
            for key, v in ww.items():
                acc[key] = max(acc.get(key, 0.0), v)
    shutil.rmtree(d, ignore_errors=True)
    assert n == cfg.batch * cfg.h_kv
    for name in plans:
        p = plans_used[name]
        print(f"[{cfg.name} layer {layer} {name}] cells={n} of {cfg.batch}x{cfg.h_kv} "
              f"plan team={p['team']} chunks={p['chunks']} chunk={p['chunk']} worst={worst.get(name)}",
              flush=True)
    return worst


@pytest.mark.parametrize("idx", [2, 3, 4, 5])
def test_every_cell_of_a_full_size_layer(gpu_lib, pool, tmp_path, idx):
    cfg = CONFIGS[idx]
    plans = {"library": (0, 0)}
    if cfg.split_tokens:
        plans["split-%d" % cfg.split_tokens] = (cfg.split_tokens, 0)
    check_layer(pool, tmp_path, cfg, cfg.layers - 1, plans)


@pytest.mark.parametrize("layer", range(CONFIGS[3].layers - 1))
def test_every_cell_of_the_batch64_step_by_layer(gpu_lib, pool, tmp_path, layer):
    """The 36-layer batch-64 workload: outputs and meter fields of every cell
    of every other layer (stored codes are checked on the last layer above)."""
    check_layer(pool, tmp_path, CONFIGS[3], layer, {"library": (0, 0)}, stored=False)
