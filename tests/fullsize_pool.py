"""Every-cell parity of a full-size layer, with the oracle in a process pool.

The GPU side runs in the test process (GpuCase); its inputs, stored cache
and results are written to .npy files, and spawned workers (no GPU) map
them and run the same checks as every other parity test (cells.oracle_cell,
check_stored, check_results) on a share of the (request, KV head) cells.
Nothing here does arithmetic of the method: it moves arrays and calls the
oracle and the shared checks."""
from __future__ import annotations

import json
import os
import sys
from types import SimpleNamespace

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
TENSORS = ("k", "v", "k_scale", "v_scale", "witness", "v_witness", "k_outliers")


def _np(t):
    import torch
    t = t.detach().cpu().contiguous()
    if t.dtype in (torch.bfloat16, torch.float16):
        return t.view(torch.int16).numpy(), str(t.dtype).split(".")[1]
    return t.numpy(), ""


def dump(case, results: dict, d: str) -> None:
    """Write the case's inputs, stored regions and each named result (out,
    meter dict) under directory d."""
    os.makedirs(d, exist_ok=True)
    dtypes = {}

    def save(name, t):
        a, kind = _np(t)
        np.save(os.path.join(d, name + ".npy"), a)
        dtypes[name] = kind

    for k, t in case.inp.items():
        save("inp." + k, t)
    for region, st in (("suffix", case.suffix_store), ("prefix", case.prefix_store)):
        if st is None:
            continue
        for f in TENSORS:
            t = getattr(st, f)
            if t is not None:
                save(f"{region}.{f}", t)
    for name, (out, m) in results.items():
        save(f"res.{name}.out", out)
        for k, t in m.items():
            save(f"res.{name}.m.{k}", t)
    with open(os.path.join(d, "dtypes.json"), "w") as f:
        json.dump(dtypes, f)


def _load(d: str):
    import torch
    with open(os.path.join(d, "dtypes.json")) as f:
        kinds = json.load(f)
    out = {}
    for name, kind in kinds.items():
        a = np.load(os.path.join(d, name + ".npy"), mmap_mode="c")
        t = torch.from_numpy(a)
        if kind:
            t = t.view(getattr(torch, kind))
        out[name] = t
    return out


def _case(d: str, cfg, layer: int, value_witness: bool, opairs):
    """A CPU stand-in of cells.GpuCase with the dumped arrays."""
    a = _load(d)
    inp = {k[4:]: t for k, t in a.items() if k.startswith("inp.")}

    def stored(region):
        if not any(k.startswith(region + ".") for k in a):
            return None
        return SimpleNamespace(**{f: a.get(f"{region}.{f}") for f in TENSORS})

    case = SimpleNamespace(cfg=cfg, layer=layer, inp=inp, fp32_exact=False, value_witness=value_witness,
                           opairs=opairs, suffix_store=stored("suffix"), prefix_store=stored("prefix"))
    case.prefix_view = True if case.prefix_store is not None else None
    results = {}
    for k, t in a.items():
        if k.startswith("res."):
            _, name, rest = k.split(".", 2)
            out, m = results.setdefault(name, [None, {}])
            if rest == "out":
                results[name][0] = t
            else:
                m[rest[2:]] = t
    return case, results


def init_worker():
    os.environ["OMP_NUM_THREADS"] = "1"
    os.environ["HIP_VISIBLE_DEVICES"] = ""             # the workers never touch a GPU
    for p in (ROOT, os.path.join(ROOT, "tests")):
        if p not in sys.path:
            sys.path.insert(0, p)
    # one thread per worker: numpy is already imported here (this module),
    # so its BLAS pool is limited now rather than through the environment
    from threadpoolctl import threadpool_limits
    threadpool_limits(1)
    import torch
    torch.set_num_threads(1)


def check_cells(d, cfg, layer, cells, tier_b_delta=None, value_witness=False, opairs=None, stored=True):
    """Oracle and checks for `cells` [(b, kvh)]; returns (count, worst errors
    per result name).  Any bar missed raises (AssertionError with the cell)."""
    from cells import check_results, check_stored, oracle_cell
    case, results = _case(d, cfg, layer, value_witness, opairs)
    worst = {}
    for b, kvh in cells:
        encs, ref = oracle_cell(case, b, kvh, tier_b_delta=tier_b_delta)
        if stored:
            check_stored(case, b, kvh, encs)
        for name, (out, m) in results.items():
            try:
                w = check_results(case, out, m, b, kvh, ref)
            except AssertionError as e:
                raise AssertionError(f"{name}: cell (request {b}, KV head {kvh}): {e}") from None
            ww = worst.setdefault(name, {})
            for k, v in w.items():
                ww[k] = max(ww.get(k, 0.0), v)
    return len(cells), worst


def workers() -> int:
    return max(1, min(16, len(os.sched_getaffinity(0))))
