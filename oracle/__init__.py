"""Oracle: a plain, slow, float64 CPU reference of the quantized-KV decode path.

TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check of
``__graft_entry__`` and the ``cpu_baseline`` leg of ``bench.py`` may import
this package.  It shares no code with the HIP library and imports nothing from
it; the two meet only through the seeded inputs of ``workloads``.

Modules
-------
numerics    FP8 E4M3FN codec, fp16 round-up, bf16 rounding (definitions).
philox      Philox4x32-10 (Salmon et al., SC 2011) and the dither stream.
quant       FP8 per-token and dithered INT8 encoders, the band-norm witness.
attention   logits, softmaxes, output, TV, Theorem 1 bound, meter.
pipeline    one (layer, request, KV head) cell end to end.
accounting  raw payload and algorithmic byte counts.

Every function is pinned by tests under tests/ (test_oracle_*.py) against
values the pages print, closed forms, invariants or brute force, except where
its docstring says "parity unpinned".
"""
from . import accounting, attention, numerics, philox, pipeline, quant  # noqa: F401
