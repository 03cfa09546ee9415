"""Seeded synthetic inputs for the quantized-KV decode step.

This package holds only input synthesis (random numbers, the RoPE rotation
that makes keys post-RoPE, bf16 rounding of the exact cache).  It holds none of
the method's arithmetic (no quantization, witness, attention or meter) and
imports neither the oracle nor the HIP library; both sides receive the same
tensors from here.
"""
from .configs import CONFIGS, Config, RegionCfg, small_variant  # noqa: F401
from .gen import gen_layer, outlier_channels  # noqa: F401
