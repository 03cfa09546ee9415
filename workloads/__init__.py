"""Seeded synthetic inputs for the quantized-KV decode step.

This package holds only input synthesis (random numbers, the RoPE rotation
that makes keys post-RoPE, bf16 rounding of the exact cache).  It holds none of
the method's arithmetic (no quantization, witness, attention or meter) and
imports neither the oracle nor the HIP library; both sides receive the same
tensors from here.
"""
from .configs import (CONFIGS, INT8_DITHER_B8_S32K, LONG_B4_S128K_SPLIT, QWEN3_B64_S12628_K8V8,  # noqa: F401
                      QWEN3_SHARED_CARTRIDGE_PAGED, TINY_K16V8_CARTRIDGE, Config, RegionCfg, small_variant)
from .gen import gen_layer, outlier_channels  # noqa: F401
