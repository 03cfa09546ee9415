"""The five decode-step workloads and their small parity variants.

Shapes follow the pages: the Qwen3-8B shape (36 layers, 8 KV heads, head_dim
128) and its 632-position cartridge and 12,628-token KV (cartridge page, byte
table); the 32,768-token synthetic-K setting and the 128k long-context setting
of WitCert (Sec. 5, 6.3.1).  32 query heads (GQA group 4) and RoPE theta 1e6
complete the model shape.
"""
from __future__ import annotations

import dataclasses
from dataclasses import dataclass, field
from typing import List, Optional


@dataclass(frozen=True)
class RegionCfg:
    length: int                  # tokens (suffix: per-request capacity)
    k_fmt: str                   # "bf16" | "fp8" | "int8"
    v_fmt: str
    exact_k: bool                # exact keys kept for the TV (False: stored keys are exact)
    witness: bool                # witness stored for the keys
    paged: bool = False
    page_size: int = 16
    k_input: str = "bf16"        # precision of the exact cache ("bf16" or "fp32")


@dataclass(frozen=True)
class Config:
    index: int
    name: str
    layers: int
    batch: int
    h_q: int
    h_kv: int
    prefix: Optional[RegionCfg]
    suffix: RegionCfg
    rope: bool
    key_dist: str                # "outlier4x8" | "student_t3_8ch"
    split_tokens: int = 0        # 0: library default
    theta: float = 1.0e6
    head_dim: int = 128
    suffix_lens: Optional[tuple] = None   # ragged per-request lengths (None: all full)
    description: str = ""

    @property
    def group(self) -> int:
        return self.h_q // self.h_kv

    @property
    def seed(self) -> int:
        return 20260000 + self.index

    def lens(self) -> List[int]:
        if self.suffix_lens is not None:
            return list(self.suffix_lens)
        return [self.suffix.length] * self.batch

    def context_tokens(self) -> int:
        """Sum over requests of (prefix + suffix) tokens."""
        p = self.prefix.length if self.prefix else 0
        return sum(p + n for n in self.lens())


CONFIGS = {
    1: Config(1, "tiny-k16v8-cartridge", layers=1, batch=1, h_q=4, h_kv=1,
              prefix=RegionCfg(632, "bf16", "fp8", exact_k=False, witness=False),
              suffix=RegionCfg(64, "bf16", "fp8", exact_k=False, witness=False),
              rope=False, key_dist="outlier4x8",
              description="1 layer, 1 KV head, G=4, batch 1, 632-position prefix + 64 suffix, "
                          "K BF16 / V FP8 per-token"),
    2: Config(2, "qwen3-8b-layer-shared-cartridge", layers=1, batch=16, h_q=32, h_kv=8,
              prefix=RegionCfg(632, "bf16", "fp8", exact_k=False, witness=False),
              suffix=RegionCfg(1024, "bf16", "bf16", exact_k=False, witness=False,
                               paged=True, page_size=16),
              rope=True, key_dist="outlier4x8",
              description="1 layer, 32 q / 8 KV heads, batch 16, shared 632-position K16/V8 "
                          "prefix + paged BF16 suffix of 1,024 tokens"),
    3: Config(3, "qwen3-8b-b64-12628-k8v8", layers=36, batch=64, h_q=32, h_kv=8,
              prefix=None,
              suffix=RegionCfg(12628, "fp8", "fp8", exact_k=True, witness=True),
              rope=True, key_dist="outlier4x8",
              description="36 layers, 32 q / 8 KV heads, batch 64, 12,628 tokens, K8/V8 FP8 "
                          "per-token vs BF16 exact, TV + witness bound"),
    4: Config(4, "int8-dither-b8-32k", layers=28, batch=8, h_q=32, h_kv=8,
              prefix=None,
              suffix=RegionCfg(32768, "int8", "int8", exact_k=True, witness=True),
              rope=True, key_dist="outlier4x8",
              description="28 layers, 32 q / 8 KV heads, batch 8, 32,768 tokens, dithered INT8 "
                          "K and V with per-(256-token block, channel) fp16 scales"),
    5: Config(5, "long-context-b4-128k-split", layers=1, batch=4, h_q=32, h_kv=8,
              prefix=None,
              suffix=RegionCfg(131072, "fp8", "fp8", exact_k=True, witness=True),
              rope=True, key_dist="student_t3_8ch", split_tokens=1024,
              description="1 layer, 32 q / 8 KV heads, batch 4, 131,072 tokens, K8/V8 FP8, "
                          "Student-t(3) keys on 8 channels, 1,024-token split-K"),
}


# the workloads by name (CONFIGS is keyed by workload number)
TINY_K16V8_CARTRIDGE = CONFIGS[1]
QWEN3_SHARED_CARTRIDGE_PAGED = CONFIGS[2]
QWEN3_B64_S12628_K8V8 = CONFIGS[3]
INT8_DITHER_B8_S32K = CONFIGS[4]
LONG_B4_S128K_SPLIT = CONFIGS[5]


def small_variant(cfg: Config, *, batch: int = 2, layers: int = 1, prefix_len: Optional[int] = None,
                  suffix_len: Optional[int] = None, lens: Optional[tuple] = None,
                  h_kv: Optional[int] = None, **kw) -> Config:
    """A reduced copy of a workload (same formats and distributions) that the
    oracle finishes in seconds; the name records the change."""
    pre = cfg.prefix
    if pre is not None and prefix_len is not None:
        pre = dataclasses.replace(pre, length=prefix_len)
    suf = cfg.suffix
    if suffix_len is not None:
        suf = dataclasses.replace(suf, length=suffix_len)
    for key in list(kw):
        if key.startswith("suffix_"):
            suf = dataclasses.replace(suf, **{key[len("suffix_"):]: kw.pop(key)})
    hk = h_kv if h_kv is not None else cfg.h_kv
    hq = cfg.group * hk
    return dataclasses.replace(cfg, name=cfg.name + "-small", batch=batch, layers=layers,
                               prefix=pre, suffix=suf, h_kv=hk, h_q=hq, suffix_lens=lens, **kw)
