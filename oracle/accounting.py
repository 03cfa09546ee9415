"""Byte accounting of the cache layouts.

TEST INFRASTRUCTURE ONLY: nothing on the product path imports this module.

Raw payload per token (cartridge page, table "Keys carry the cartridge
quantization loss"): layers * kv_heads * head_dim * (key bytes + value bytes),
without scales or metadata.  BF16 is 2 bytes per element and FP8 E4M3 is 1.

Algorithmic bytes per token-head of one decode step are what the method itself
must move for one cached token of one KV head in one layer: key payload, value
payload, their scales, the stored witness (WitCert, Sec. 4.1: 2B = 32 bytes)
and, when the exact TV is measured, the exact bf16 key.
"""
from __future__ import annotations

ELEM_BYTES = {"bf16": 2, "fp8": 1, "int8": 1, "int8g32": 1, "fp32": 4}
KIB = 1024
MIB = 1024 ** 2
GIB = 1024 ** 3


def raw_bytes_per_token(k_fmt: str, v_fmt: str, layers: int = 36,
                        kv_heads: int = 8, head_dim: int = 128) -> int:
    return layers * kv_heads * head_dim * (ELEM_BYTES[k_fmt] + ELEM_BYTES[v_fmt])


def payload_table(tokens_full: int = 12628, cartridge: int = 632):
    """Rows of the four layouts: (name, KiB/token, GiB per full KV, MiB per cartridge)."""
    rows = []
    for name, kf, vf in (("K16/V16", "bf16", "bf16"), ("K16/V8", "bf16", "fp8"),
                         ("K8/V16", "fp8", "bf16"), ("K8/V8", "fp8", "fp8")):
        b = raw_bytes_per_token(kf, vf)
        rows.append((name, b / KIB, b * tokens_full / GIB, b * cartridge / MIB))
    return rows


def token_head_bytes(k_fmt: str, v_fmt: str, *, exact_k: bool, witness: bool,
                     head_dim: int = 128, n_bands: int = 16,
                     block: int = 256) -> float:
    """Algorithmic bytes for one token of one KV head in one layer."""
    total = 0.0
    for fmt in (k_fmt, v_fmt):
        total += head_dim * ELEM_BYTES[fmt]
        if fmt == "fp8":
            total += 4.0                              # fp32 per-token scale
        elif fmt == "int8":
            total += 2.0 * head_dim / block           # fp16 per (block, channel)
        elif fmt == "int8g32":
            total += 2.0 * head_dim / 32              # fp16 per (token, 32-channel group)
    if witness:
        total += 2.0 * n_bands
    if exact_k:
        total += 2.0 * head_dim
    return total
