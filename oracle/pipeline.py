"""End-to-end reference for one (layer, request, KV head) cell.

TEST INFRASTRUCTURE ONLY: nothing on the product path imports this module.

Chains the write path (oracle.quant) and the read path (oracle.attention) the
way the WitCert meter loop (Sec. 6, "The meter loop") orders them: quantize and
store the witness at write time, then attend and meter at read time.  Region
formats: "bf16" (stored as is), "fp8" (E4M3 per-token scale) and "int8"
(dithered INT8 with per-(256-token block, channel) scales).
"""
from __future__ import annotations

from dataclasses import dataclass
from typing import Optional

import numpy as np

from . import attention, quant
from .numerics import f64_to_bf16_bits, bf16_bits_to_f64
from .philox import dither


@dataclass
class RegionSpec:
    k_fmt: str
    v_fmt: str
    seed: int = 0
    layer: int = 0
    stream: int = 0           # dither stream id of this (region, request)
    witness: bool = True      # store/use a witness for the keys
    exact_k: bool = True      # the exact keys are available for TV
    value_witness: bool = False   # store/use the value record (rho, ||v||)


@dataclass
class EncodedRegion:
    k_codes: np.ndarray
    k_scale: Optional[np.ndarray]
    v_codes: np.ndarray
    v_scale: Optional[np.ndarray]
    w: Optional[np.ndarray]          # unrounded witness (float64)
    w16: Optional[np.ndarray]        # stored witness (float16, rounded up)
    k_hat: np.ndarray
    v_hat: np.ndarray
    clipped: int
    v_rec: Optional[np.ndarray] = None   # float16 (T, 2): rho, ||v||


def _encode_one(x, fmt, spec: RegionSpec, kv: int, kv_head: int):
    x = np.asarray(x, np.float64)
    if fmt == "bf16":
        codes = f64_to_bf16_bits(x)
        return codes, None, bf16_bits_to_f64(codes), 0
    if fmt == "fp8":
        codes, s = quant.fp8_token_quantize(x)
        return codes, s, quant.fp8_token_dequant(codes, s), 0
    if fmt == "int8":
        xi = dither(spec.seed, spec.layer, kv, kv_head, spec.stream,
                    np.arange(x.shape[0]), x.shape[1])
        codes, s, clipped = quant.int8_dither_quantize(x, xi)
        return codes, s, quant.int8_dither_dequant(codes, s, xi), clipped
    raise ValueError(fmt)


def encode_region(k, v, spec: RegionSpec, kv_head: int) -> EncodedRegion:
    """Quantize one (region, request, KV head) slice and store its witness."""
    kc, ks, kh, c1 = _encode_one(k, spec.k_fmt, spec, 0, kv_head)
    vc, vs, vh, c2 = _encode_one(v, spec.v_fmt, spec, 1, kv_head)
    w = w16 = None
    if spec.witness:
        w, w16 = quant.witness(kh, k)
    v_rec = quant.value_witness(vh, v) if spec.value_witness else None
    return EncodedRegion(kc, ks, vc, vs, w, w16, kh, vh, c1 + c2, v_rec)


def key_dither_steps(enc: EncodedRegion, spec: RegionSpec, n: int) -> np.ndarray:
    """(n, d) dither step of the stored keys per token and channel: the
    block's scale for INT8 (WitCert Sec. 4.2: the residual is uniform on
    [-s/2, s/2]), 0 for keys stored exactly (BF16).  FP8 keys have no dither."""
    if spec.k_fmt == "int8":
        return np.asarray(enc.k_scale, np.float64)[np.arange(n) // quant.BLOCK]
    if spec.k_fmt == "bf16":
        return np.zeros((n, np.asarray(enc.k_hat).shape[1]))
    raise ValueError("Tier B needs dithered INT8 keys or keys stored exactly")


def decode_cell(q, regions, sm_scale: float, delta_loc=None):
    """regions: list of (k_exact, EncodedRegion, RegionSpec) in logical order.
    delta_loc: Tier B's failure probability (None: Tier B not computed)."""
    ke = np.concatenate([np.asarray(r[0], np.float64) for r in regions])
    kh = np.concatenate([r[1].k_hat for r in regions])
    vh = np.concatenate([r[1].v_hat for r in regions])
    any_w = any(r[1].w16 is not None for r in regions)
    w16 = None
    if any_w:
        w16 = np.concatenate([
            r[1].w16.astype(np.float64) if r[1].w16 is not None
            else np.zeros((np.asarray(r[0]).shape[0], 16)) for r in regions])
    # regions whose exact keys are not available count as exact (TV term 0)
    ke_used = np.concatenate([
        np.asarray(r[0], np.float64) if r[2].exact_k else r[1].k_hat
        for r in regions])
    s_key = None
    if delta_loc is not None:
        s_key = np.concatenate([key_dither_steps(r[1], r[2], np.asarray(r[0]).shape[0])
                                for r in regions])
    v_rec = None
    if all(r[1].v_rec is not None for r in regions):
        v_rec = np.concatenate([r[1].v_rec.astype(np.float64) for r in regions])
    res = attention.decode_step(q, ke_used, kh, vh, w16, sm_scale, s_key=s_key, delta_loc=delta_loc,
                                v_rec=v_rec)
    res["k_exact_all"] = ke
    return res
