"""End-to-end reference for one (layer, request, KV head) cell.

TEST INFRASTRUCTURE ONLY: nothing on the product path imports this module.

Chains the write path (oracle.quant) and the read path (oracle.attention) the
way the WitCert meter loop (Sec. 6, "The meter loop") orders them: quantize and
store the witness at write time, then attend and meter at read time.  Region
formats: "bf16" (stored as is), "fp8" (E4M3 per-token scale), "int8"
(dithered INT8 with per-(256-token block, channel) scales) and "int8g32"
(dithered INT8 with per-(token, 32-channel group) scales).
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
    # fixed outlier RoPE pairs of the keys (WitCert Sec. 6.2.5), "int8g32" keys
    # only: (h_kv, m) pair indices, one set per KV head
    outlier_pairs: Optional[np.ndarray] = None


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
    k_out: Optional[np.ndarray] = None   # (T, 2m) stored outlier values of the keys
    k_bypass: Optional[np.ndarray] = None   # bool (d,) channels those values replace


def _encode_one(x, fmt, spec: RegionSpec, kv: int, kv_head: int, pairs=None):
    x = np.asarray(x, np.float64)
    if fmt == "bf16":
        codes = f64_to_bf16_bits(x)
        return codes, None, bf16_bits_to_f64(codes), 0
    if fmt == "fp8":
        codes, s = quant.fp8_token_quantize(x)
        return codes, s, quant.fp8_token_dequant(codes, s), 0
    if fmt in ("int8", "int8g32"):
        xi = dither(spec.seed, spec.layer, kv_head, spec.stream,
                    np.arange(x.shape[0]), x.shape[1])
        if fmt == "int8g32":
            if pairs is not None and len(pairs) > 0:
                mask, _ = quant.outlier_mask(pairs, x.shape[1])
                quant.outlier_values(x, pairs)               # exactness check
                codes, s, clipped = quant.int8_dither_g32_quantize(x, xi, bypass=mask)
                return codes, s, quant.int8_dither_g32_dequant(codes, s, xi, bypass=mask, x_bypass=x), clipped
            codes, s, clipped = quant.int8_dither_g32_quantize(x, xi)
            return codes, s, quant.int8_dither_g32_dequant(codes, s, xi), clipped
        codes, s, clipped = quant.int8_dither_quantize(x, xi)
        return codes, s, quant.int8_dither_dequant(codes, s, xi), clipped
    raise ValueError(fmt)


def encode_region(k, v, spec: RegionSpec, kv_head: int) -> EncodedRegion:
    """Quantize one (region, request, KV head) slice and store its witness."""
    pairs = None
    if spec.outlier_pairs is not None:
        if spec.k_fmt != "int8g32":
            raise ValueError("outlier pairs need int8g32 keys")
        pairs = np.asarray(spec.outlier_pairs)[kv_head]
    kc, ks, kh, c1 = _encode_one(k, spec.k_fmt, spec, 0, kv_head, pairs)
    vc, vs, vh, c2 = _encode_one(v, spec.v_fmt, spec, 1, kv_head)
    w = w16 = None
    if spec.witness:
        w, w16 = quant.witness(kh, k)
    v_rec = quant.value_witness(vh, v) if spec.value_witness else None
    k_out = k_bypass = None
    if pairs is not None:
        k_out = quant.outlier_values(k, pairs)
        k_bypass = quant.outlier_mask(pairs, np.asarray(k).shape[1])[0]
    return EncodedRegion(kc, ks, vc, vs, w, w16, kh, vh, c1 + c2, v_rec, k_out, k_bypass)


def key_dither_steps(enc: EncodedRegion, spec: RegionSpec, n: int) -> np.ndarray:
    """(n, d) dither step of the stored keys per token and channel: the
    block's scale for INT8 (WitCert Sec. 4.2: the residual is uniform on
    [-s/2, s/2]), 0 for keys stored exactly (BF16).  FP8 keys have no dither."""
    if spec.k_fmt == "int8":
        return np.asarray(enc.k_scale, np.float64)[np.arange(n) // quant.BLOCK]
    if spec.k_fmt == "int8g32":
        steps = np.repeat(np.asarray(enc.k_scale, np.float64)[:n], quant.GROUP, axis=1)
        if enc.k_bypass is not None:                     # stored exactly: no dither
            steps[:, enc.k_bypass] = 0.0
        return steps
    if spec.k_fmt == "bf16":
        return np.zeros((n, np.asarray(enc.k_hat).shape[1]))
    raise ValueError("Tier B needs dithered INT8 keys or keys stored exactly")


def block_report(res, region_lengths, region_capacities, block: int = quant.BLOCK):
    """Block-decomposable risk report (WitCert Sec. 6.3.5): blocks of 256
    tokens aligned at the start of each region (the INT8 scale blocks), in
    logical order, numbered over the regions' capacities.  Per query head and
    block j:
        mass_j     = sum_{t in j} p~_t
        excess_j   = sum_{t in j} p~_t (e^{c_t} - 1)    (sum_j excess_j = A - 1)
        excess_b_j = mass_j (e^{u_j} - 1)              (Tier B; u shared by the block)
        order      = blocks by decreasing excess (excess_b when Tier B was
                     computed), ties by lower index.
    res: a decode_step result; region_lengths: tokens present per region;
    region_capacities: tokens per region that fix the block numbering."""
    pt, c = res["p_tilde"], res["c"]
    G = pt.shape[0]
    n_blocks = sum(-(-cap // block) for cap in region_capacities)
    mass = np.zeros((G, n_blocks))
    excess = np.zeros((G, n_blocks))
    excess_b = np.zeros((G, n_blocks))
    t0 = 0
    b0 = 0
    for n, cap in zip(region_lengths, region_capacities):
        for j in range(-(-n // block)):
            sl = slice(t0 + j * block, t0 + min(n, (j + 1) * block))
            mass[:, b0 + j] = np.sum(pt[:, sl], axis=1)
            excess[:, b0 + j] = np.sum(pt[:, sl] * np.expm1(c[:, sl]), axis=1)
            if "u" in res:
                excess_b[:, b0 + j] = mass[:, b0 + j] * np.expm1(res["u"][:, sl.start])
        t0 += n
        b0 += -(-cap // block)
    key = excess_b if "u" in res else excess
    order = np.array([sorted(range(n_blocks), key=lambda j: (-key[h, j], j)) for h in range(G)],
                     dtype=np.int64).reshape(G, n_blocks)
    return dict(block_mass=mass, block_excess=excess, block_excess_b=excess_b, block_order=order)


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
