"""Write path of the quantized cache: encoders, dequantizers and the witness.

TEST INFRASTRUCTURE ONLY: nothing on the product path imports this module.

Every function takes one (region, KV head) slice: x has shape (T, d) and holds
the exact cache values (bf16 or fp32 inputs, carried as float64, exact).

FP8 per-token (cartridge page, byte table and "What fake quantization does"):
    amax = max_c |x_c|;  s = fp32(amax / 448)  (s = 1 when amax = 0)
    y_c  = fp32(x_c / s) clamped to [-448, 448];  code = E4M3(y_c)
    x^_c = E4M3value(code) * s                       (exact in float64)
  The scale is stored as fp32 and the same stored scale encodes and decodes
  (WitCert, Sec. 6.2.1: quantize with the stored scale).

INT8 with subtractive dither, per (256-token block, channel) scales
(WitCert, Sec. 4.2 "Subtractive dither" and Sec. 6.1.1 "BLK = 256"):
    s32 = fp32(amax_blk,c / 126.5);  s = fp16(s32) rounded to nearest even
    y = fp32(x / s);  z = fp32(y + xi);  code = rint(z) (ties to even), |code| <= 127
    x^ = s * (code - xi)                              (exact in float64)
  with xi the Philox dither of oracle.philox.  s = 0 gives code 0 and x^ = 0.

Value record: rho = ||v^ - v|| and ||v|| per token, the two norms of the output
bound (WitCert Sec. 3), summed in coordinate order and rounded up the same way.

Witness (WitCert, Sec. 4.1, Eq. (2)): r = x^ - x;  w_b = ||r_b|| over the 8
coordinates of band b, stored as fp16 rounded toward +infinity.  Bands follow
the rotate-half RoPE pairing (coordinate j pairs with j + d/2); band b holds
pairs 4b..4b+3, i.e. coordinates {4b..4b+3} and {d/2+4b..d/2+4b+3} for d=128,
B=16.  The sum of squares is taken in float64 in that coordinate order, one
rounded operation per square and per addition, then a correctly rounded sqrt.
The residual r is exact in float64 for every format here.  Before the fp16
round-up the norm is multiplied (one rounded float64 product) by 1 + 2^-48,
which exceeds the relative error of the float64 steps, so the stored value is
an upper bound of the exact norm (soundness of Theorem 2 after storage).
"""
from __future__ import annotations

import numpy as np

from .numerics import E4M3_MAX, e4m3_decode, e4m3_encode, fp16_round_up

INT8_Q = 127
INT8_DIV = 126.5          # Q - 1/2
BLOCK = 256
N_BANDS = 16


def band_coords(d: int = 128, n_bands: int = N_BANDS) -> np.ndarray:
    """(n_bands, 2 * pairs_per_band) coordinate indices, in summation order."""
    half = d // 2
    ppb = half // n_bands
    rows = []
    for b in range(n_bands):
        first = [b * ppb + i for i in range(ppb)]
        rows.append(first + [half + j for j in first])
    return np.array(rows, dtype=np.int64)


def fp8_token_quantize(x: np.ndarray):
    """x (T, d) exact values -> (codes uint8 (T, d), scale float32 (T,))."""
    x = np.asarray(x, dtype=np.float64)
    x32 = x.astype(np.float32)
    if not np.array_equal(x32.astype(np.float64), x):
        raise ValueError("fp8_token_quantize: inputs must be float32-exact")
    amax = np.max(np.abs(x32), axis=1)
    s = (amax / np.float32(E4M3_MAX)).astype(np.float32)
    s = np.where(amax == 0, np.float32(1.0), s).astype(np.float32)
    y = (x32 / s[:, None]).astype(np.float32)
    y = np.clip(y, np.float32(-E4M3_MAX), np.float32(E4M3_MAX))
    return e4m3_encode(y), s


def fp8_token_dequant(codes: np.ndarray, scale: np.ndarray) -> np.ndarray:
    return e4m3_decode(codes) * np.asarray(scale, np.float64)[:, None]


def int8_dither_quantize(x: np.ndarray, xi: np.ndarray, block: int = BLOCK):
    """x (T, d) exact values, xi (T, d) float32 dither.

    Returns (codes int8 (T, d), scale float16 (ceil(T/block), d), clipped count).
    """
    x = np.asarray(x, dtype=np.float64)
    x32 = x.astype(np.float32)
    if not np.array_equal(x32.astype(np.float64), x):
        raise ValueError("int8_dither_quantize: inputs must be float32-exact")
    xi = np.asarray(xi, dtype=np.float32)
    T, d = x.shape
    nb = (T + block - 1) // block
    codes = np.zeros((T, d), np.int8)
    scales = np.zeros((nb, d), np.float16)
    clipped = 0
    for j in range(nb):
        sl = slice(j * block, min(T, (j + 1) * block))
        amax = np.max(np.abs(x32[sl]), axis=0)
        s32 = (amax / np.float32(INT8_DIV)).astype(np.float32)
        s16 = s32.astype(np.float16)             # round to nearest even
        scales[j] = s16
        s = s16.astype(np.float32)
        with np.errstate(divide="ignore", invalid="ignore"):
            y = (x32[sl] / s[None, :]).astype(np.float32)
            z = (y + xi[sl]).astype(np.float32)
        c = np.rint(z)
        c = np.where(s[None, :] == 0, 0.0, c)
        clipped += int(np.sum(np.abs(c) > INT8_Q))
        codes[sl] = np.clip(c, -INT8_Q, INT8_Q).astype(np.int8)
    return codes, scales, clipped


def int8_dither_dequant(codes: np.ndarray, scales: np.ndarray, xi: np.ndarray,
                        block: int = BLOCK) -> np.ndarray:
    codes = np.asarray(codes, dtype=np.float64)
    T = codes.shape[0]
    s = np.asarray(scales, np.float64)[np.arange(T) // block]
    out = s * (codes - np.asarray(xi, np.float32).astype(np.float64))
    return np.where(s == 0, 0.0, out)


GROUP = 32


def outlier_mask(pairs, d: int = 128):
    """Channels of a fixed set of outlier RoPE pairs (WitCert Sec. 6.2.5: one
    channel set per (layer, KV head), m pairs): under the rotate-half pairing
    pair j is channels j and j + d/2.  Slot i is active when its index lies
    in [0, d/2) and no earlier slot holds the same index; inactive slots
    bypass nothing.
    Returns (bool (d,) bypassed channels, list of active flags per slot)."""
    mask = np.zeros(d, dtype=bool)
    active = []
    seen = set()
    for j in (int(p) for p in (pairs if pairs is not None else ())):
        ok = 0 <= j < d // 2 and j not in seen
        active.append(ok)
        if ok:
            seen.add(j)
            mask[j] = mask[j + d // 2] = True
    return mask, active


def outlier_values(x: np.ndarray, pairs) -> np.ndarray:
    """The bypassed values of every token, slot by slot: (T, 2m) with
    [:, 2i] = x[:, P_i] and [:, 2i + 1] = x[:, P_i + d/2] for an active slot,
    0 for an inactive one.  They are stored exactly (the keys' own 16-bit
    values), so they must be bf16-exact."""
    x = np.asarray(x, np.float64)
    d = x.shape[1]
    _, active = outlier_mask(pairs, d)
    out = np.zeros((x.shape[0], 2 * len(active)))
    for i, (j, ok) in enumerate(zip(pairs if pairs is not None else (), active)):
        if ok:
            out[:, 2 * i] = x[:, int(j)]
            out[:, 2 * i + 1] = x[:, int(j) + d // 2]
    bf = out.astype(np.float32).view(np.uint32) & np.uint32(0xFFFF0000)
    if not np.array_equal(bf.view(np.float32).astype(np.float64), out):
        raise ValueError("outlier_values: bypassed values must be bf16-exact")
    return out


def int8_dither_g32_quantize(x: np.ndarray, xi: np.ndarray, group: int = GROUP,
                             bypass: np.ndarray = None, amax_excludes_bypass: bool = True):
    """Per-token channel-group scales (WitCert Sec. 6.2.3, Table 4: token x
    G_c-channel groups, G_c = 32 the default; paging-safe): every token and
    group of 32 channels has its own s = fp16(fp32(amax / 126.5)); the codes
    are encoded exactly as in the block format, with the same dither.

    bypass: bool (d,) channels stored exactly beside the codes (the fixed
    outlier pairs of Sec. 6.2.5); they leave the group maximum (the page's
    second step; amax_excludes_bypass=False keeps them in, the "bypass, amax
    unchanged" treatment of its Table 5) and their codes are 0.

    x (T, d) exact values, xi (T, d) float32 dither.
    Returns (codes int8 (T, d), scale float16 (T, d / group), clipped count)."""
    x = np.asarray(x, dtype=np.float64)
    x32 = x.astype(np.float32)
    if not np.array_equal(x32.astype(np.float64), x):
        raise ValueError("int8_dither_g32_quantize: inputs must be float32-exact")
    xi = np.asarray(xi, dtype=np.float32)
    T, d = x.shape
    ng = d // group
    byp = np.zeros(d, dtype=bool) if bypass is None else np.asarray(bypass, dtype=bool)
    a = np.abs(x32)
    if amax_excludes_bypass:
        a = np.where(byp[None, :], np.float32(0.0), a)
    amax = np.max(a.reshape(T, ng, group), axis=2)
    s16 = (amax / np.float32(INT8_DIV)).astype(np.float32).astype(np.float16)
    s = np.repeat(s16.astype(np.float32), group, axis=1)
    with np.errstate(divide="ignore", invalid="ignore"):
        y = (x32 / s).astype(np.float32)
        z = (y + xi).astype(np.float32)
    c = np.rint(z)
    c = np.where((s == 0) | byp[None, :], 0.0, c)
    clipped = int(np.sum(np.abs(c) > INT8_Q))
    return np.clip(c, -INT8_Q, INT8_Q).astype(np.int8), s16, clipped


def int8_dither_g32_dequant(codes: np.ndarray, scales: np.ndarray, xi: np.ndarray,
                            group: int = GROUP, bypass: np.ndarray = None,
                            x_bypass: np.ndarray = None) -> np.ndarray:
    """x^ = s (code - xi) per group; bypassed channels take their stored
    exact values x_bypass (T, d) instead."""
    s = np.repeat(np.asarray(scales, np.float64), group, axis=1)
    out = s * (np.asarray(codes, np.float64) - np.asarray(xi, np.float32).astype(np.float64))
    out = np.where(s == 0, 0.0, out)
    if bypass is not None:
        out = np.where(np.asarray(bypass, bool)[None, :], np.asarray(x_bypass, np.float64), out)
    return out


WITNESS_INFLATE = 1.0 + 2.0 ** -48


def value_witness(v_hat: np.ndarray, v: np.ndarray) -> np.ndarray:
    """Value record of each token (WitCert Sec. 3 output bound, Sec. 4.2
    "Value side"): rho = ||v^_t - v_t|| and ||v_t||, each summed in float64 over
    coordinates 0..d-1 in order (one rounding per square and per addition),
    square-rooted, multiplied by 1 + 2^-48 and rounded up to fp16.
    Returns float16 (T, 2): [:, 0] = rho, [:, 1] = ||v||."""
    out = np.empty((np.asarray(v).shape[0], 2), np.float16)
    for col, x in enumerate((np.asarray(v_hat, np.float64) - np.asarray(v, np.float64),
                             np.asarray(v, np.float64))):
        acc = x[:, 0] * x[:, 0]
        for c in range(1, x.shape[1]):
            acc = acc + x[:, c] * x[:, c]
        out[:, col] = fp16_round_up(np.sqrt(acc) * WITNESS_INFLATE)
    return out


def witness(x_hat: np.ndarray, x: np.ndarray, n_bands: int = N_BANDS):
    """Per-band residual norms: (w float64 (T, B), w16 float16 (T, B) rounded up)."""
    r = np.asarray(x_hat, np.float64) - np.asarray(x, np.float64)
    coords = band_coords(r.shape[1], n_bands)
    w = np.empty((r.shape[0], n_bands), np.float64)
    for b in range(n_bands):
        acc = r[:, coords[b, 0]] * r[:, coords[b, 0]]
        for c in coords[b, 1:]:
            acc = acc + r[:, c] * r[:, c]
        w[:, b] = np.sqrt(acc)
    return w, fp16_round_up(w * WITNESS_INFLATE)
