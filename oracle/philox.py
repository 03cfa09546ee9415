"""Philox4x32-10 counter-based generator and the dither stream built on it.

TEST INFRASTRUCTURE ONLY: nothing on the product path imports this module.

Philox4x32 is the counter-based generator of Salmon, Moraes, Dror and Shaw,
"Parallel random numbers: as easy as 1, 2, 3" (SC 2011), the reference WitCert
cites for its dither (WitCert, Sec. 6.2.1).  One round maps a 4-word counter
(c0, c1, c2, c3) and a 2-word key (k0, k1) through two 32x32->64 bit products
with the multipliers 0xD2511F53 and 0xCD9E8D57:
    (hi0, lo0) = M0 * c0,  (hi1, lo1) = M1 * c2
    out = (hi1 ^ c1 ^ k0, lo1, hi0 ^ c3 ^ k1, lo0)
and between rounds the key is advanced by the Weyl constants 0x9E3779B9 and
0xBB67AE85.  Ten rounds give Philox4x32-10.

Dither stream (WitCert, Sec. 6.2.1: the dither is regenerated at read time
from a counter built from (request, layer, KV head, token, channel), and
Sec. 6.3.1: Philox4x32-10 on that five-tuple, one generator call serving four
channels).  The five-tuple has no key/value component, so a token's keys and
values share their dither.  The pages fix neither the word layout nor the
mapping to [-1/2, 1/2); our reading:
    counter = (token, channel >> 2, (layer << 16) | kv_head, stream)
    key     = (seed & 0xFFFFFFFF, seed >> 32)
    u       = output word (channel & 3)
    xi      = (u >> 8) * 2^-24 - 1/2          (exact in float32)
with layer < 2^15 and kv_head < 2^16.
"""
from __future__ import annotations

import numpy as np

M0 = 0xD2511F53
M1 = 0xCD9E8D57
W0 = 0x9E3779B9
W1 = 0xBB67AE85
MASK32 = 0xFFFFFFFF


def philox4x32_10(ctr: np.ndarray, key) -> np.ndarray:
    """Philox4x32-10 on an (N, 4) array of uint32 counters; key = (k0, k1)."""
    c = np.asarray(ctr, dtype=np.uint64).reshape(-1, 4).copy() & MASK32
    k0 = np.uint64(int(key[0]) & MASK32)
    k1 = np.uint64(int(key[1]) & MASK32)
    m0 = np.uint64(M0)
    m1 = np.uint64(M1)
    for r in range(10):
        if r > 0:
            k0 = np.uint64((int(k0) + W0) & MASK32)
            k1 = np.uint64((int(k1) + W1) & MASK32)
        p0 = m0 * c[:, 0]            # < 2^64: exact in uint64
        p1 = m1 * c[:, 2]
        hi0, lo0 = p0 >> np.uint64(32), p0 & np.uint64(MASK32)
        hi1, lo1 = p1 >> np.uint64(32), p1 & np.uint64(MASK32)
        n0 = hi1 ^ c[:, 1] ^ k0
        n2 = hi0 ^ c[:, 3] ^ k1
        c = np.stack([n0, lo1, n2, lo0], axis=1)
    return c.astype(np.uint32)


def dither_counters(tokens, channels, layer: int, kv_head: int, stream: int):
    """Counter words for every (token, channel) pair (broadcast shapes)."""
    t = np.asarray(tokens, dtype=np.uint64)
    ch = np.asarray(channels, dtype=np.uint64)
    t, ch = np.broadcast_arrays(t, ch)
    w2 = (int(layer) << 16) | int(kv_head)
    ctr = np.stack([t & MASK32, ch >> np.uint64(2),
                    np.full(t.shape, w2, np.uint64),
                    np.full(t.shape, int(stream) & MASK32, np.uint64)], axis=-1)
    return ctr


def dither(seed: int, layer: int, kv_head: int, stream: int,
           tokens: np.ndarray, n_channels: int = 128) -> np.ndarray:
    """Dither xi in [-1/2, 1/2) as float32, shape (len(tokens), n_channels);
    the same for a token's keys and values."""
    if not (0 <= layer < 1 << 15 and 0 <= kv_head < 1 << 16):
        raise ValueError("dither: layer/kv_head out of range")
    tokens = np.asarray(tokens, dtype=np.int64)
    t = np.repeat(tokens, n_channels // 4)
    cg = np.tile(np.arange(0, n_channels, 4), len(tokens))
    ctr = dither_counters(t, cg, layer, kv_head, stream).reshape(-1, 4)
    out = philox4x32_10(ctr, (seed & MASK32, (seed >> 32) & MASK32))
    u = out.reshape(len(tokens), n_channels)      # word (c & 3) of group c >> 2
    xi = (u >> np.uint32(8)).astype(np.float64) * 2.0 ** -24 - 0.5
    return xi.astype(np.float32)                  # exact: 24-bit fraction
