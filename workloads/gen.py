"""Seeded generation of q, k, v for one layer of a workload.

Recipe (every tensor has its own seed, so any (layer, tensor, request) slice
can be regenerated alone):
  * q ~ N(0, 1) float32, [batch, h_q, d], rotated by RoPE at the query position
    (prefix length + the request's suffix length).
  * k ~ N(0, 1) float32 with fixed heavy channels, applied before RoPE:
      "outlier4x8":     4 channels (drawn once per workload) scaled by 8;
      "student_t3_8ch": 8 channels (drawn once per workload) replaced by
                        Student-t(3) samples z / sqrt(chi2_3 / 3).
    Keys are then rotated by RoPE at their positions (prefix 0..P-1, suffix
    P..P+n-1) when the workload uses RoPE, and rounded to bf16 (nearest even):
    the exact cache.  The float32 keys are also returned when a workload keeps
    an fp32 exact cache.
  * v ~ N(0, 1), rounded to bf16.
RoPE uses the rotate-half pairing (coordinate j with j + d/2) and frequencies
theta^(-2j/d); angles are formed in float64 on the host.
"""
from __future__ import annotations

import functools
from typing import Dict, Optional

import numpy as np
import torch

from .configs import Config

_T_Q, _T_KPRE, _T_VPRE, _T_KSUF, _T_VSUF = 1, 2, 3, 4, 5


def _seed(cfg: Config, layer: int, tensor: int, part: int) -> int:
    return (cfg.seed * 1_000_003 + layer * 7_919 + tensor * 104_729 + part * 15_485_863) % (2 ** 62)


def outlier_channels(cfg: Config) -> np.ndarray:
    n = 8 if cfg.key_dist == "student_t3_8ch" else 4
    return np.sort(np.random.default_rng(cfg.seed).choice(cfg.head_dim, n, replace=False))


@functools.lru_cache(maxsize=64)
def _rope_tables_cached(pos0: int, n: int, d: int, theta: float, device: str):
    cos, sin = _rope_tables(np.arange(pos0, pos0 + n), d, theta)
    return torch.from_numpy(cos).to(device), torch.from_numpy(sin).to(device)


def _rope_tables(positions: np.ndarray, d: int, theta: float):
    half = d // 2
    inv = theta ** (-np.arange(half, dtype=np.float64) * 2.0 / d)
    ang = positions.astype(np.float64)[:, None] * inv[None, :]
    return np.cos(ang).astype(np.float32), np.sin(ang).astype(np.float32)


def _apply_rope(x: torch.Tensor, cos: torch.Tensor, sin: torch.Tensor) -> torch.Tensor:
    half = x.shape[-1] // 2
    a, b = x[..., :half], x[..., half:]
    return torch.cat([a * cos - b * sin, a * sin + b * cos], dim=-1)


def _randn(shape, seed: int, device) -> torch.Tensor:
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    return torch.randn(shape, generator=g, device=device, dtype=torch.float32)


def _keys(cfg: Config, n_tok: int, pos0: int, seed: int, device, h_kv: int) -> torch.Tensor:
    d = cfg.head_dim
    k = _randn((h_kv, n_tok, d), seed, device)
    ch = torch.as_tensor(outlier_channels(cfg), device=device)
    if cfg.key_dist == "outlier4x8":
        k[..., ch] *= 8.0
    elif cfg.key_dist == "student_t3_8ch":
        z = _randn((h_kv, n_tok, len(ch), 4), seed ^ 0x5A5A5A5A, device)
        chi2 = (z[..., 1:] ** 2).sum(-1)
        k[..., ch] = z[..., 0] / torch.sqrt(chi2 / 3.0)
    else:
        raise ValueError(cfg.key_dist)
    if cfg.rope and n_tok > 0:
        cos, sin = _rope_tables_cached(pos0, n_tok, d, cfg.theta, str(device))
        k = _apply_rope(k, cos, sin)
    return k


def gen_layer(cfg: Config, layer: int, device="cpu", requests: Optional[list] = None,
              want_fp32_keys: bool = False) -> Dict[str, torch.Tensor]:
    """Inputs of one layer.  requests: subset of request indices (default all).

    Returns q [nb, h_q, d] f32; prefix_k / prefix_v [h_kv, P, d] bf16 (if the
    workload has a prefix); suffix_k / suffix_v [nb, h_kv, cap, d] bf16 with
    rows past each request's length zero; suffix_lens [nb] int32; and
    *_k32 float32 keys when want_fp32_keys.
    """
    d = cfg.head_dim
    reqs = list(range(cfg.batch)) if requests is None else list(requests)
    lens = cfg.lens()
    P = cfg.prefix.length if cfg.prefix else 0
    cap = cfg.suffix.length
    out: Dict[str, torch.Tensor] = {}
    if cfg.prefix is not None and P > 0:
        k32 = _keys(cfg, P, 0, _seed(cfg, layer, _T_KPRE, 0), device, cfg.h_kv)
        out["prefix_k"] = k32.to(torch.bfloat16)
        if want_fp32_keys:
            out["prefix_k32"] = k32
        out["prefix_v"] = _randn((cfg.h_kv, P, d), _seed(cfg, layer, _T_VPRE, 0), device).to(torch.bfloat16)
    qs, ks, vs, k32s = [], [], [], []
    for b in reqs:
        n = lens[b]
        q = _randn((cfg.h_q, d), _seed(cfg, layer, _T_Q, b), device)
        if cfg.rope:
            cos, sin = _rope_tables(np.array([P + n]), d, cfg.theta)
            q = _apply_rope(q, torch.from_numpy(cos).to(device), torch.from_numpy(sin).to(device))
        qs.append(q)
        k = torch.zeros((cfg.h_kv, cap, d), dtype=torch.float32, device=device)
        v = torch.zeros((cfg.h_kv, cap, d), dtype=torch.bfloat16, device=device)
        if n > 0:
            k[:, :n] = _keys(cfg, n, P, _seed(cfg, layer, _T_KSUF, b), device, cfg.h_kv)
            v[:, :n] = _randn((cfg.h_kv, n, d), _seed(cfg, layer, _T_VSUF, b), device).to(torch.bfloat16)
        ks.append(k.to(torch.bfloat16))
        if want_fp32_keys:
            k32s.append(k)
        vs.append(v)
        del k
    out["q"] = torch.stack(qs).contiguous()
    out["suffix_k"] = torch.stack(ks).contiguous()
    out["suffix_v"] = torch.stack(vs).contiguous()
    if want_fp32_keys:
        out["suffix_k32"] = torch.stack(k32s).contiguous()
    out["suffix_lens"] = torch.tensor([lens[b] for b in reqs], dtype=torch.int32, device=device)
    return out
