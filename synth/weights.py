"""Seeded random-init decoder weights, laid out as layer-major arenas.

Every matrix is i.i.d. N(0, std) (std 0.02 by default) and is stored in the
model's weight dtype (bfloat16 or float32).  Norm gains are 1 unless
``gain_std`` asks for jitter (tests use jitter so that a wrong gain index
shows up).  Generation is deterministic for a given (seed, device): each
tensor, and for arenas each layer slice, has its own torch generator seed.

Arena layouts (row-major):
  embed      [V][d]
  attn_norm  [L][d]              float32
  wqkv       [L][(hq+2hkv)*hd][d]   rows: q heads, then k heads, then v heads
  bqkv       [L][(hq+2hkv)*hd]   float32, or None
  wo         [L][d][hq*hd]
  ffn_norm   [L][d]              float32
  w_gate_up  [L][2*ffn][d]       rows: gate, then up
  w_down     [L][d][ffn]
  final_norm [d]                 float32
  lm_head    [V][d]
"""
from __future__ import annotations

import torch

from .configs import ModelShape, BF16

WEIGHT_KEYS = ("embed", "attn_norm", "wqkv", "bqkv", "wo", "ffn_norm",
               "w_gate_up", "w_down", "final_norm", "lm_head")

_TID = {k: i for i, k in enumerate(WEIGHT_KEYS)}


def _gen(seed: int, device) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(int(seed) & 0x7FFFFFFFFFFFFFFF)
    return g


def _normal(shape, seed, std, dtype, device):
    g = _gen(seed, device)
    t = torch.randn(shape, generator=g, device=device, dtype=torch.float32)
    t.mul_(std)
    return t.to(dtype)


def make_weights(shape: ModelShape, seed: int, device="cpu", std: float = 0.02,
                 gain_std: float = 0.0, bias_std: float = 0.02,
                 zero_mask=None) -> dict:
    """Build the weight arenas for ``shape``.

    zero_mask: optional dict {key: iterable of layer indices} whose slices are
    zeroed (used by tests that build special-case models).
    """
    wdt = torch.bfloat16 if shape.dtype == BF16 else torch.float32
    L, d, V = shape.n_layers, shape.d_model, shape.vocab
    base = int(seed) * 1_000_003

    def s(key, layer=0):
        return base + 7919 * _TID[key] + 104729 * (layer + 1)

    def arena(key, rows, cols, dtype=wdt, sd=std):
        out = torch.empty((L, rows, cols) if cols else (L, rows), dtype=dtype, device=device)
        for l in range(L):
            sh = (rows, cols) if cols else (rows,)
            out[l] = _normal(sh, s(key, l), sd, dtype, device)
        return out

    def gains(key, n):
        if gain_std == 0.0:
            return torch.ones(n, d, dtype=torch.float32, device=device)
        return 1.0 + _normal((n, d), s(key), gain_std, torch.float32, device)

    w = {}
    w["embed"] = _normal((V, d), s("embed"), std, wdt, device)
    w["attn_norm"] = gains("attn_norm", L)
    w["wqkv"] = arena("wqkv", shape.qkv_rows, d)
    w["bqkv"] = (arena("bqkv", shape.qkv_rows, 0, torch.float32, bias_std)
                 if shape.qkv_bias else None)
    w["wo"] = arena("wo", d, shape.q_dim)
    w["ffn_norm"] = gains("ffn_norm", L)
    w["w_gate_up"] = arena("w_gate_up", 2 * shape.d_ffn, d)
    w["w_down"] = arena("w_down", d, shape.d_ffn)
    w["final_norm"] = gains("final_norm", 1)[0].contiguous()
    w["lm_head"] = _normal((V, d), s("lm_head"), std, wdt, device)
    if zero_mask:
        for key, layers in zero_mask.items():
            for l in layers:
                w[key][l].zero_()
    return w
