"""Shared helpers for tests: tiny model pairs built from the synth package."""
import numpy as np
import torch

from synth import make_weights, tiny_shape
from synth.configs import BF16, F32


def tiny_pair(V=64, dtype=F32, draft_layers=4, base_layers=3, d=32, hq=4, hkv=2, hd=8, ffn=64,
              seed=7, gain_std=0.1, bias=False, draft_noise=None):
    """A (draft, base) pair of tiny decoders sharing the vocabulary.

    draft_noise: if given, the draft is the base's weights plus N(0, noise)
    perturbations (same depth as the base), which gives high acceptance."""
    base_shape = tiny_shape(base_layers, d, hq, hkv, hd, ffn, V, dtype=dtype, qkv_bias=bias)
    bw = make_weights(base_shape, seed + 1, gain_std=gain_std, std=0.08)
    if draft_noise is None:
        draft_shape = tiny_shape(draft_layers, d, hq, hkv, hd, ffn, V, dtype=dtype, qkv_bias=bias)
        dw = make_weights(draft_shape, seed, gain_std=gain_std, std=0.08)
    else:
        draft_shape = base_shape
        g = torch.Generator().manual_seed(seed + 99)
        dw = {}
        for k_, t in bw.items():
            if t is None:
                dw[k_] = None
                continue
            n = torch.randn(t.shape, generator=g) * draft_noise
            dw[k_] = (t.float() + n).to(t.dtype)
    return draft_shape, dw, base_shape, bw
