"""Seeded uniform-random prompts (token ids in [0, vocab))."""
from __future__ import annotations

import numpy as np


def make_prompts(vocab: int, length: int, batch: int, seed_of_b) -> np.ndarray:
    """Return int32 [batch][length]; row b drawn from Generator(Philox(seed_of_b(b)))."""
    out = np.empty((batch, length), dtype=np.int32)
    for b in range(batch):
        g = np.random.Generator(np.random.Philox(int(seed_of_b(b))))
        out[b] = g.integers(0, vocab, size=length, dtype=np.int64).astype(np.int32)
    return out
