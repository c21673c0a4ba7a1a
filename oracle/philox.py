"""Philox4x64-10 and the uniform streams the sampler draws from.

Philox4x64 is the counter-based generator of Salmon, Moraes, Dror and Shaw,
"Parallel Random Numbers: As Easy as 1, 2, 3" (SC'11): ten rounds, each of two
64x64->128-bit multiplications by fixed multipliers, an exchange of words and an
xor with the key; the key is bumped by two Weyl constants between rounds.
Written here with 32-bit limbs in NumPy uint64 arithmetic.

Stream layout (the build's reading; the pages specify no sampler):
  key     = (seed, sequence index b)
  counter = (v >> 2, position of the token being decided, 0, purpose)
  word    = v & 3 of the block; u = ((word >> 41) + 0.5) * 2**-23
          (an odd multiple of 2**-24, exactly representable in float32)
Purposes: DRAFT = 0 (draft-token sampling), ACCEPT = 1 (accept test, v = 0),
TARGET = 2 (residual / bonus sampling from the base distribution).
"""
from __future__ import annotations

import numpy as np

M0 = np.uint64(0xD2E7470EE14C6C93)
M1 = np.uint64(0xCA5A826395121157)
W0 = np.uint64(0x9E3779B97F4A7C15)
W1 = np.uint64(0xBB67AE8584CAA73B)

DRAFT = 0
ACCEPT = 1
TARGET = 2

_MASK32 = np.uint64(0xFFFFFFFF)
_S32 = np.uint64(32)


def mulhilo64(a, b):
    """Full 128-bit product of uint64 arrays -> (hi, lo)."""
    a = np.asarray(a, dtype=np.uint64)
    b = np.asarray(b, dtype=np.uint64)
    a_lo, a_hi = a & _MASK32, a >> _S32
    b_lo, b_hi = b & _MASK32, b >> _S32
    ll = a_lo * b_lo
    lh = a_lo * b_hi
    hl = a_hi * b_lo
    hh = a_hi * b_hi
    mid = (ll >> _S32) + (lh & _MASK32) + (hl & _MASK32)
    lo = (ll & _MASK32) | ((mid & _MASK32) << _S32)
    hi = hh + (lh >> _S32) + (hl >> _S32) + (mid >> _S32)
    return hi, lo


def philox4x64_10(ctr, key):
    """ctr: 4 uint64 arrays (broadcastable), key: 2 uint64 arrays -> 4 words."""
    with np.errstate(over="ignore"):
        c0, c1, c2, c3 = (np.asarray(c, dtype=np.uint64) for c in ctr)
        k0, k1 = (np.asarray(k, dtype=np.uint64) for k in key)
        for r in range(10):
            if r:
                k0 = k0 + W0
                k1 = k1 + W1
            hi0, lo0 = mulhilo64(M0, c0)
            hi1, lo1 = mulhilo64(M1, c2)
            c0, c1, c2, c3 = hi1 ^ c1 ^ k0, lo1, hi0 ^ c3 ^ k1, lo0
    return c0, c1, c2, c3


def words_to_uniform(w) -> np.ndarray:
    """Uniform in (0, 1) on the grid (2m + 1) * 2**-24, m < 2**23; exact in float32."""
    w = np.asarray(w, dtype=np.uint64)
    return ((w >> np.uint64(41)).astype(np.float64) + 0.5) * (2.0 ** -23)


def stream_uniforms(seed: int, b, pos, purpose: int, n: int) -> np.ndarray:
    """Uniforms u_v for v = 0..n-1 of stream (seed, b, pos, purpose).

    b and pos may be arrays of equal shape S; the result has shape S + (n,).
    """
    b = np.asarray(b, dtype=np.uint64)
    pos = np.asarray(pos, dtype=np.uint64)
    v = np.arange(n, dtype=np.uint64)
    shp = np.broadcast(b, pos).shape
    bb = np.broadcast_to(b, shp)[..., None]
    pp = np.broadcast_to(pos, shp)[..., None]
    blk = v >> np.uint64(2)
    words = philox4x64_10((blk, pp, np.uint64(0), np.uint64(purpose)),
                          (np.uint64(seed), bb))
    w = np.stack(np.broadcast_arrays(*words), axis=-1)          # S + (n, 4)
    sel = (v & np.uint64(3)).astype(np.int64)
    picked = np.take_along_axis(w, np.broadcast_to(sel[:, None], w.shape[:-1] + (1,)), -1)[..., 0]
    return words_to_uniform(picked)


def stream_uniform0(seed: int, b, pos, purpose: int) -> np.ndarray:
    """Word 0 of block 0 of the stream (the single accept-test uniform)."""
    return stream_uniforms(seed, b, pos, purpose, 1)[..., 0]
