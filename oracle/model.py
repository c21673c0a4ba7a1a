"""Decoder forward passes: the precise sequential forward and the fuzzy
layer-parallel draft step.

Model definition (the pages give none; the configurations are Llama- and
Qwen-shaped pre-norm decoders):
  h   = E[token]
  per layer l:  x = RMSNorm(h; g1_l);  [q; k; v] = W_qkv,l x (+ b_qkv,l)
                RoPE (rotate-half, pairs (j, j + hd/2), angle pos * theta^(-2j/hd))
                on q and k; k, v appended to layer l's KV cache at pos;
                o = softmax(q K^T / sqrt(hd)) V over cached positions <= pos
                (GQA: q head h reads kv head floor(h * hkv / hq));
                h = h + W_o,l o
                y = RMSNorm(h; g2_l);  h = h + W_down,l (SiLU(W_gate,l y) * (W_up,l y))
  logits = W_lm RMSNorm(h; g_f)
RMSNorm(x; g) = g * x / sqrt(mean(x^2) + eps).

Layer-parallel ("fuzzy") set, from the EasySpec abstract (inter-layer data
dependencies in the draft are broken so that layers run simultaneously) and the
rebuttal (only attention is layer-parallel and takes the same input; the MLPs
still run one after another; the fuzzy attentions produce a set of KV entries):
every attention of a set reads the set's incoming hidden state h0 and writes
its own layer's KV.  How the attention outputs re-enter the residual stream is
not stated; reading (A), the default: h = h0; for each layer i of the set in
order: h = h + a_i; h = h + MLP_i(h).  The "parallel MLP" variant: h = h0 +
sum_i (a_i + MLP_i(h0 + a_i)).  Both equal the sequential layer for a set of
size 1.

bf16 path: weights and the KV cache hold bfloat16 values (the weights are
given as such; K and V are rounded to bfloat16 when they are written, see
oracle.numerics); every activation is float64 here.
"""
from __future__ import annotations

from dataclasses import dataclass
from typing import Dict, List, Optional

import numpy as np

from .numerics import round_bf16

MLP_SEQUENTIAL = 0
MLP_PARALLEL = 1


def to_numpy_weights(w: dict, ftype=np.float64) -> Dict[str, Optional[np.ndarray]]:
    """Convert a dict of torch tensors (any float dtype) to float arrays."""
    out = {}
    for k, t in w.items():
        out[k] = None if t is None else t.detach().to("cpu").float().numpy().astype(ftype, copy=False)
    return out


@dataclass
class OracleModel:
    shape: object                 # synth.ModelShape
    w: Dict[str, Optional[np.ndarray]]
    bf16: bool

    @classmethod
    def from_torch(cls, shape, weights, ftype=np.float64):
        return cls(shape, to_numpy_weights(weights, ftype), shape.dtype == 1)

    def rnd(self, x):
        return round_bf16(x) if self.bf16 else x


class KVCache:
    """K and V as [L][B][hkv][capacity][hd] arrays (float64, or float32)."""

    def __init__(self, shape, batch: int, capacity: int, ftype=np.float64):
        dims = (shape.n_layers, batch, shape.n_kv_heads, capacity, shape.head_dim)
        self.k = np.zeros(dims, dtype=ftype)
        self.v = np.zeros(dims, dtype=ftype)
        self.capacity = capacity

    def copy(self):
        c = KVCache.__new__(KVCache)
        c.k, c.v, c.capacity = self.k.copy(), self.v.copy(), self.capacity
        return c


# ----------------------------------------------------------------- primitives
def linear(x, W):
    """x W^T for x [n][in], W [out][in] (computed as (W x^T)^T so that NumPy
    hands the row-major weight to BLAS as is).  The product is formed in the
    weights' precision: float64 for the default float64 model; float32 for a
    model whose weights are held as float32 (workload-size models whose
    float64 copy would not fit), whose residual stream stays float64."""
    if W.dtype == np.float32 and x.dtype != np.float32:
        x = x.astype(np.float32)
    return (W @ x.T).T


def rmsnorm(x, g, eps):
    ms = np.mean(x * x, axis=-1, keepdims=True)
    return x / np.sqrt(ms + eps) * g


def silu(x):
    return x / (1.0 + np.exp(-x))


def rope(x, positions, theta):
    """x: [n][heads][hd]; rotate-half pairs (j, j + hd/2)."""
    hd = x.shape[-1]
    half = hd // 2
    j = np.arange(half, dtype=np.float64)
    inv_freq = theta ** (-2.0 * j / hd)
    ang = np.asarray(positions, dtype=np.float64)[:, None] * inv_freq[None, :]
    c = np.cos(ang)[:, None, :]
    s = np.sin(ang)[:, None, :]
    x1, x2 = x[..., :half], x[..., half:]
    return np.concatenate([x1 * c - x2 * s, x2 * c + x1 * s], axis=-1)


def attention(q, K, V, positions, n_kv):
    """q [n][hq][hd]; K, V [hkv][cap][hd]; row r attends to keys 0..positions[r]."""
    n, hq, hd = q.shape
    grp = hq // n_kv
    out = np.zeros_like(q)
    scale = 1.0 / np.sqrt(hd)
    for r in range(n):
        p = int(positions[r])
        for h in range(hq):
            kv = h // grp
            s = K[kv, :p + 1] @ q[r, h] * scale
            s = np.exp(s - s.max())
            s /= s.sum()
            out[r, h] = s @ V[kv, :p + 1]
    return out


# ------------------------------------------------------------- layer pieces
def attn_part(m: OracleModel, cache: KVCache, l: int, b: int, h_in, positions):
    """Attention sub-block of layer l on inputs h_in [n][d] at `positions`.

    Writes k, v of layer l into the cache at the positions and returns W_o o.
    """
    sh, w = m.shape, m.w
    hq, hkv, hd = sh.n_q_heads, sh.n_kv_heads, sh.head_dim
    x = rmsnorm(h_in, w["attn_norm"][l], sh.rms_eps)
    qkv = linear(x, w["wqkv"][l])
    if w.get("bqkv") is not None:
        qkv = qkv + w["bqkv"][l]
    n = h_in.shape[0]
    q = qkv[:, :hq * hd].reshape(n, hq, hd)
    k = qkv[:, hq * hd:(hq + hkv) * hd].reshape(n, hkv, hd)
    v = qkv[:, (hq + hkv) * hd:].reshape(n, hkv, hd)
    q = rope(q, positions, sh.rope_theta)
    k = rope(k, positions, sh.rope_theta)
    for r, p in enumerate(positions):
        cache.k[l, b, :, p] = m.rnd(k[r])
        cache.v[l, b, :, p] = m.rnd(v[r])
    o = attention(q, cache.k[l, b], cache.v[l, b], positions, hkv)
    o = o.reshape(n, hq * hd)
    return linear(o, w["wo"][l])


def mlp_part(m: OracleModel, l: int, h_in):
    sh, w = m.shape, m.w
    f = sh.d_ffn
    y = rmsnorm(h_in, w["ffn_norm"][l], sh.rms_eps)
    gu = linear(y, w["w_gate_up"][l])
    act = silu(gu[:, :f]) * gu[:, f:]
    return linear(act, w["w_down"][l])


def embed(m: OracleModel, tokens):
    return m.w["embed"][np.asarray(tokens, dtype=np.int64)].copy()


def final_logits(m: OracleModel, h):
    x = rmsnorm(h, m.w["final_norm"], m.shape.rms_eps)
    return linear(x, m.w["lm_head"])


# ----------------------------------------------------------------- forwards
def forward_hidden(m: OracleModel, cache: KVCache, b: int, tokens, positions):
    """Precise (sequential) forward of sequence b over new tokens at
    `positions` (consecutive, causal among themselves).  Writes every layer's
    KV at those positions and returns the final hidden states [n][d]."""
    positions = [int(p) for p in positions]
    h = embed(m, tokens)
    for l in range(m.shape.n_layers):
        h = h + attn_part(m, cache, l, b, h, positions)
        h = h + mlp_part(m, l, h)
    return h


def forward(m: OracleModel, cache: KVCache, b: int, tokens, positions, logits="all"):
    """Precise forward; logits: 'all' -> [n][V], 'last' -> [V], None -> None.

    This is the base model's verify pass (k+1 tokens) and prompt prefill, and
    the draft model's bonus calibration (EasySpec abstract: the draft KV cache
    is calibrated in a single forward pass after each draft-and-verify
    iteration)."""
    h = forward_hidden(m, cache, b, tokens, positions)
    if logits is None:
        return None
    if logits == "last":
        return final_logits(m, h[-1:])[0]
    return final_logits(m, h)


def fuzzy_step_hidden(m: OracleModel, cache: KVCache, b: int, token: int, pos: int,
                      sets: List[List[int]], mlp_mode: int = MLP_SEQUENTIAL,
                      trace: Optional[list] = None):
    """One layer-parallel draft step for one token of sequence b at `pos`.

    `sets` is the plan (contiguous layer sets covering all layers).  Returns
    the final hidden state [1][d].  If `trace` is a list, the attention input
    actually used by each layer and the precise input it stands in for are
    appended (for the cosine-similarity diagnostic)."""
    positions = [int(pos)]
    h = embed(m, [token])
    for s in sets:
        h0 = h
        a = [attn_part(m, cache, l, b, h0, positions) for l in s]
        if mlp_mode == MLP_SEQUENTIAL:
            h = h0
            for i, l in enumerate(s):
                if trace is not None:
                    trace.append((l, h0.copy(), h.copy()))
                h = h + a[i]
                h = h + mlp_part(m, l, h)
        elif mlp_mode == MLP_PARALLEL:
            acc = h0.copy()
            for i, l in enumerate(s):
                acc = acc + a[i]
                acc = acc + mlp_part(m, l, h0 + a[i])
            h = acc
        else:
            raise ValueError("unknown mlp mode")
    return h


def fuzzy_step(m, cache, b, token, pos, sets, mlp_mode=MLP_SEQUENTIAL):
    return final_logits(m, fuzzy_step_hidden(m, cache, b, token, pos, sets, mlp_mode))[0]
