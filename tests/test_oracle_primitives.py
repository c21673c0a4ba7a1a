"""Pins for the oracle's layer primitives against library routines and
closed-form properties."""
import numpy as np
import pytest
import torch
import torch.nn.functional as F

from oracle import model as om
from oracle.numerics import round_bf16, bf16_bits_to_f64
from oracle.model import KVCache, OracleModel, forward
from synth import make_weights, tiny_shape
from synth.configs import BF16, F32


def test_rmsnorm_matches_torch():
    rng = np.random.default_rng(0)
    x = rng.normal(size=(5, 48)) * 3
    g = rng.normal(size=48)
    ref = F.rms_norm(torch.from_numpy(x), (48,), torch.from_numpy(g), eps=1e-5).numpy()
    np.testing.assert_allclose(om.rmsnorm(x, g, 1e-5), ref, rtol=1e-12, atol=1e-12)


def test_silu_matches_torch():
    x = np.linspace(-30, 30, 1001)
    np.testing.assert_allclose(om.silu(x), F.silu(torch.from_numpy(x)).numpy(), rtol=1e-12, atol=1e-15)


@pytest.mark.parametrize("hq,hkv", [(4, 4), (8, 2), (6, 1)])
def test_attention_matches_torch_sdpa_causal_gqa(hq, hkv):
    rng = np.random.default_rng(hq * 10 + hkv)
    n, hd = 7, 16
    q = rng.normal(size=(n, hq, hd))
    K = rng.normal(size=(hkv, n, hd))
    V = rng.normal(size=(hkv, n, hd))
    out = om.attention(q, K, V, list(range(n)), hkv)
    tq = torch.from_numpy(q).permute(1, 0, 2)[None]                 # [1][hq][n][hd]
    tk = torch.from_numpy(K).repeat_interleave(hq // hkv, 0)[None]
    tv = torch.from_numpy(V).repeat_interleave(hq // hkv, 0)[None]
    ref = F.scaled_dot_product_attention(tq, tk, tv, is_causal=True)[0].permute(1, 0, 2).numpy()
    np.testing.assert_allclose(out, ref, rtol=1e-10, atol=1e-12)


def test_attention_offset_rows_are_causal_suffix():
    # rows at positions 3..5 against a cache of 6 keys == last 3 rows of the full causal result
    rng = np.random.default_rng(3)
    q = rng.normal(size=(6, 4, 8))
    K = rng.normal(size=(2, 6, 8))
    V = rng.normal(size=(2, 6, 8))
    full = om.attention(q, K, V, list(range(6)), 2)
    part = om.attention(q[3:], K, V, [3, 4, 5], 2)
    np.testing.assert_allclose(part, full[3:], rtol=1e-13)


def test_rope_relative_position_property():
    # <R(m) q, R(n) k> depends only on m - n
    rng = np.random.default_rng(4)
    q = rng.normal(size=(1, 1, 32))
    k = rng.normal(size=(1, 1, 32))
    def dot(m, n):
        return float(np.sum(om.rope(q, [m], 10000.0) * om.rope(k, [n], 10000.0)))
    for (m, n), (m2, n2) in [((5, 2), (103, 100)), ((0, 9), (41, 50)), ((7, 7), (1000, 1000))]:
        assert abs(dot(m, n) - dot(m2, n2)) < 1e-9
    assert abs(dot(5, 2) - dot(2, 5)) > 1e-6          # not symmetric in general
    # position 0 is the identity, and the rotation preserves norms
    np.testing.assert_allclose(om.rope(q, [0], 10000.0), q, rtol=0, atol=0)
    np.testing.assert_allclose(np.linalg.norm(om.rope(q, [12345], 5e5)), np.linalg.norm(q), rtol=1e-12)


def test_rope_pairs_rotate_half():
    # the pair (j, j + hd/2) rotates by pos * theta^(-2j/hd): check one pair by hand
    x = np.zeros((1, 1, 8))
    x[0, 0, 1] = 1.0                      # j = 1, partner index 5
    out = om.rope(x, [3], 100.0)
    ang = 3 * 100.0 ** (-2.0 / 8)
    assert abs(out[0, 0, 1] - np.cos(ang)) < 1e-14
    assert abs(out[0, 0, 5] - np.sin(ang)) < 1e-14
    assert np.count_nonzero(np.abs(out) > 1e-15) == 2


def test_bf16_rounding_matches_torch():
    rng = np.random.default_rng(5)
    x = np.concatenate([rng.normal(size=100000) * 10.0 ** rng.integers(-8, 8, size=100000),
                        np.array([0.0, -0.0, 1.0, 1.00390625, 1.01171875, 3.0e38])])
    ref = torch.from_numpy(x.astype(np.float32)).to(torch.bfloat16).float().numpy().astype(np.float64)
    np.testing.assert_array_equal(round_bf16(x), ref)
    bits = torch.from_numpy(x.astype(np.float32)).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    np.testing.assert_array_equal(bf16_bits_to_f64(bits), ref)


@pytest.mark.parametrize("dtype", [F32, BF16])
def test_incremental_decode_equals_full_forward(dtype):
    sh = tiny_shape(3, 32, 4, 2, 8, 64, 50, dtype=dtype, qkv_bias=True)
    m = OracleModel.from_torch(sh, make_weights(sh, 11, gain_std=0.1, std=0.08))
    toks = [3, 14, 15, 9, 2, 6, 5, 35]
    c1 = KVCache(sh, 1, 16)
    full = forward(m, c1, 0, toks, range(8))
    c2 = KVCache(sh, 1, 16)
    forward(m, c2, 0, toks[:3], range(3))
    z = [forward(m, c2, 0, [toks[i]], [i])[0] for i in range(3, 8)]
    np.testing.assert_allclose(np.stack(z), full[3:], rtol=1e-9, atol=1e-11)
    np.testing.assert_allclose(c1.k[:, :, :, :8], c2.k[:, :, :, :8], rtol=1e-9, atol=1e-11)


def test_forward_matches_torch_reference_decoder():
    """An independent torch float64 statement of the same decoder (layer by
    layer with torch's own rms_norm / SDPA / silu) gives the same logits."""
    sh = tiny_shape(2, 32, 4, 2, 8, 64, 40, qkv_bias=True)
    w = make_weights(sh, 13, gain_std=0.1, std=0.08)
    m = OracleModel.from_torch(sh, w)
    toks = [1, 7, 3, 39, 0, 12]
    n = len(toks)
    ours = forward(m, KVCache(sh, 1, 8), 0, toks, range(n))
    W = {k: (None if v is None else v.double()) for k, v in w.items()}
    hq, hkv, hd, d = 4, 2, 8, 32
    h = W["embed"][torch.tensor(toks)]
    pos = torch.arange(n, dtype=torch.float64)
    inv = sh.rope_theta ** (-torch.arange(0, hd, 2, dtype=torch.float64) / hd)
    ang = pos[:, None] * inv[None]
    cos = torch.cat([ang.cos(), ang.cos()], -1)[:, None]
    sin = torch.cat([ang.sin(), ang.sin()], -1)[:, None]

    def rot(x):
        x1, x2 = x[..., :hd // 2], x[..., hd // 2:]
        return x * cos + torch.cat([-x2, x1], -1) * sin
    for l in range(2):
        x = F.rms_norm(h, (d,), W["attn_norm"][l], eps=sh.rms_eps)
        qkv = x @ W["wqkv"][l].T + W["bqkv"][l]
        q = rot(qkv[:, :hq * hd].view(n, hq, hd))
        k = rot(qkv[:, hq * hd:(hq + hkv) * hd].view(n, hkv, hd))
        v = qkv[:, (hq + hkv) * hd:].view(n, hkv, hd)
        o = F.scaled_dot_product_attention(q.transpose(0, 1)[None],
                                           k.transpose(0, 1).repeat_interleave(2, 0)[None],
                                           v.transpose(0, 1).repeat_interleave(2, 0)[None],
                                           is_causal=True)[0].transpose(0, 1).reshape(n, hq * hd)
        h = h + o @ W["wo"][l].T
        y = F.rms_norm(h, (d,), W["ffn_norm"][l], eps=sh.rms_eps)
        gu = y @ W["w_gate_up"][l].T
        h = h + (F.silu(gu[:, :64]) * gu[:, 64:]) @ W["w_down"][l].T
    ref = F.rms_norm(h, (d,), W["final_norm"], eps=sh.rms_eps) @ W["lm_head"].T
    np.testing.assert_allclose(ours, ref.numpy(), rtol=1e-10, atol=1e-12)
