"""The layer-streamed forward behind the 80-layer verify test
(test_gpu_zdepth.streamed_verify) is the oracle's forward restated for
several sequences at once and one layer of weights at a time.  Pinned here
to the oracle's own forward on a small bf16 model (ragged positions after a
random K / V context, three layers), with a planted one-position shift that
must fail the same comparison."""
import numpy as np
import torch

from oracle.model import KVCache, OracleModel, forward
from synth import get_config, make_weights
from test_gpu_zdepth import streamed_verify


def _case():
    cfg = get_config("llama-8b-70b")
    sh = cfg.base.replace(n_layers=3, d_model=256, n_q_heads=8, n_kv_heads=2, head_dim=32, d_ffn=512, vocab=1000)
    w = make_weights(sh, 9, device="cpu")
    B, m, ctx, cap = 3, 7, 200, 210
    g = torch.Generator().manual_seed(3)
    K = torch.randn(sh.n_layers, B, sh.n_kv_heads, cap, sh.head_dim, generator=g).to(torch.bfloat16)
    V = torch.randn(sh.n_layers, B, sh.n_kv_heads, cap, sh.head_dim, generator=g).to(torch.bfloat16)
    K[:, :, :, ctx:] = 0
    V[:, :, :, ctx:] = 0
    toks = np.random.default_rng(4).integers(0, sh.vocab, size=(B, m)).astype(np.int32)
    pos = ctx - 1 - np.arange(B) * 3
    return sh, w, K, V, toks, pos


def _oracle(sh, w, K, V, toks, pos):
    om = OracleModel.from_torch(sh, w, np.float32)
    kv = KVCache.__new__(KVCache)
    kv.k, kv.v, kv.capacity = K.float().numpy().copy(), V.float().numpy().copy(), K.shape[3]
    m = toks.shape[1]
    return [forward(om, kv, b, toks[b], range(int(pos[b]), int(pos[b]) + m), logits="all")
            for b in range(toks.shape[0])]


def _rel(a, b):
    return float(np.max(np.abs(a - b)) / np.max(np.abs(b)))


def test_streamed_verify_equals_the_oracle_forward():
    sh, w, K, V, toks, pos = _case()
    z = streamed_verify(sh, w, (K.clone(), V.clone()), toks, pos)
    zo = _oracle(sh, w, K, V, toks, pos)
    for b in range(toks.shape[0]):
        assert _rel(z[b], zo[b]) < 1e-4, (b, _rel(z[b], zo[b]))


def test_streamed_verify_planted_position_shift_fails():
    sh, w, K, V, toks, pos = _case()
    z = streamed_verify(sh, w, (K.clone(), V.clone()), toks, pos + 1)
    zo = _oracle(sh, w, K, V, toks, pos)
    assert max(_rel(z[b], zo[b]) for b in range(toks.shape[0])) > 1e-2
