"""Oracle computations the full-size GPU tests compose from the oracle's
primitives, pinned to the oracle's own forward on small bf16 models, each
with a planted mistake that must fail the same comparison:

* the layer-streamed forward behind the 80-layer verify test
  (test_gpu_zdepth.streamed_verify): the oracle's forward restated for
  several sequences at once and one layer of weights at a time (ragged
  positions after a random K / V context, three layers);
* the sampled-row and last-row pipelines of the full-size 70B-shaped prefill
  tests (test_gpu_fullsize)."""
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


# The sampled-row pipelines of the full-size 70B-shaped prefill tests
# (test_gpu_fullsize: layer0_kv, layer0_output, layer1_kv_at): layer 0's K / V
# on every row, layer 0's output and layer 1's K / V on sampled rows, and the
# last row's logits, against the oracle's forward over the whole prompt.

def _prefill_case(n_layers):
    from oracle.model import KVCache as _KV
    cfg = get_config("llama-8b-70b")
    sh = cfg.base.replace(n_layers=n_layers, d_model=256, n_q_heads=8, n_kv_heads=2, head_dim=32, d_ffn=512,
                          vocab=1000)
    om = OracleModel.from_torch(sh, make_weights(sh, 5, device="cpu"), np.float32)
    P = 300
    toks = np.random.default_rng(1).integers(0, sh.vocab, size=P)
    kv = _KV(sh, 1, P + 2, np.float32)
    z = forward(om, kv, 0, toks, range(P), logits="last")
    return om, toks, kv, z


def test_sampled_prefill_pipeline_equals_the_oracle_forward():
    from test_gpu_fullsize import layer0_kv, layer0_output, layer1_kv_at
    om, toks, kv, _ = _prefill_case(2)
    P = len(toks)
    rows = [0, 1, 15, 16, 100, 255, 298, 299]
    h0, qkv, K0, V0 = layer0_kv(om, toks)
    assert np.array_equal(kv.k[0, 0, :, :P], K0) and np.array_equal(kv.v[0, 0, :, :P], V0)
    K1, V1 = layer1_kv_at(om, layer0_output(om, h0, qkv, K0, V0, rows), rows)
    assert _rel(K1, kv.k[1, 0][:, rows]) < 1e-5 and _rel(V1, kv.v[1, 0][:, rows]) < 1e-5
    # planted: layer 0's attention one key short of causal
    shifted = layer0_output(om, h0, qkv, K0, V0, [max(r - 1, 0) for r in rows])
    _, V1b = layer1_kv_at(om, shifted, rows)
    assert _rel(V1b, kv.v[1, 0][:, rows]) > 1e-2


def test_last_row_pipeline_equals_the_oracle_forward():
    from oracle.model import final_logits
    from test_gpu_fullsize import layer0_kv, layer0_output
    om, toks, _, z = _prefill_case(1)
    P = len(toks)
    h0, qkv, K0, V0 = layer0_kv(om, toks)
    zo = final_logits(om, layer0_output(om, h0, qkv, K0, V0, [P - 1]))[0]
    assert _rel(zo, z) < 1e-5
    zb = final_logits(om, layer0_output(om, h0, qkv, K0, V0, [P - 2]))[0]
    assert _rel(zb, z) > 1e-2
