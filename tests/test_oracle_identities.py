"""Pins of the oracle's fuzzy step, calibration and round loop against special
cases and invariants that the pages and the mathematics fix."""
import numpy as np
import pytest
import torch

from oracle import philox
from oracle.decode import spec_generate, vanilla_generate
from oracle.model import (KVCache, OracleModel, forward, fuzzy_step, fuzzy_step_hidden,
                          MLP_PARALLEL, MLP_SEQUENTIAL, rmsnorm)
from oracle.plan import default_group_plan
from synth import make_weights, tiny_shape
from synth.configs import BF16, F32
from helpers import tiny_pair


def _model(sh, seed, **kw):
    return OracleModel.from_torch(sh, make_weights(sh, seed, gain_std=0.1, std=0.08, **kw))


def _prefill(m, toks):
    c = KVCache(m.shape, 1, 64)
    forward(m, c, 0, toks, range(len(toks)), logits=None)
    return c


@pytest.mark.parametrize("dtype", [F32, BF16])
@pytest.mark.parametrize("mode", [MLP_SEQUENTIAL, MLP_PARALLEL])
def test_singleton_plan_equals_sequential(dtype, mode):
    # a plan of singletons breaks no dependency: the fuzzy step is the precise step
    sh = tiny_shape(5, 32, 4, 2, 8, 64, 40, dtype=dtype)
    m = _model(sh, 21)
    toks = [5, 9, 1, 33]
    c1, c2 = _prefill(m, toks), _prefill(m, toks)
    z1 = fuzzy_step(m, c1, 0, 17, 4, [[l] for l in range(5)], mode)
    z2 = forward(m, c2, 0, [17], [4])[0]
    np.testing.assert_array_equal(z1, z2)
    np.testing.assert_array_equal(c1.k, c2.k)


def test_fuzzy_set_differs_from_sequential():
    sh = tiny_shape(4, 32, 4, 2, 8, 64, 40)
    m = _model(sh, 22)
    c1, c2 = _prefill(m, [1, 2, 3]), _prefill(m, [1, 2, 3])
    z1 = fuzzy_step(m, c1, 0, 7, 3, [[0], [1, 2], [3]])
    z2 = forward(m, c2, 0, [7], [3])[0]
    assert np.max(np.abs(z1 - z2)) > 1e-4


@pytest.mark.parametrize("mode", [MLP_SEQUENTIAL, MLP_PARALLEL])
@pytest.mark.parametrize("live", [0, 1, 2])
def test_zero_residual_identity(mode, live):
    """If inside a set only one layer has non-zero W_o and W_down, that set
    computes exactly what the sequential layers compute (the dead layers add
    nothing to the residual stream), for either MLP reading."""
    L = 5
    sets = [[0], [1, 2, 3], [4]]
    dead = [l for l in (1, 2, 3) if l != 1 + live]
    sh = tiny_shape(L, 32, 4, 2, 8, 64, 40)
    w = make_weights(sh, 23, gain_std=0.1, std=0.08, zero_mask={"wo": dead, "w_down": dead})
    m = OracleModel.from_torch(sh, w)
    toks = [4, 8, 15, 16]
    c1, c2 = _prefill(m, toks), _prefill(m, toks)
    for step, tok in enumerate([23, 39, 7]):
        z1 = fuzzy_step(m, c1, 0, tok, 4 + step, sets, mode)
        z2 = forward(m, c2, 0, [tok], [4 + step])[0]
        np.testing.assert_array_equal(z1, z2)
    # the live layer's KV is identical; dead layers after the live one differ
    np.testing.assert_array_equal(c1.k[1 + live], c2.k[1 + live])


def test_parallel_and_sequential_mlp_readings_differ_only_for_sets():
    sh = tiny_shape(4, 32, 4, 2, 8, 64, 40)
    m = _model(sh, 24)
    sets = [[0], [1, 2], [3]]
    c1, c2 = _prefill(m, [1, 2]), _prefill(m, [1, 2])
    za = fuzzy_step(m, c1, 0, 5, 2, sets, MLP_SEQUENTIAL)
    zb = fuzzy_step(m, c2, 0, 5, 2, sets, MLP_PARALLEL)
    assert np.max(np.abs(za - zb)) > 1e-6
    # attention inputs of the set are h0 under both readings; later layers differ
    np.testing.assert_array_equal(c1.k[:3], c2.k[:3])


@pytest.mark.parametrize("dtype", [F32, BF16])
def test_calibration_restores_precise_kv(dtype):
    """After every calibration the draft KV for all committed positions equals
    a fresh sequential prefill of the committed tokens (fuzzy entries live for
    one speculation phase only)."""
    ds, dw, bs, bw = tiny_pair(V=32, dtype=dtype, draft_layers=5, draft_noise=None)
    d, b = OracleModel.from_torch(ds, dw), OracleModel.from_torch(bs, bw)
    prompt = [3, 1, 4, 1, 5, 9]
    sets = default_group_plan(5, 3)
    cap = 64
    dkv, bkv = KVCache(ds, 1, cap), KVCache(bs, 1, cap)

    toks, rounds = spec_generate(d, b, prompt, 3, sets, 12, 1.0, 5, caches=(dkv, bkv), capacity=cap)
    seq = prompt + toks
    # final state: every calibrated position (all but the tail of the last round)
    last_cal = len(prompt) + sum(r["a"] + 1 for r in rounds[:-1])
    ref = _prefill_model(d, seq[:last_cal], cap)
    np.testing.assert_allclose(dkv.k[:, :, :, :last_cal], ref.k[:, :, :, :last_cal], rtol=1e-9, atol=1e-12)
    np.testing.assert_allclose(dkv.v[:, :, :, :last_cal], ref.v[:, :, :, :last_cal], rtol=1e-9, atol=1e-12)
    # and the base KV is the precise prefix too (rejected positions are dead)
    upto = min(last_cal + rounds[-1]["a"], len(seq))   # the last round may be truncated
    bref = _prefill_model(b, seq[:upto], cap)
    np.testing.assert_allclose(bkv.k[:, :, :, :upto], bref.k[:, :, :, :upto], rtol=1e-9, atol=1e-12)


def _prefill_model(m, toks, cap):
    c = KVCache(m.shape, 1, cap)
    forward(m, c, 0, toks, range(len(toks)), logits=None)
    return c


@pytest.mark.parametrize("k,N", [(1, 2), (3, 1), (3, 2), (4, 3), (5, 4)])
def test_greedy_speculative_equals_vanilla(k, N):
    """Lossless: greedy speculative output equals greedy decoding of the base,
    for any plan, set size and draft length."""
    ds, dw, bs, bw = tiny_pair(V=24, base_layers=5, draft_noise=0.01)
    d, b = OracleModel.from_torch(ds, dw), OracleModel.from_torch(bs, bw)
    prompt = [2, 7, 1, 8, 2, 8]
    sets = default_group_plan(5, N)
    spec, rounds = spec_generate(d, b, prompt, k, sets, 20, 0.0, 0)
    van = vanilla_generate(b, prompt, 20, 0.0, 0)
    assert spec == van
    assert len(spec) == 20
    # the draft is a near copy of the base: acceptance must be exercised
    assert sum(r["a"] for r in rounds) > 0


@pytest.mark.parametrize("k,N", [(1, 2), (3, 2), (4, 3), (5, 4)])
def test_greedy_speculative_equals_vanilla_separate_calibration(k, N):
    """The separate-pass reading of the calibration (all k drafts from fuzzy
    steps, the committed fuzzy tokens rewritten afterwards) changes only the
    drafts, so greedy output is still the base's greedy output."""
    ds, dw, bs, bw = tiny_pair(V=24, base_layers=5, draft_noise=0.01)
    d, b = OracleModel.from_torch(ds, dw), OracleModel.from_torch(bs, bw)
    prompt = [2, 7, 1, 8, 2, 8]
    sets = default_group_plan(5, N)
    spec, rounds = spec_generate(d, b, prompt, k, sets, 20, 0.0, 0, separate=True)
    assert spec == vanilla_generate(b, prompt, 20, 0.0, 0)
    assert sum(r["a"] for r in rounds) > 0


@pytest.mark.parametrize("dtype", [F32, BF16])
def test_separate_calibration_restores_precise_kv(dtype):
    """Separate-pass reading: the draft prefills P-1 tokens, and each
    calibration rewrites [x_t, d_1..d_a] at t..t+a, so after the last one the
    draft KV up to the pending position equals a sequential prefill."""
    ds, dw, bs, bw = tiny_pair(V=32, dtype=dtype, draft_layers=5, draft_noise=None)
    d, b = OracleModel.from_torch(ds, dw), OracleModel.from_torch(bs, bw)
    prompt = [3, 1, 4, 1, 5, 9]
    sets = default_group_plan(5, 3)
    cap = 64
    dkv, bkv = KVCache(ds, 1, cap), KVCache(bs, 1, cap)
    toks, rounds = spec_generate(d, b, prompt, 3, sets, 12, 1.0, 5, caches=(dkv, bkv), capacity=cap,
                                 separate=True)
    assert len(rounds) > 1
    seq = prompt + toks
    last_cal = len(prompt) - 1 + sum(r["a"] + 1 for r in rounds[:-1])
    assert last_cal == rounds[-1]["t"]
    ref = _prefill_model(d, seq[:last_cal], cap)
    np.testing.assert_allclose(dkv.k[:, :, :, :last_cal], ref.k[:, :, :, :last_cal], rtol=1e-9, atol=1e-12)
    np.testing.assert_allclose(dkv.v[:, :, :, :last_cal], ref.v[:, :, :, :last_cal], rtol=1e-9, atol=1e-12)
    # the pending token's own entry is fuzzy (a set member's attention input
    # is the set's input, not the running state): it differs from the prefill
    ref2 = _prefill_model(d, seq[:last_cal + 1], cap)
    assert not np.allclose(dkv.k[:, :, :, last_cal], ref2.k[:, :, :, last_cal], rtol=1e-6, atol=1e-9)


@pytest.mark.parametrize("inv_temp", [0.0, 1.0])
def test_self_draft_accepts_everything(inv_temp):
    """Draft identical to the base and a sequential plan: p = q at every step, so
    every draft is accepted (u * q < p holds for every u < 1)."""
    _, _, bs, bw = tiny_pair(V=24, base_layers=3)
    b = OracleModel.from_torch(bs, bw)
    prompt = [1, 2, 3, 4]
    spec, rounds = spec_generate(b, b, prompt, 4, [[0], [1], [2]], 15, inv_temp, 9)
    assert all(r["a"] == 4 for r in rounds)
    if inv_temp == 0.0:
        assert spec == vanilla_generate(b, prompt, 15, 0.0, 9)
    # with a layer-parallel set the fuzzy draft is no longer exact
    _, rounds2 = spec_generate(b, b, prompt, 4, [[0, 1], [2]], 15, inv_temp, 9)
    assert np.max(np.abs(rounds2[0]["q_logits"][1:] - rounds2[0]["p_logits"][1:4])) > 1e-6


def test_sampled_spec_is_deterministic_and_seeded():
    ds, dw, bs, bw = tiny_pair(V=24, base_layers=3, draft_noise=0.05)
    d, b = OracleModel.from_torch(ds, dw), OracleModel.from_torch(bs, bw)
    sets = default_group_plan(3, 2)
    a1, _ = spec_generate(d, b, [1, 2, 3], 3, sets, 10, 1.0, 42)
    a2, _ = spec_generate(d, b, [1, 2, 3], 3, sets, 10, 1.0, 42)
    a3, _ = spec_generate(d, b, [1, 2, 3], 3, sets, 10, 1.0, 43)
    assert a1 == a2 and a1 != a3


def test_cosine_similarity_invariant_under_entry_norm():
    """Rebuttal reply on Table 3: with a normalisation at the attention entry,
    cos(h1, h2) = cos(h1', h2').  True for a uniform gain; in general false for
    a non-uniform gain (the assumption behind the statement)."""
    rng = np.random.default_rng(8)
    h1, h2 = rng.normal(size=64), rng.normal(size=64) + 0.5
    cos = lambda a, b: a @ b / np.linalg.norm(a) / np.linalg.norm(b)
    g = np.full(64, 1.7)
    assert abs(cos(h1, h2) - cos(rmsnorm(h1, g, 1e-6), rmsnorm(h2, g, 1e-6))) < 1e-12
    g2 = rng.uniform(0.2, 3.0, size=64)
    assert abs(cos(h1, h2) - cos(rmsnorm(h1, g2, 1e-6), rmsnorm(h2, g2, 1e-6))) > 1e-3
