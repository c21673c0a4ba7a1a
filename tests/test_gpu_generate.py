"""End-to-end GPU speculative decoding against the oracle in lock step, and
the lossless greedy property on the GPU."""
import numpy as np
import pytest
import torch

from oracle.model import MLP_PARALLEL, MLP_SEQUENTIAL, OracleModel
from oracle.plan import default_group_plan, offsets_to_sets, plan_offsets
from synth import get_config, make_prompts, make_weights, tiny_shape
from synth.configs import BF16
from gpu_common import TOL_BF16, TOL_F32, exclusion, say, to_dev
from lockstep import lockstep

pytestmark = pytest.mark.gpu


def _pair(cfg, draft_noise=None):
    dw = make_weights(cfg.draft, cfg.seed_draft)
    bw = make_weights(cfg.base, cfg.seed_base)
    return dw, bw


@pytest.mark.parametrize("inv_temp", [0.0, 1.0])
@pytest.mark.parametrize("plan_kind", ["paper", "explicit"])
def test_tiny_config_lockstep(inv_temp, plan_kind):
    from layer_speculative_decoding_amd.runtime import SpecDecoder
    cfg = get_config("tiny")
    say(f"lockstep tiny invT={inv_temp} plan={plan_kind}")
    dw, bw = _pair(cfg)
    sets = default_group_plan(cfg.draft.n_layers, cfg.group_size) if plan_kind == "paper" else [[0, 1]]
    prompts = make_prompts(cfg.draft.vocab, cfg.prompt_len, cfg.batch, cfg.prompt_seed)
    dec = SpecDecoder(cfg.draft, to_dev(dw), cfg.base, to_dev(bw), cfg.batch, cfg.capacity, cfg.k,
                      plan_offsets(sets), cfg.prompt_len, inv_temp, cfg.sample_seed)
    st = lockstep(dec, OracleModel.from_torch(cfg.draft, dw), OracleModel.from_torch(cfg.base, bw), prompts,
                  cfg.k, sets, cfg.new_tokens, dec.inv_temp, cfg.sample_seed, MLP_SEQUENTIAL, TOL_F32)
    say(f"  checked {st['checked']} flipped {st['flipped']} excluded {st['excluded']} max rel err {st['err']:.2e}; "
        f"rounds {len(dec.records)} accepted {sum(int(r.n_acc[0]) for r in dec.records)}")
    assert st["excluded"] + st["flipped"] <= max(2, st["checked"] // 50)


# the near-copy pairs' 4-layer plan with a real layer-parallel set (the default
# grouping of 4 layers in sets of 2 has only singletons)
FUZZY4 = [[0], [1, 2], [3]]


def _near_copy_pair(dtype, V=512, L=4, seed=3, noise=0.004):
    sh = tiny_shape(L, 128, 8, 2, 16, 384, V, dtype=dtype, qkv_bias=True)
    bw = make_weights(sh, seed, gain_std=0.1, std=0.05)
    g = torch.Generator().manual_seed(seed + 1)
    dw = {k: (None if v is None else (v.float() + noise * torch.randn(v.shape, generator=g)).to(v.dtype))
          for k, v in bw.items()}
    return sh, dw, bw


@pytest.mark.parametrize("dtype", [0, BF16])
@pytest.mark.parametrize("mlp", [MLP_SEQUENTIAL, MLP_PARALLEL])
@pytest.mark.parametrize("inv_temp", [0.0, 1.0])
def test_near_copy_lockstep_batch(dtype, mlp, inv_temp):
    """Draft = base + small noise (high acceptance), batch of 3 independent
    sequences with ragged accept counts, a layer-parallel set of 2."""
    from layer_speculative_decoding_amd.runtime import SpecDecoder
    sh, dw, bw = _near_copy_pair(dtype)
    say(f"near-copy lockstep dtype={dtype} mlp={mlp} invT={inv_temp}")
    sets = FUZZY4
    B, P, k, new = 3, 12, 4, 24
    prompts = make_prompts(sh.vocab, P, B, lambda b: 77 + b)
    dec = SpecDecoder(sh, to_dev(dw), sh, to_dev(bw), B, P + new + k + 2, k, plan_offsets(sets), P, inv_temp,
                      4242, mlp)
    tol = TOL_F32 if dtype == 0 else TOL_BF16
    st = lockstep(dec, OracleModel.from_torch(sh, dw), OracleModel.from_torch(sh, bw), prompts, k, sets, new,
                  dec.inv_temp, 4242, mlp, tol)
    acc = sum(int(a) for r in dec.records for a in r.n_acc)
    say(f"  checked {st['checked']} flipped {st['flipped']} excluded {st['excluded']} max rel err {st['err']:.2e}; "
        f"accepted {acc}")
    assert acc > 0
    assert st["excluded"] + st["flipped"] <= 2 + st["checked"] // 50


@pytest.mark.parametrize("dtype", [0, BF16])
@pytest.mark.parametrize("inv_temp", [0.0, 1.0])
def test_no_calibration_ablation_lockstep(dtype, inv_temp):
    """The ablation without KV calibration: accepted drafts keep their fuzzy
    KV entries and only the emitted token runs precisely; GPU and oracle run
    the same loop in lock step."""
    from layer_speculative_decoding_amd.runtime import SpecDecoder
    sh, dw, bw = _near_copy_pair(dtype)
    say(f"no-calibration lockstep dtype={dtype} invT={inv_temp}")
    sets = FUZZY4
    B, P, k, new = 3, 12, 4, 24
    prompts = make_prompts(sh.vocab, P, B, lambda b: 91 + b)
    dec = SpecDecoder(sh, to_dev(dw), sh, to_dev(bw), B, P + new + k + 2, k, plan_offsets(sets), P, inv_temp,
                      515, MLP_SEQUENTIAL, calibrate=False)
    tol = TOL_F32 if dtype == 0 else TOL_BF16
    st = lockstep(dec, OracleModel.from_torch(sh, dw), OracleModel.from_torch(sh, bw), prompts, k, sets, new,
                  dec.inv_temp, 515, MLP_SEQUENTIAL, tol, calibrate=False)
    acc = sum(int(a) for r in dec.records for a in r.n_acc)
    say(f"  checked {st['checked']} flipped {st['flipped']} excluded {st['excluded']} max rel err {st['err']:.2e}; "
        f"accepted {acc}")
    assert acc > 0
    assert st["excluded"] + st["flipped"] <= 2 + st["checked"] // 50


@pytest.mark.parametrize("dtype", [0, BF16])
@pytest.mark.parametrize("inv_temp", [0.0, 1.0])
def test_separate_calibration_lockstep(dtype, inv_temp):
    """The separate-pass reading of the calibration: all k drafts from fuzzy
    steps, then a precise pass over [x_t, d_1..d_a] at t..t+a; GPU and
    oracle run the same loop in lock step."""
    from layer_speculative_decoding_amd.runtime import SpecDecoder
    sh, dw, bw = _near_copy_pair(dtype)
    say(f"separate-calibration lockstep dtype={dtype} invT={inv_temp}")
    sets = FUZZY4
    B, P, k, new = 3, 12, 4, 24
    prompts = make_prompts(sh.vocab, P, B, lambda b: 133 + b)
    dec = SpecDecoder(sh, to_dev(dw), sh, to_dev(bw), B, P + new + k + 2, k, plan_offsets(sets), P, inv_temp,
                      616, MLP_SEQUENTIAL, separate=True)
    tol = TOL_F32 if dtype == 0 else TOL_BF16
    st = lockstep(dec, OracleModel.from_torch(sh, dw), OracleModel.from_torch(sh, bw), prompts, k, sets, new,
                  dec.inv_temp, 616, MLP_SEQUENTIAL, tol, separate=True)
    acc = sum(int(a) for r in dec.records for a in r.n_acc)
    say(f"  checked {st['checked']} flipped {st['flipped']} excluded {st['excluded']} max rel err {st['err']:.2e}; "
        f"accepted {acc}")
    assert acc > 0
    assert st["excluded"] + st["flipped"] <= 2 + st["checked"] // 50


@pytest.mark.parametrize("dtype", [0, BF16])
def test_greedy_speculative_equals_vanilla_on_gpu(dtype):
    """Lossless greedy decoding on the GPU.  float32: identical outputs.  bf16:
    verification (k+1 rows, matrix-core kernel) and vanilla decoding (one row)
    accumulate in different orders, so an arg-max may flip only at a near tie:
    the outputs must agree up to the first divergence, and there the oracle's
    base logits must have their top two tokens within the bf16 error bound,
    the two runs having picked exactly those two tokens."""
    from layer_speculative_decoding_amd.runtime import SpecDecoder, VanillaDecoder
    from oracle.model import KVCache, forward
    sh, dw, bw = _near_copy_pair(dtype, noise=0.01)
    say(f"greedy == vanilla dtype={dtype}")
    B, P, k, new = 2, 10, 5, 40
    prompts = make_prompts(sh.vocab, P, B, lambda b: 11 + b)
    sets = default_group_plan(sh.n_layers, 3)
    cap = P + new + k + 2
    dec = SpecDecoder(sh, to_dev(dw), sh, to_dev(bw), B, cap, k, plan_offsets(sets), P, 0.0, 1)
    spec = dec.generate(prompts, new)
    van = VanillaDecoder(sh, to_dev(bw), B, cap, P, 0.0, 1).generate(prompts, new)
    if dtype == 0:
        assert spec == van
        return
    ob = OracleModel.from_torch(sh, bw)
    for b in range(B):
        if spec[b] == van[b]:
            continue
        i = next(j for j in range(new) if spec[b][j] != van[b][j])
        z = forward(ob, KVCache(sh, 1, cap), 0, list(prompts[b]) + van[b][:i], range(P + i), logits="last")
        top = np.argsort(z)[::-1][:2]
        gap = float(z[top[0]] - z[top[1]])
        say(f"  b={b}: first divergence at {i}, oracle top-2 {top.tolist()} gap {gap:.2e}")
        assert {spec[b][i], van[b][i]} == set(top.tolist())
        assert gap < 2 * TOL_BF16 * float(np.max(np.abs(z)))
